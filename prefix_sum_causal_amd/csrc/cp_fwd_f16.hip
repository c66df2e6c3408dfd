// Forward and normalised-forward kernel instances, and the backward's segment
// increment pass, fp16 I/O.
#include "cp_fwd_launch.hpp"

namespace cp {

fwd_fn fwd_f16(int E, int M, bool norm) { return norm ? pick_fwd<_Float16, true>(E, M) : pick_fwd<_Float16, false>(E, M); }

seg_fn seg_f16(int E, int M) { return pick_seg<_Float16>(E, M); }

}  // namespace cp
