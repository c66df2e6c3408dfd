// Forward and normalised-forward kernel instances, and the backward's segment
// increment pass, bf16 I/O.
#include "cp_fwd_launch.hpp"

namespace cp {

fwd_fn fwd_bf16(int E, int M, bool norm) { return norm ? pick_fwd<__bf16, true>(E, M) : pick_fwd<__bf16, false>(E, M); }

seg_fn seg_bf16(int E, int M) { return pick_seg<__bf16>(E, M); }

}  // namespace cp
