// Forward and normalised-forward kernel instances, and the backward's segment
// increment pass, f32 I/O.
#include "cp_fwd_launch.hpp"

namespace cp {

fwd_fn fwd_f32(int E, int M, bool norm) { return norm ? pick_fwd<float, true>(E, M) : pick_fwd<float, false>(E, M); }

seg_fn seg_f32(int E, int M) { return pick_seg<float>(E, M); }

}  // namespace cp
