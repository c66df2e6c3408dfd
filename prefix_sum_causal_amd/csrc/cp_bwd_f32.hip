// Backward kernel instances (causal product and normalised form), f32 I/O.
#include "cp_bwd_launch.hpp"

namespace cp {

bwd_fn bwd_f32(int E, int M, bool norm) { return norm ? pick_bwd<float, true>(E, M) : pick_bwd<float, false>(E, M); }

}  // namespace cp
