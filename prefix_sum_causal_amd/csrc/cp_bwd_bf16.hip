// Backward kernel instances (causal product and normalised form), bf16 I/O.
#include "cp_bwd_launch.hpp"

namespace cp {

bwd_fn bwd_bf16(int E, int M, bool norm) { return norm ? pick_bwd<__bf16, true>(E, M) : pick_bwd<__bf16, false>(E, M); }

}  // namespace cp
