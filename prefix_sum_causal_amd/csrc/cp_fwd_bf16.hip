// Forward and normalised-forward kernel instances, bf16 I/O.
#include "cp_fwd_launch.hpp"

namespace cp {

fwd_fn fwd_bf16(int E, int M, bool norm) { return norm ? pick_fwd<__bf16, true>(E, M) : pick_fwd<__bf16, false>(E, M); }

}  // namespace cp
