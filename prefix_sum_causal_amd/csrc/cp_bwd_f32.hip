// Backward kernel instances, f32 I/O.
#include "cp_bwd.hpp"
#include "cp_launch.hpp"
#include "cp_tune.hpp"

namespace cp {
namespace {

template <int E, int M>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    using T = float;
    using P = Tune<T, E, M>;
    auto kern = cp_bwd_kernel<T, E, M, P::BC, P::BG, P::BNPF>;
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K), *v = static_cast<const T *>(a.V),
            *g = static_cast<const T *>(a.G);
    const float *s0 = a.state_in, *st = a.state_final;
    T *dq = static_cast<T *>(a.dQ), *dk = static_cast<T *>(a.dK), *dv = static_cast<T *>(a.dV);
    float *ds0 = a.dstate_in;
    int L = a.L, NS = a.NS;
    void *args[] = {&q, &k, &v, &g, &s0, &st, &dq, &dk, &dv, &ds0, &L, &NS};
    return launch_kernel(reinterpret_cast<const void *>(kern), dim3(NS * P::BG), dim3(bwd_threads<T, E, M, P::BG>()), args, s);
}

}  // namespace

bwd_fn bwd_f32(int E, int M) {
    static const bwd_fn table[4][4] = {
        {launch_bwd<16, 16>, launch_bwd<16, 32>, launch_bwd<16, 64>, launch_bwd<16, 128>},
        {launch_bwd<32, 16>, launch_bwd<32, 32>, launch_bwd<32, 64>, launch_bwd<32, 128>},
        {launch_bwd<64, 16>, launch_bwd<64, 32>, launch_bwd<64, 64>, launch_bwd<64, 128>},
        {launch_bwd<128, 16>, launch_bwd<128, 32>, launch_bwd<128, 64>, launch_bwd<128, 128>},
    };
    const int ie = size_index(E), im = size_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

}  // namespace cp
