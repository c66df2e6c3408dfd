// Forward and normalised-forward kernel instances, f32 I/O.
#include "cp_fwd.hpp"
#include "cp_launch.hpp"
#include "cp_tune.hpp"

namespace cp {
namespace {

template <int E, int M, bool NORM, bool FMAP>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t s) {
    using T = float;
    using P = Tune<T, E, M>;
    auto kern = cp_fwd_kernel<T, E, M, P::FC, P::FG, P::FRS, P::FNPF, P::FOST, NORM, FMAP>;
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K), *v = static_cast<const T *>(a.V);
    T *o = static_cast<T *>(a.Out);
    float *st = a.state_out;
    int L = a.L, NS = a.NS;
    float eps = a.eps;
    void *args[] = {&q, &k, &v, &o, &st, &L, &NS, &eps};
    return launch_kernel(reinterpret_cast<const void *>(kern), dim3(NS * P::FG), dim3(64 * (M / 16 / P::FG) * P::FRS), args,
                         s);
}

template <int E, int M, bool NORM>
hipError_t launch_fwd_fm(const FwdArgs &a, hipStream_t s) {
    if (NORM && a.fmap) return launch_fwd<E, M, NORM, true>(a, s);
    return launch_fwd<E, M, NORM, false>(a, s);
}

template <bool NORM>
fwd_fn pick(int E, int M) {
    static const fwd_fn table[4][4] = {
        {launch_fwd_fm<16, 16, NORM>, launch_fwd_fm<16, 32, NORM>, launch_fwd_fm<16, 64, NORM>, launch_fwd_fm<16, 128, NORM>},
        {launch_fwd_fm<32, 16, NORM>, launch_fwd_fm<32, 32, NORM>, launch_fwd_fm<32, 64, NORM>, launch_fwd_fm<32, 128, NORM>},
        {launch_fwd_fm<64, 16, NORM>, launch_fwd_fm<64, 32, NORM>, launch_fwd_fm<64, 64, NORM>, launch_fwd_fm<64, 128, NORM>},
        {launch_fwd_fm<128, 16, NORM>, launch_fwd_fm<128, 32, NORM>, launch_fwd_fm<128, 64, NORM>, launch_fwd_fm<128, 128, NORM>},
    };
    const int ie = size_index(E), im = size_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

}  // namespace

fwd_fn fwd_f32(int E, int M, bool norm) { return norm ? pick<true>(E, M) : pick<false>(E, M); }

}  // namespace cp
