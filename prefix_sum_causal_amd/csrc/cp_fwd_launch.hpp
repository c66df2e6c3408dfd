// cp_fwd_launch.hpp -- host side of the forward and normalised-forward
// launches, shared by the bf16, fp16 and fp32 translation units.
#pragma once

#include "cp_fwd.hpp"
#include "cp_launch.hpp"
#include "cp_tune.hpp"

#ifndef CP_FWD_SCAN_MIN_SEGS
#define CP_FWD_SCAN_MIN_SEGS 12
#endif

namespace cp {

template <typename T, int E, int M, bool NORM, bool FMAP>
hipError_t launch_fwd_t(const FwdArgs &a, hipStream_t s) {
    using P = Tune<T, E, M>;
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K), *v = static_cast<const T *>(a.V);
    T *o = static_cast<T *>(a.Out);
    const float *s0 = a.state_in, *z0 = a.z_in;
    float *st = a.state_out, *zt = a.z_out, *dn = a.den_out;
    int L = a.L, NS = a.NS, Ea = a.Ea, Ma = a.Ma;
    float eps = a.eps;
    // the normalised form runs one row set per workgroup (plus, but for the
    // widest heads, its denominator wave)
    constexpr bool DW = NORM && P::FDW;
    constexpr int FRS = NORM ? 1 : P::FRS, FRG = NORM ? P::FRG_N : P::FRG;
    const dim3 block(64 * ((M / 16 / P::FG) * FRS + (DW ? 1 : 0)));

    const SegPlan plan = plan_segments(L, NS, P::FG * FRG, P::FC);
    const int nseg = plan.nseg;
    int seg_len = plan.seg_len;
    // many segments: their increments scanned once rather than summed by
    // every sweep (a third launch, which a call of few segments does not repay)
    int cum = nseg >= CP_FWD_SCAN_MIN_SEGS ? 1 : 0;
    // per slice and segment: the E x M increment of the state, then E of z
    const size_t need = nseg > 1 ? (size_t)NS * nseg * (E * M + E) * sizeof(float) : 0;
    if (a.ws_need) {
        *a.ws_need = need;
        return hipSuccess;
    }
    float *ws = nullptr;
    bool owned = false;
    hipError_t e = hipSuccess;
    if (nseg > 1) {
        if (a.ws) {
            if (a.ws_bytes < need) return hipErrorInvalidValue;
            ws = a.ws;
        } else {
            if (a.noalloc) return hipErrorInvalidValue;
            e = hipMallocAsync(reinterpret_cast<void **>(&ws), need, s);
            if (e != hipSuccess) return e;
            owned = true;
        }
        constexpr int SW = seg_state_waves<M>();
        auto k1 = cp_seg_state_kernel<T, E, M, P::FC, SW, CP_SEG_NPF, NORM, FMAP>;
        const T *none = nullptr;
        const float *noden = nullptr;
        float *nows = nullptr;
        int first1 = 0, sub = 1;
        void *args1[] = {&k, &v, &ws, &none, &none, &none, &noden, &nows, &L, &NS, &seg_len, &sub, &first1, &Ea, &Ma};
        e = launch_kernel(reinterpret_cast<const void *>(k1), dim3(NS * (nseg - 1)), dim3(64 * SW), args1, s);
        if (e == hipSuccess && cum) {  // inclusive prefix sums of the slots: one read per sweep
            int nslot = nseg, lo1 = 0, hi1 = nseg - 1, sfx = 0, lo2 = 0;
            void *sargs[] = {&ws, &nows, &NS, &nslot, &lo1, &hi1, &sfx, &lo2};
            const long long threads = (long long)NS * ((E * M + E) / 4);
            e = launch_kernel(reinterpret_cast<const void *>(cp_seg_scan_kernel<E, M>),
                              dim3((unsigned)((threads + 255) / 256)), dim3(256), sargs, s);
        }
    }
    if (e == hipSuccess) {
        auto k2 = cp_fwd_kernel<T, E, M, P::FC, P::FG, FRS, FRG, P::FNPF, NORM, FMAP, DW>;
        void *args2[] = {&q, &k, &v, &o, &s0, &z0, &st, &zt, &dn, &ws, &L, &NS, &seg_len, &cum, &eps, &Ea, &Ma};
        e = launch_kernel(reinterpret_cast<const void *>(k2), dim3(NS * P::FG * FRG * nseg), block, args2, s);
    }
    if (owned) {
        const hipError_t f = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = f;
    }
    return e;
}

template <typename T, int E, int M, bool NORM>
hipError_t launch_fwd_fm(const FwdArgs &a, hipStream_t s) {
    if (NORM && a.fmap) return launch_fwd_t<T, E, M, NORM, true>(a, s);
    return launch_fwd_t<T, E, M, NORM, false>(a, s);
}

template <typename T, bool NORM>
fwd_fn pick_fwd(int E, int M) {
    static const fwd_fn table[4][4] = {
        {launch_fwd_fm<T, 16, 16, NORM>, launch_fwd_fm<T, 16, 32, NORM>, launch_fwd_fm<T, 16, 64, NORM>,
         launch_fwd_fm<T, 16, 128, NORM>},
        {launch_fwd_fm<T, 32, 16, NORM>, launch_fwd_fm<T, 32, 32, NORM>, launch_fwd_fm<T, 32, 64, NORM>,
         launch_fwd_fm<T, 32, 128, NORM>},
        {launch_fwd_fm<T, 64, 16, NORM>, launch_fwd_fm<T, 64, 32, NORM>, launch_fwd_fm<T, 64, 64, NORM>,
         launch_fwd_fm<T, 64, 128, NORM>},
        {launch_fwd_fm<T, 128, 16, NORM>, launch_fwd_fm<T, 128, 32, NORM>, launch_fwd_fm<T, 128, 64, NORM>,
         launch_fwd_fm<T, 128, 128, NORM>},
    };
    const int ie = tile_index(E), im = tile_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

// The backward's two-job segment-increment pass (see SegArgs), on the
// forward's instances of the kernel.
template <typename T, int E, int M, bool NORM, bool FMAP>
hipError_t launch_seg_nf(const SegArgs &a, hipStream_t s) {
    using P = Tune<T, E, M>;
    const T *k1 = static_cast<const T *>(a.K1), *v1 = static_cast<const T *>(a.V1);
    const T *k2 = static_cast<const T *>(a.K2), *v2 = static_cast<const T *>(a.V2), *o2 = static_cast<const T *>(a.O2);
    const float *den2 = a.den2;
    float *ws1 = a.ws1, *ws2 = a.ws2;
    int L = a.L, NS = a.NS, seg_len = a.seg_len, sub = a.sub, first1 = a.first1, Ea = a.Ea, Ma = a.Ma;
    const int nseg = (L + seg_len - 1) / seg_len;
    constexpr int SW = seg_state_waves<M>();
    auto kern = cp_seg_state_kernel<T, E, M, P::FC, SW, CP_SEG_NPF, NORM, FMAP>;
    void *args[] = {&k1, &v1, &ws1, &k2, &v2, &o2, &den2, &ws2, &L, &NS, &seg_len, &sub, &first1, &Ea, &Ma};
    return launch_kernel(reinterpret_cast<const void *>(kern), dim3(NS * (k2 ? 2 : 1) * (nseg - 1) * sub),
                         dim3(64 * SW), args, s);
}

template <typename T, int E, int M>
hipError_t launch_seg_t(const SegArgs &a, hipStream_t s) {
    if (!a.norm) return launch_seg_nf<T, E, M, false, false>(a, s);
    if (a.fmap) return launch_seg_nf<T, E, M, true, true>(a, s);
    return launch_seg_nf<T, E, M, true, false>(a, s);
}

template <typename T>
seg_fn pick_seg(int E, int M) {
    static const seg_fn table[4][4] = {
        {launch_seg_t<T, 16, 16>, launch_seg_t<T, 16, 32>, launch_seg_t<T, 16, 64>, launch_seg_t<T, 16, 128>},
        {launch_seg_t<T, 32, 16>, launch_seg_t<T, 32, 32>, launch_seg_t<T, 32, 64>, launch_seg_t<T, 32, 128>},
        {launch_seg_t<T, 64, 16>, launch_seg_t<T, 64, 32>, launch_seg_t<T, 64, 64>, launch_seg_t<T, 64, 128>},
        {launch_seg_t<T, 128, 16>, launch_seg_t<T, 128, 32>, launch_seg_t<T, 128, 64>, launch_seg_t<T, 128, 128>},
    };
    const int ie = tile_index(E), im = tile_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

}  // namespace cp
