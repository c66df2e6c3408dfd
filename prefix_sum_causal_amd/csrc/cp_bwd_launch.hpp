// cp_bwd_launch.hpp -- host side of the backward launches (causal product and
// normalised form), shared by the bf16, fp16 and fp32 translation units.
#pragma once

#include <type_traits>

#include "cp_bwd.hpp"
#include "cp_launch.hpp"
#include "cp_tune.hpp"

#ifndef CP_BWD_SEG_SUB
#define CP_BWD_SEG_SUB 2
#endif

namespace cp {

// One kernel per call, no scratch, when the slices fill the GPU.  The
// normalised form's extra terms (dn = dO / den, dd = -(dO . out) / den, the
// normaliser before each chunk) are formed inside the sweep from the
// forward's output, denominators and final (or initial) normaliser.
//
// Few slices: each slice is cut into nseg sequence segments of seg_len rows
// (a multiple of C) and run in two launches, the scan's carry one level up,
// as in the forward.  The first computes every segment's increments of the
// prefix state (sum of k v^T, all but the last segment; normalised form: with
// the sum of phi(k)) and of the suffix state (sum of q dO^T, all but the
// first; normalised form: of phi(q) dn^T, with the sum of dd phi(q)) into
// the caller's workspace or, without one, a stream-ordered scratch buffer;
// the second sweeps each segment with the states at its ends summed from
// those increments (see SegCarry).
template <typename T, int E, int M, bool NORM, bool FMAP>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
    using P = Tune<T, E, M>;
    constexpr int C = P::BC;
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K), *v = static_cast<const T *>(a.V),
            *g = static_cast<const T *>(a.G), *o = static_cast<const T *>(a.Out);
    const float *s0 = a.state_in, *st = a.state_final, *den = a.den, *z0 = a.z_in, *zf = a.z_final;
    T *dq = static_cast<T *>(a.dQ), *dk = static_cast<T *>(a.dK), *dv = static_cast<T *>(a.dV);
    float *ds0 = a.dstate_in, *dz0 = a.dz_in;
    int L = a.L, NS = a.NS, Ea = a.Ea, Ma = a.Ma;

    const SegPlan plan = plan_segments(L, NS, P::BG * P::BRG, C, kBwdSegWgPerCU);
    const int nseg = plan.nseg;
    int seg_len = plan.seg_len;
    constexpr int WS = E * M + E;
    // parts per segment increment: two for the normalised form where the
    // increment pass's two jobs would leave CUs idle (its second job, which
    // also reads the output and forms dn and dd, is the longer one; the
    // causal product's two jobs are even, and a second part costs it more
    // than it gains)
    int sub = NORM && nseg > 1 && (long long)2 * (nseg - 1) * NS < kCUs ? CP_BWD_SEG_SUB : 1;
    // prefix then suffix increments: per slice, segment and part E x M then E floats each
    const size_t need = nseg > 1 ? (size_t)2 * NS * nseg * sub * WS * sizeof(float) : 0;
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
            e = hipMallocAsync(reinterpret_cast<void **>(&ws), need, s);
            if (e != hipSuccess) return e;
            owned = true;
        }
        // with the final states used, the sweeps subtract the later segments'
        // increments from them: the prefix increments of segments 1 .. nseg-1
        const bool use_final = st && (!NORM || zf) && !(NORM && std::is_same<T, float>::value);
        const SegArgs sa{k,  v,  ws,      q,  g,  o,  den, ws + (size_t)NS * nseg * sub * WS, L, NS, seg_len,
                         sub, use_final ? 1 : 0, Ea, Ma, NORM, FMAP};
        const seg_fn fn = std::is_same<T, float>::value ? seg_f32(E, M)
                          : std::is_same<T, __bf16>::value ? seg_bf16(E, M)
                                                           : seg_f16(E, M);
        e = fn ? fn(sa, s) : hipErrorInvalidValue;
        if (e == hipSuccess) {  // the slots made cumulative for the sweeps
            float *w1 = ws, *w2 = ws + (size_t)NS * nseg * sub * WS;
            int ns = NS, nslot = nseg * sub, lo1 = sub, hi1 = (nseg - 1) * sub, sfx = use_final ? 1 : 0, lo2 = sub;
            void *sargs[] = {&w1, &w2, &ns, &nslot, &lo1, &hi1, &sfx, &lo2};
            const long long threads = 2LL * NS * (WS / 4);
            e = launch_kernel(reinterpret_cast<const void *>(cp_seg_scan_kernel<E, M>),
                              dim3((unsigned)((threads + 255) / 256)), dim3(256), sargs, s);
        }
    }
    if (e == hipSuccess) {
        const float *wsc = ws;
        auto kern = cp_bwd_kernel<T, E, M, C, P::BG, P::BNB, P::BIDLE, P::BRG, NORM ? P::BNPF_N : P::BNPF, NORM, FMAP>;
        void *args[] = {&q,  &k,   &v,   &g,   &s0, &st, &o,  &den,     &z0,  &zf, &dq,
                        &dk, &dv,  &ds0, &dz0, &wsc, &L, &NS, &seg_len, &sub, &Ea, &Ma};
        e = launch_kernel(reinterpret_cast<const void *>(kern), dim3(NS * P::BG * P::BRG * nseg),
                          dim3(64 * bwd_waves<E, M, P::BG, P::BNB, P::BIDLE>()), args, s);
    }
    if (owned) {
        const hipError_t f = hipFreeAsync(ws, s);
        if (e == hipSuccess) e = f;
    }
    return e;
}

template <typename T, int E, int M, bool NORM>
hipError_t launch_bwd_fm(const BwdArgs &a, hipStream_t s) {
    if (NORM && a.fmap) return launch_bwd_t<T, E, M, NORM, true>(a, s);
    return launch_bwd_t<T, E, M, NORM, false>(a, s);
}

template <typename T, bool NORM>
bwd_fn pick_bwd(int E, int M) {
    static const bwd_fn table[4][4] = {
        {launch_bwd_fm<T, 16, 16, NORM>, launch_bwd_fm<T, 16, 32, NORM>, launch_bwd_fm<T, 16, 64, NORM>,
         launch_bwd_fm<T, 16, 128, NORM>},
        {launch_bwd_fm<T, 32, 16, NORM>, launch_bwd_fm<T, 32, 32, NORM>, launch_bwd_fm<T, 32, 64, NORM>,
         launch_bwd_fm<T, 32, 128, NORM>},
        {launch_bwd_fm<T, 64, 16, NORM>, launch_bwd_fm<T, 64, 32, NORM>, launch_bwd_fm<T, 64, 64, NORM>,
         launch_bwd_fm<T, 64, 128, NORM>},
        {launch_bwd_fm<T, 128, 16, NORM>, launch_bwd_fm<T, 128, 32, NORM>, launch_bwd_fm<T, 128, 64, NORM>,
         launch_bwd_fm<T, 128, 128, NORM>},
    };
    const int ie = tile_index(E), im = tile_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

}  // namespace cp
