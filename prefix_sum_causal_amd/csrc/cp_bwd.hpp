// cp_bwd.hpp -- reverse-scan backward kernel of the causal dot product, for
// gfx950.
//
// For f = sum_i out_i . dO_i with out_i = sum_{j<=i} (q_i . k_j) v_j (the
// causal dot product of "Transformers are RNNs", Algorithm 1, named in the
// opening post of "Dot Product Computes Wrong Values", triton-lang/triton
// issue 217, inclusive of token i):
//
//     dq_i = S_i dO_i,    S_i = sum_{j<=i} k_j v_j^T   (prefix)
//     dk_j = R_j v_j,     R_j = sum_{i>=j} q_i dO_i^T  (suffix)
//     dv_j = R_j^T k_j
//
// Split at chunk boundaries, with P_c = (dO_c V_c^T) (.) T and
// A_c = (Q_c K_c^T) (.) T (T the inclusive lower-triangular mask):
//
//     dQ_c = P_c K_c + dO_c S_{c-1}^T
//     dK_c = P_c^T Q_c + V_c R_{c+1}^T
//     dV_c = A_c^T dO_c + K_c R_{c+1}
//
// One launch holds three kinds of waves per (n, h) slice, all sweeping the
// chunks from last to first so that the waves of a slice read the same rows
// at the same time (they run on one XCD and share its L2):
//   dQ waves, one per 16-column block of E: carry S^T (M x 16).  Given the
//     slice's final state S_{L-1} they start from it and subtract each chunk
//     (S_{c-1} = S_{L-1} - sum_{c' >= c} K_c'^T V_c'); without it they sweep
//     forward from S = 0 instead.
//   dK waves, one per 16-column block of E: carry R^T (M x 16).
//   dV waves, one per 16-column block of M: carry R (E x 16).
// Every wave recomputes its chunk's P or A tiles; nothing from the forward
// pass is stored except the optional final state.
#pragma once

#include "cp_device.hpp"

namespace cp {

// Natural fragments of one chunk: full-width X (XW columns) and Y (YW
// columns) plus one 16-column block of Z.
template <typename T, int XW, int YW, int C>
struct BwdChunk {
    using F = typename Ops<T>::frag;
    static constexpr int XB = XW / 16, YB = YW / 16, CB = C / 16;
    F x[CB][XB];
    F y[CB][YB];
    F z[CB];
    // Rows outside [0, L) (and whole chunks outside the sequence) load as zero.
    __device__ __forceinline__ void load(const T *x_, const T *y_, const T *z_, int zld, int zcb, int row0,
                                         int L) {
        const Rows<T> rx(x_, XW, row0, L, C), ry(y_, YW, row0, L, C), rz(z_, zld, row0, L, C);
#pragma unroll
        for (int b = 0; b < CB; ++b) {
#pragma unroll
            for (int e = 0; e < XB; ++e) x[b][e] = ld_nat<T>(rx, b, e);
#pragma unroll
            for (int e = 0; e < YB; ++e) y[b][e] = ld_nat<T>(ry, b, e);
            z[b] = ld_nat<T>(rz, b, zcb);
        }
    }
};

// dQ wave for the E-column block eb.  x = V, y = dO (both M wide), z = K[:, eb].
template <typename T, int E, int M, int C, int NBUF, bool HILO, bool REV>
__device__ __forceinline__ void bwd_dq(const T *k_, const T *v_, const T *g_, const float *st, T *dq_, int L,
                                       int eb, T *lds) {
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int MB = M / 16, CB = C / 16;
    constexpr int RSY = M + O::kPad, RSZ = 16 + O::kPad;
    T *ldsV = lds, *ldsK = lds + C * RSY;
    const int g = lane_g(), r = lane_r();

    f32x4 W[MB];  // S^T[16 mb + 4g + t][16 eb + r]
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        W[m] = zero4();
        if (REV) {
#pragma unroll
            for (int t = 0; t < 4; ++t) W[m][t] = st[(16 * eb + r) * M + 16 * m + 4 * g + t];
        }
    }
    // steps padded to a multiple of NBUF; padded chunks lie outside the
    // sequence, load as zero and store nothing
    const int n = (L + C - 1) / C;
    const int nsteps = (n + NBUF - 1) / NBUF * NBUF;
    BwdChunk<T, M, M, C> buf[NBUF];
    auto chunk_of = [&](int s) { return REV ? n - 1 - s : s; };
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
        buf[s].load(v_, g_, k_, E, eb, chunk_of(s) * C, L);
        __builtin_amdgcn_sched_barrier(0);  // buffers complete in order
    }

    for (int s0 = 0; s0 < nsteps; s0 += NBUF) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
            const int step = s0 + s;
            const int row0 = chunk_of(step) * C;
            BwdChunk<T, M, M, C> &cur = buf[s];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int m = 0; m < MB; ++m) st_lds<T>(ldsV, RSY, b, m, cur.x[b][m]);
                st_lds<T>(ldsK, RSZ, b, 0, cur.z[b]);
            }
            wave_lds_sync();
            F vt[CB][MB], kt[CB];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int m = 0; m < MB; ++m) vt[b][m] = O::tr_frag(ldsV, RSY, b, m);
                kt[b] = O::tr_frag(ldsK, RSZ, b, 0);
            }
            buf[(s + NBUF - 1) % NBUF].load(v_, g_, k_, E, eb, chunk_of(step + NBUF - 1) * C, L);
            // keep the prefetch here: sunk towards the loop end it would be
            // the youngest load at the next chunk and stall the pipeline
            __builtin_amdgcn_sched_barrier(0);
            if (REV) {  // W = S_{c-1}^T = S_{L-1}^T - sum_{chunks >= c} V^T K
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk<T>(W[m], 0, CB, [&](int J) { return vt[J][m]; }, [&](int J) { return O::neg(kt[J]); });
            }
            const Rows<T> rdq(dq_, E, row0, L, C);
            F wh[MB], wl[MB];  // A = S (rows e, k = m)
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if constexpr (HILO) O::split(W[m], wh[m], wl[m]);
                else wh[m] = O::cvt(W[m]);
            }
#pragma unroll
            for (int I = 0; I < CB; ++I) {
                f32x4 d = zero4();
                // dQ^T += S dO_I^T
                dotk<T>(d, 0, MB, [&](int m) { return wh[m]; }, [&](int m) { return cur.y[I][m]; });
                if constexpr (HILO)
                    dotk<T>(d, 0, MB, [&](int m) { return wl[m]; }, [&](int m) { return cur.y[I][m]; });
                // P^T(J, I) = V_J dO_I^T, causal on the diagonal
                F pt[CB];
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    f32x4 p = zero4();
                    dotk<T>(p, 0, MB, [&](int m) { return cur.x[J][m]; }, [&](int m) { return cur.y[I][m]; });
                    if (J == I) p = mask_keys_rows(p);
                    pt[J] = O::cvt(p);
                }
                // dQ^T += K^T P^T
                dotk<T>(d, 0, I + 1, [&](int J) { return kt[J]; }, [&](int J) { return pt[J]; });
                st_out<T>(rdq, I, eb, d);
            }
            if (!REV) {  // W = S_c^T = S_{c-1}^T + V_c^T K_c
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk<T>(W[m], 0, CB, [&](int J) { return vt[J][m]; }, [&](int J) { return kt[J]; });
            }
            wave_lds_sync();
        }
    }
}

// dK wave for the E-column block eb.  x = dO, y = V (both M wide), z = Q[:, eb].
template <typename T, int E, int M, int C, int NBUF, bool HILO>
__device__ __forceinline__ void bwd_dk(const T *q_, const T *v_, const T *g_, T *dk_, int L, int eb, T *lds) {
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int MB = M / 16, CB = C / 16;
    constexpr int RSX = M + O::kPad, RSZ = 16 + O::kPad;
    T *ldsG = lds, *ldsQ = lds + C * RSX;

    f32x4 Rt[MB];  // R^T[16 mb + 4g + t][16 eb + r]
#pragma unroll
    for (int m = 0; m < MB; ++m) Rt[m] = zero4();
    const int n = (L + C - 1) / C;
    const int nsteps = (n + NBUF - 1) / NBUF * NBUF;
    BwdChunk<T, M, M, C> buf[NBUF];
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
        buf[s].load(g_, v_, q_, E, eb, (n - 1 - s) * C, L);
        __builtin_amdgcn_sched_barrier(0);  // buffers complete in order
    }

    for (int s0 = 0; s0 < nsteps; s0 += NBUF) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
            const int step = s0 + s;
            const int row0 = (n - 1 - step) * C;
            BwdChunk<T, M, M, C> &cur = buf[s];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int m = 0; m < MB; ++m) st_lds<T>(ldsG, RSX, b, m, cur.x[b][m]);
                st_lds<T>(ldsQ, RSZ, b, 0, cur.z[b]);
            }
            wave_lds_sync();
            F gt[CB][MB], qt[CB];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int m = 0; m < MB; ++m) gt[b][m] = O::tr_frag(ldsG, RSX, b, m);
                qt[b] = O::tr_frag(ldsQ, RSZ, b, 0);
            }
            buf[(s + NBUF - 1) % NBUF].load(g_, v_, q_, E, eb, (n - 1 - (step + NBUF - 1)) * C, L);
            // keep the prefetch here: sunk towards the loop end it would be
            // the youngest load at the next chunk and stall the pipeline
            __builtin_amdgcn_sched_barrier(0);
            const Rows<T> rdk(dk_, E, row0, L, C);
            F rh[MB], rl[MB];  // A = R (rows e, k = m)
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if constexpr (HILO) O::split(Rt[m], rh[m], rl[m]);
                else rh[m] = O::cvt(Rt[m]);
            }
#pragma unroll
            for (int J = 0; J < CB; ++J) {
                f32x4 d = zero4();
                // dK^T += R_{c+1} V_J^T
                dotk<T>(d, 0, MB, [&](int m) { return rh[m]; }, [&](int m) { return cur.y[J][m]; });
                if constexpr (HILO)
                    dotk<T>(d, 0, MB, [&](int m) { return rl[m]; }, [&](int m) { return cur.y[J][m]; });
                // P(I, J) = dO_I V_J^T for I >= J, causal on the diagonal
                F p[CB];
#pragma unroll
                for (int I = J; I < CB; ++I) {
                    f32x4 a = zero4();
                    dotk<T>(a, 0, MB, [&](int m) { return cur.x[I][m]; }, [&](int m) { return cur.y[J][m]; });
                    if (I == J) a = mask_query_rows(a);
                    p[I] = O::cvt(a);
                }
                // dK^T += Q^T P
                dotk<T>(d, J, CB, [&](int I) { return qt[I]; }, [&](int I) { return p[I]; });
                st_out<T>(rdk, J, eb, d);
            }
            // R^T += dO_c^T Q_c
#pragma unroll
            for (int m = 0; m < MB; ++m)
                dotk<T>(Rt[m], 0, CB, [&](int I) { return gt[I][m]; }, [&](int I) { return qt[I]; });
            wave_lds_sync();
        }
    }
}

// dV wave for the M-column block mb.  x = Q, y = K (both E wide), z = dO[:, mb].
template <typename T, int E, int M, int C, int NBUF, bool HILO>
__device__ __forceinline__ void bwd_dv(const T *q_, const T *k_, const T *g_, T *dv_, int L, int mb, T *lds) {
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int EB = E / 16, CB = C / 16;
    constexpr int RSX = E + O::kPad, RSZ = 16 + O::kPad;
    T *ldsQ = lds, *ldsG = lds + C * RSX;

    f32x4 R[EB];  // R[16 eb + 4g + t][16 mb + r]
#pragma unroll
    for (int e = 0; e < EB; ++e) R[e] = zero4();
    const int n = (L + C - 1) / C;
    const int nsteps = (n + NBUF - 1) / NBUF * NBUF;
    BwdChunk<T, E, E, C> buf[NBUF];
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
        buf[s].load(q_, k_, g_, M, mb, (n - 1 - s) * C, L);
        __builtin_amdgcn_sched_barrier(0);  // buffers complete in order
    }

    for (int s0 = 0; s0 < nsteps; s0 += NBUF) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
            const int step = s0 + s;
            const int row0 = (n - 1 - step) * C;
            BwdChunk<T, E, E, C> &cur = buf[s];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int e = 0; e < EB; ++e) st_lds<T>(ldsQ, RSX, b, e, cur.x[b][e]);
                st_lds<T>(ldsG, RSZ, b, 0, cur.z[b]);
            }
            wave_lds_sync();
            F qt[CB][EB], gt[CB];
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int e = 0; e < EB; ++e) qt[b][e] = O::tr_frag(ldsQ, RSX, b, e);
                gt[b] = O::tr_frag(ldsG, RSZ, b, 0);
            }
            buf[(s + NBUF - 1) % NBUF].load(q_, k_, g_, M, mb, (n - 1 - (step + NBUF - 1)) * C, L);
            // keep the prefetch here: sunk towards the loop end it would be
            // the youngest load at the next chunk and stall the pipeline
            __builtin_amdgcn_sched_barrier(0);
            const Rows<T> rdv(dv_, M, row0, L, C);
            F rh[EB], rl[EB];  // A = R^T (rows m, k = e)
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                if constexpr (HILO) O::split(R[e], rh[e], rl[e]);
                else rh[e] = O::cvt(R[e]);
            }
#pragma unroll
            for (int J = 0; J < CB; ++J) {
                f32x4 d = zero4();
                // dV^T += R^T K_J^T
                dotk<T>(d, 0, EB, [&](int e) { return rh[e]; }, [&](int e) { return cur.y[J][e]; });
                if constexpr (HILO)
                    dotk<T>(d, 0, EB, [&](int e) { return rl[e]; }, [&](int e) { return cur.y[J][e]; });
                // A(I, J) = Q_I K_J^T for I >= J, causal on the diagonal
                F a[CB];
#pragma unroll
                for (int I = J; I < CB; ++I) {
                    f32x4 s_ = zero4();
                    dotk<T>(s_, 0, EB, [&](int e) { return cur.x[I][e]; }, [&](int e) { return cur.y[J][e]; });
                    if (I == J) s_ = mask_query_rows(s_);
                    a[I] = O::cvt(s_);
                }
                // dV^T += dO^T A
                dotk<T>(d, J, CB, [&](int I) { return gt[I]; }, [&](int I) { return a[I]; });
                st_out<T>(rdv, J, mb, d);
            }
            // R += Q_c^T dO_c
#pragma unroll
            for (int e = 0; e < EB; ++e)
                dotk<T>(R[e], 0, CB, [&](int I) { return qt[I][e]; }, [&](int I) { return gt[I]; });
            wave_lds_sync();
        }
    }
}

template <typename T, int E, int M, int C, int NBUF, bool HILO>
__global__ __launch_bounds__(64) void cp_bwd_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                    const T *__restrict__ V, const T *__restrict__ G,
                                                    const float *__restrict__ state_in, T *__restrict__ dQ,
                                                    T *__restrict__ dK, T *__restrict__ dV, int L, int NS) {
    constexpr int EB = E / 16, MB = M / 16, P = 2 * EB + MB;
    constexpr int W = (E > M ? E : M);
    __shared__ __attribute__((aligned(16))) T lds[C * (W + Ops<T>::kPad) + C * (16 + Ops<T>::kPad)];
    int slice, part;
    map_block(blockIdx.x, NS, P, slice, part);
    const int64_t oe = (int64_t)slice * L * E, om = (int64_t)slice * L * M;
    if (part < EB) {
        if (state_in)
            bwd_dq<T, E, M, C, NBUF, HILO, true>(K + oe, V + om, G + om, state_in + (int64_t)slice * E * M,
                                                 dQ + oe, L, part, lds);
        else
            bwd_dq<T, E, M, C, NBUF, HILO, false>(K + oe, V + om, G + om, nullptr, dQ + oe, L, part, lds);
    } else if (part < 2 * EB) {
        bwd_dk<T, E, M, C, NBUF, HILO>(Q + oe, V + om, G + om, dK + oe, L, part - EB, lds);
    } else {
        bwd_dv<T, E, M, C, NBUF, HILO>(Q + oe, K + oe, G + om, dV + om, L, part - 2 * EB, lds);
    }
}

}  // namespace cp
