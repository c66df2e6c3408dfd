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
// A workgroup owns one (n, h) slice and one of G groups of 16-column blocks
// of the outputs (every G-th block of dQ and of dK, and of dV).  Each wave
// owns one output column block for every row of the chunk:
//   dQ wave (columns b of E) carries S^T[:, b]  (M x 16),
//   dK wave (columns b of E) carries R^T[:, b]  (M x 16),
//   dV wave (columns b of M) carries R[:, b]    (E x 16),
// and forms the chunk's causal tiles it needs itself (P^T for dQ, P for dK,
// A for dV: cheaper than exchanging them through LDS).  The chunks are swept
// from last to first; per chunk all threads copy Q, K, V and dO into LDS
// (double buffered, one barrier per chunk) while the next chunks' loads are
// in flight.  The dQ wave starts from the slice's final state S_{L-1} and
// subtracts each chunk (S_{c-1} = S_{L-1} - sum_{c' >= c} K_c'^T V_c'); the
// state comes from the forward pass, or, when it is not given, from a
// forward pre-pass of the workgroup over K and V starting at the initial
// state S0.  At the end the dV waves hold R_0 = sum_i q_i dO_i^T, the
// gradient of S0.  Carried states keep the
// rows of their contraction index (m or e) in the order of the 16-byte
// natural reads of the other operand (see EOps), so no operand is read twice.
#pragma once

#include "cp_device.hpp"

namespace cp {

enum BwdRole { kDQ = 0, kDK = 1, kDV = 2, kIdle = 3 };

// The whole sweep of one wave role.  Every role runs the same staging and
// barriers; only the math differs, so each wave's loop is straight-line code.
template <typename T, int E, int M, int C, int G, int NPF, int ROLE>
__device__ __forceinline__ void bwd_sweep(const T *q_, const T *k_, const T *v_, const T *g_, const float *s0,
                                          const float *st, T *out_, float *ds0, int L, int b, T *lds) {
    using O = Ops<T>;
    using F = typename O::frag;
    using EE = EOps<T, E>;  // contraction over e
    using EM = EOps<T, M>;  // contraction over m
    constexpr int EB = E / 16, MB = M / 16, CB = C / 16;
    constexpr int EG = (EB + G - 1) / G, MG = (MB + G - 1) / G, NT = 64 * (2 * EG + MG);
    using SE = Stage<T, NT, C, E>;
    using SM = Stage<T, NT, C, M>;
    constexpr int RE = SE::RS, RM = SM::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;  // Q, K, V, dO
    const int g = lane_g(), r = lane_r();
    const int n = (L + C - 1) / C;
    const Diag diag;

    // carried state (fp32 accumulator tiles)
    //   dQ: W[mt] = S^T[ecol_M(mt) + estride_M g + t][16 b + r]
    //   dK: W[mt] = R^T[ecol_M(mt) + estride_M g + t][16 b + r]
    //   dV: X[et] = R[ecol_E(et) + estride_E g + t][16 b + r]
    f32x4 W[MB], X[EB];
#pragma unroll
    for (int m = 0; m < MB; ++m) W[m] = zero4();
#pragma unroll
    for (int e = 0; e < EB; ++e) X[e] = zero4();

    if (st) {
        if constexpr (ROLE == kDQ) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int t = 0; t < 4; ++t) W[m][t] = st[(16 * b + r) * M + EM::ecol(m) + EM::estride * g + t];
        }
    } else {
        // forward pre-pass: S_{L-1}^T[:, b] = S0^T[:, b] + sum over chunks of V^T K[:, b]
        if constexpr (ROLE == kDQ) {
            if (s0) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int t = 0; t < 4; ++t) W[m][t] = s0[(16 * b + r) * M + EM::ecol(m) + EM::estride * g + t];
            }
        }
        SE sk;
        SM sv;
        sk.load(Rows<T>(k_, E, 0, L, C), 0);
        sv.load(Rows<T>(v_, M, 0, L, C), 0);
        for (int c = 0; c < n; ++c) {
            T *Ks = lds + (c & 1) * BUF, *Vs = Ks + C * RE;
            sk.store(Ks);
            sv.store(Vs);
            __syncthreads();
            sk.load(Rows<T>(k_, E, (c + 1) * C, L, C), 0);
            sv.load(Rows<T>(v_, M, (c + 1) * C, L, C), 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ROLE == kDQ) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk<T>(W[m], 0, CB, [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                            [&](int J) { return O::tr_frag(Ks, RE, J, b); });
            }
        }
        __syncthreads();  // the main sweep reuses the buffers
    }

    constexpr int OW = ROLE == kDV ? M : E;

    // Ring of NPF register stages (NPF-1 chunks in flight while one is
    // computed); the step loop is padded to a multiple of NPF with chunks
    // before the start of the sequence, which load as zero and store nothing.
    struct Stages {
        SE q, k;
        SM v, g;
        __device__ __forceinline__ void load(const T *q_, const T *k_, const T *v_, const T *g_, int row0, int L) {
            q.load(Rows<T>(q_, E, row0, L, C), 0);
            k.load(Rows<T>(k_, E, row0, L, C), 0);
            v.load(Rows<T>(v_, M, row0, L, C), 0);
            g.load(Rows<T>(g_, M, row0, L, C), 0);
        }
    };
    Stages stg[NPF];
#pragma unroll
    for (int s = 0; s < NPF - 1; ++s) {
        stg[s].load(q_, k_, v_, g_, (n - 1 - s) * C, L);
        __builtin_amdgcn_sched_barrier(0);  // stages complete in order
    }
    const int nsteps = (n + NPF - 1) / NPF * NPF;
    for (int s0 = 0; s0 < nsteps; s0 += NPF) {
#pragma unroll
        for (int s = 0; s < NPF; ++s) {
            const int step = s0 + s;
            const int row0 = (n - 1 - step) * C;
            T *Qs = lds + (step & 1) * BUF, *Ks = Qs + C * RE, *Vs = Ks + C * RE, *Gs = Vs + C * RM;
            stg[s].q.store(Qs);
            stg[s].k.store(Ks);
            stg[s].v.store(Vs);
            stg[s].g.store(Gs);
            __syncthreads();
            stg[(s + NPF - 1) % NPF].load(q_, k_, v_, g_, row0 - (NPF - 1) * C, L);
            __builtin_amdgcn_sched_barrier(0);

            f32x4 pend[CB];  // this chunk's output tiles (rows 16 I + r)
            if constexpr (ROLE == kDQ) {
                // W = S_{c-1}^T = S_c^T - V_c^T K_c[:, b]
                F kt[CB];  // K_J[:, b] transposed: lane (g, r) <- K[16 J + 4g + t][16 b + r]
#pragma unroll
                for (int J = 0; J < CB; ++J) kt[J] = O::tr_frag(Ks, RE, J, b);
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk<T>(W[m], 0, CB, [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                            [&](int J) { return O::neg(kt[J]); });
                typename EM::rf wa[EM::STEPS], vf[CB][EM::STEPS];
#pragma unroll
                for (int k = 0; k < EM::STEPS; ++k) wa[k] = EM::state(W, k);
#pragma unroll
                for (int J = 0; J < CB; ++J)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) vf[J][k] = EM::load(Vs, RM, J, k);
#pragma unroll
                for (int I = 0; I < CB; ++I) {
                    typename EM::rf gf[EM::STEPS];
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) gf[k] = EM::load(Gs, RM, I, k);
                    // dQ^T = S dO_I^T + K^T P^T with P^T(J, I) = V_J dO_I^T, causal on the diagonal
                    f32x4 d = zero4();
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) EM::mma(d, wa[k], gf[k]);
                    F pt[CB];
#pragma unroll
                    for (int J = 0; J <= I; ++J) {
                        f32x4 p = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(p, vf[J][k], gf[k]);
                        if (J == I) p = diag.keys(p);
                        pt[J] = O::cvt(p);
                    }
                    dotk<T>(d, 0, I + 1, [&](int J) { return kt[J]; }, [&](int J) { return pt[J]; });
                    pend[I] = d;
                }
            } else if constexpr (ROLE == kDK) {
                F qt[CB];  // Q_I[:, b] transposed
#pragma unroll
                for (int I = 0; I < CB; ++I) qt[I] = O::tr_frag(Qs, RE, I, b);
                typename EM::rf wa[EM::STEPS], gf[CB][EM::STEPS];
#pragma unroll
                for (int k = 0; k < EM::STEPS; ++k) wa[k] = EM::state(W, k);  // R_{c+1}
#pragma unroll
                for (int I = 0; I < CB; ++I)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) gf[I][k] = EM::load(Gs, RM, I, k);
#pragma unroll
                for (int J = 0; J < CB; ++J) {
                    typename EM::rf vf[EM::STEPS];
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) vf[k] = EM::load(Vs, RM, J, k);
                    // dK^T = R_{c+1} V_J^T + Q^T P with P(I, J) = dO_I V_J^T for I >= J
                    f32x4 d = zero4();
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) EM::mma(d, wa[k], vf[k]);
                    F pf[CB];
#pragma unroll
                    for (int I = J; I < CB; ++I) {
                        f32x4 p = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(p, gf[I][k], vf[k]);
                        if (I == J) p = diag.query(p);
                        pf[I] = O::cvt(p);
                    }
                    dotk<T>(d, J, CB, [&](int I) { return qt[I]; }, [&](int I) { return pf[I]; });
                    pend[J] = d;
                }
                // R^T += dO_c^T Q_c[:, b]
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk<T>(W[m], 0, CB, [&](int I) { return EM::tr_e(Gs, RM, I, m); }, [&](int I) { return qt[I]; });
            } else if constexpr (ROLE == kDV) {
                F gt[CB];  // dO_I[:, b] transposed
#pragma unroll
                for (int I = 0; I < CB; ++I) gt[I] = O::tr_frag(Gs, RM, I, b);
                typename EE::rf xa[EE::STEPS], qf[CB][EE::STEPS];
#pragma unroll
                for (int k = 0; k < EE::STEPS; ++k) xa[k] = EE::state(X, k);  // R_{c+1}^T rows
#pragma unroll
                for (int I = 0; I < CB; ++I)
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) qf[I][k] = EE::load(Qs, RE, I, k);
#pragma unroll
                for (int J = 0; J < CB; ++J) {
                    typename EE::rf kf[EE::STEPS];
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) kf[k] = EE::load(Ks, RE, J, k);
                    // dV^T = R^T K_J^T + dO^T A with A(I, J) = Q_I K_J^T for I >= J
                    f32x4 d = zero4();
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) EE::mma(d, xa[k], kf[k]);
                    F af[CB];
#pragma unroll
                    for (int I = J; I < CB; ++I) {
                        f32x4 a = zero4();
#pragma unroll
                        for (int k = 0; k < EE::STEPS; ++k) EE::mma(a, qf[I][k], kf[k]);
                        if (I == J) a = diag.query(a);
                        af[I] = O::cvt(a);
                    }
                    dotk<T>(d, J, CB, [&](int I) { return gt[I]; }, [&](int I) { return af[I]; });
                    pend[J] = d;
                }
                // R += Q_c^T dO_c[:, b]
#pragma unroll
                for (int e = 0; e < EB; ++e)
                    dotk<T>(X[e], 0, CB, [&](int I) { return EE::tr_e(Qs, RE, I, e); }, [&](int I) { return gt[I]; });
            }
            // Stores go after this step's prefetch: memory operations complete
            // in issue order, so the rows waited for at a later step were
            // issued before these stores and never wait for them.
            if constexpr (ROLE != kIdle) {
                const Rows<T> rp(out_, OW, row0, L, C);
#pragma unroll
                for (int j = 0; j < CB; ++j) st_out<T>(rp, j, b, pend[j]);
            }
        }
    }
    // the gradient of the initial state: R_0 = sum_i q_i dO_i^T, held by the
    // dV waves (column blocks b of M) at the end of the reverse sweep
    if constexpr (ROLE == kDV) {
        if (ds0) {
#pragma unroll
            for (int e = 0; e < EB; ++e)
#pragma unroll
                for (int t = 0; t < 4; ++t) ds0[(EE::ecol(e) + EE::estride * g + t) * M + 16 * b + r] = X[e][t];
        }
    }
}

// Waves of a workgroup: EG dQ waves, EG dK waves and MG dV waves; group grp
// takes the column blocks b = grp + G * i (a wave whose block is past E or M
// only helps copy).
template <typename T, int E, int M, int G>
constexpr int bwd_threads() {
    return 64 * (2 * ((E / 16 + G - 1) / G) + (M / 16 + G - 1) / G);
}

template <typename T, int E, int M, int C, int G, int NPF>
__global__ __launch_bounds__((bwd_threads<T, E, M, G>())) void cp_bwd_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, const T *__restrict__ Gr,
    const float *__restrict__ state_in, const float *__restrict__ state_final, T *__restrict__ dQ,
    T *__restrict__ dK, T *__restrict__ dV, float *__restrict__ dstate_in, int L, int NS) {
    constexpr int EB = E / 16, MB = M / 16;
    constexpr int EG = (EB + G - 1) / G, NT = bwd_threads<T, E, M, G>();
    static_assert(NT <= 1024, "at most 16 waves per workgroup");
    constexpr int RE = Stage<T, NT, C, E>::RS, RM = Stage<T, NT, C, M>::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;
    __shared__ __attribute__((aligned(16))) T lds[2 * BUF];

    int slice, grp;
    map_block(blockIdx.x, NS, G, slice, grp);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int64_t oe = (int64_t)slice * L * E, om = (int64_t)slice * L * M;
    const T *q_ = Q + oe, *k_ = K + oe, *v_ = V + om, *g_ = Gr + om;
    const float *s0 = state_in ? state_in + (int64_t)slice * E * M : nullptr;
    const float *st = state_final ? state_final + (int64_t)slice * E * M : nullptr;
    float *ds0 = dstate_in ? dstate_in + (int64_t)slice * E * M : nullptr;
    const int role = w < EG ? kDQ : w < 2 * EG ? kDK : kDV;
    const int b = grp + G * (role == kDQ ? w : role == kDK ? w - EG : w - 2 * EG);
    if (role == kDQ && b < EB)
        bwd_sweep<T, E, M, C, G, NPF, kDQ>(q_, k_, v_, g_, s0, st, dQ + oe, nullptr, L, b, lds);
    else if (role == kDK && b < EB)
        bwd_sweep<T, E, M, C, G, NPF, kDK>(q_, k_, v_, g_, s0, st, dK + oe, nullptr, L, b, lds);
    else if (role == kDV && b < MB)
        bwd_sweep<T, E, M, C, G, NPF, kDV>(q_, k_, v_, g_, s0, st, dV + om, ds0, L, b, lds);
    else
        bwd_sweep<T, E, M, C, G, NPF, kIdle>(q_, k_, v_, g_, s0, st, nullptr, nullptr, L, 0, lds);
}

}  // namespace cp
