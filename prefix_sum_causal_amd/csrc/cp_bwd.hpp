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
// A workgroup owns one (n, h) slice and one 16-column block b and runs three
// waves: the dQ wave (columns b of E) carries S^T (M x 16), the dK wave
// (columns b of E) carries R^T (M x 16), the dV wave (columns b of M) carries
// R (E x 16); a wave whose block is past E or M only helps copy.  The chunks
// are swept from last to first; per chunk all threads copy Q, K, V and dO into
// LDS (double buffered, one barrier per chunk) while the next chunk's loads
// are in flight.  The dQ wave starts from the slice's final state S_{L-1} and
// subtracts each chunk (S_{c-1} = S_{L-1} - sum_{c' >= c} K_c'^T V_c'); the
// state comes from the forward pass, or, when it is not given, from a forward
// pre-pass of the workgroup over K and V.  Every workgroup of a slice does the
// same work per chunk, so the max(E, M)/16 workgroups of a slice, placed on
// one XCD, stay in step and read the slice's rows once from HBM.
#pragma once

#include "cp_device.hpp"

namespace cp {

enum BwdRole { kIdle = 0, kDQ = 1, kDK = 2, kDV = 3 };

// The whole sweep for one wave role.  Every role runs the same staging and
// barriers; only the math differs, so each wave's loop is straight-line code.
template <typename T, int E, int M, int C, int NPF, bool HILO, int ROLE>
__device__ __forceinline__ void bwd_sweep(const T *q_, const T *k_, const T *v_, const T *g_, const float *st,
                                          T *out_, int L, int b, T *lds) {
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int NT = 192, EB = E / 16, MB = M / 16, CB = C / 16;
    using SE = Stage<T, NT, C, E>;
    using SM = Stage<T, NT, C, M>;
    constexpr int RE = SE::RS, RM = SM::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;  // Q, K, V, dO
    const int g = lane_g(), r = lane_r();
    const int n = (L + C - 1) / C;
    const Diag diag;

    // carried state: dQ W = S^T[16 m + 4g + t][16 b + r]; dK W = R^T[16 m + 4g + t][16 b + r];
    // dV X = R[16 e + 4g + t][16 b + r]
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
                for (int t = 0; t < 4; ++t) W[m][t] = st[(16 * b + r) * M + 16 * m + 4 * g + t];
        }
    } else {
        // forward pre-pass: S_{L-1}^T[:, b] = sum over chunks of V^T K[:, b]
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
                    dotk<T>(W[m], 0, CB, [&](int J) { return O::tr_frag(Vs, RM, J, m); },
                            [&](int J) { return O::tr_frag(Ks, RE, J, b); });
            }
        }
        __syncthreads();  // the main sweep reuses the buffers
    }

    f32x4 pend[CB];  // this chunk's output tiles
#pragma unroll
    for (int j = 0; j < CB; ++j) pend[j] = zero4();
    constexpr int OW = ROLE == kDV ? M : E;
    auto store_pending = [&](int prow0) {
        if constexpr (ROLE != kIdle) {
            const Rows<T> rp(out_, OW, prow0, L, C);
#pragma unroll
            for (int j = 0; j < CB; ++j) st_out<T>(rp, j, b, pend[j]);
        }
    };

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

        if constexpr (ROLE == kDQ) {
            // W = S_{c-1}^T = S_{L-1}^T - sum_{chunks >= c} V^T K[:, b]
#pragma unroll
            for (int m = 0; m < MB; ++m)
                dotk<T>(W[m], 0, CB, [&](int J) { return O::tr_frag(Vs, RM, J, m); },
                        [&](int J) { return O::neg(O::tr_frag(Ks, RE, J, b)); });
            F wh[MB], wl[MB];  // A = S (rows e, k = m)
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if constexpr (HILO) O::split(W[m], wh[m], wl[m]);
                else wh[m] = O::cvt(W[m]);
            }
#pragma unroll
            for (int I = 0; I < CB; ++I) {
                // dQ^T = S dO_I^T + K^T P^T with P^T(J, I) = V_J dO_I^T, causal on the diagonal
                f32x4 d = dotz<T>(0, MB, [&](int m) { return wh[m]; }, [&](int m) { return lds_nat<T>(Gs, RM, I, m); });
                if constexpr (HILO)
                    dotk<T>(d, 0, MB, [&](int m) { return wl[m]; }, [&](int m) { return lds_nat<T>(Gs, RM, I, m); });
                F pt[CB];
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    f32x4 p = nn_tile<T, MB>(Vs, RM, J, Gs, RM, I);
                    if (J == I) p = diag.keys(p);
                    pt[J] = O::cvt(p);
                }
                dotk<T>(d, 0, I + 1, [&](int J) { return O::tr_frag(Ks, RE, J, b); }, [&](int J) { return pt[J]; });
                pend[I] = d;
            }
        } else if constexpr (ROLE == kDK) {
            F rh[MB], rl[MB];  // A = R_{c+1} (rows e, k = m)
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if constexpr (HILO) O::split(W[m], rh[m], rl[m]);
                else rh[m] = O::cvt(W[m]);
            }
#pragma unroll
            for (int J = 0; J < CB; ++J) {
                // dK^T = R_{c+1} V_J^T + Q^T P with P(I, J) = dO_I V_J^T for I >= J
                f32x4 d = dotz<T>(0, MB, [&](int m) { return rh[m]; }, [&](int m) { return lds_nat<T>(Vs, RM, J, m); });
                if constexpr (HILO)
                    dotk<T>(d, 0, MB, [&](int m) { return rl[m]; }, [&](int m) { return lds_nat<T>(Vs, RM, J, m); });
                F pf[CB];
#pragma unroll
                for (int I = J; I < CB; ++I) {
                    f32x4 p = nn_tile<T, MB>(Gs, RM, I, Vs, RM, J);
                    if (I == J) p = diag.query(p);
                    pf[I] = O::cvt(p);
                }
                dotk<T>(d, J, CB, [&](int I) { return O::tr_frag(Qs, RE, I, b); }, [&](int I) { return pf[I]; });
                pend[J] = d;
            }
            // R^T += dO_c^T Q_c[:, b]
#pragma unroll
            for (int m = 0; m < MB; ++m)
                dotk<T>(W[m], 0, CB, [&](int I) { return O::tr_frag(Gs, RM, I, m); },
                        [&](int I) { return O::tr_frag(Qs, RE, I, b); });
        } else if constexpr (ROLE == kDV) {
            F rh[EB], rl[EB];  // A = R^T (rows m, k = e)
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                if constexpr (HILO) O::split(X[e], rh[e], rl[e]);
                else rh[e] = O::cvt(X[e]);
            }
#pragma unroll
            for (int J = 0; J < CB; ++J) {
                // dV^T = R^T K_J^T + dO^T A with A(I, J) = Q_I K_J^T for I >= J
                f32x4 d = dotz<T>(0, EB, [&](int e) { return rh[e]; }, [&](int e) { return lds_nat<T>(Ks, RE, J, e); });
                if constexpr (HILO)
                    dotk<T>(d, 0, EB, [&](int e) { return rl[e]; }, [&](int e) { return lds_nat<T>(Ks, RE, J, e); });
                F af[CB];
#pragma unroll
                for (int I = J; I < CB; ++I) {
                    f32x4 a = nn_tile<T, EB>(Qs, RE, I, Ks, RE, J);
                    if (I == J) a = diag.query(a);
                    af[I] = O::cvt(a);
                }
                dotk<T>(d, J, CB, [&](int I) { return O::tr_frag(Gs, RM, I, b); }, [&](int I) { return af[I]; });
                pend[J] = d;
            }
            // R += Q_c^T dO_c[:, b]
#pragma unroll
            for (int e = 0; e < EB; ++e)
                dotk<T>(X[e], 0, CB, [&](int I) { return O::tr_frag(Qs, RE, I, e); },
                        [&](int I) { return O::tr_frag(Gs, RM, I, b); });
        }
        // Stores go after this step's prefetch: memory operations complete in
        // issue order, so the rows waited for at a later step were issued
        // before these stores and never wait for them.
        store_pending(row0);
      }
    }
}

template <typename T, int E, int M, int C, int NPF, bool HILO>
__global__ __launch_bounds__(192) void cp_bwd_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                     const T *__restrict__ V, const T *__restrict__ G,
                                                     const float *__restrict__ state_in, T *__restrict__ dQ,
                                                     T *__restrict__ dK, T *__restrict__ dV, int L, int NS) {
    constexpr int EB = E / 16, MB = M / 16;
    constexpr int P = EB > MB ? EB : MB;
    constexpr int RE = Stage<T, 192, C, E>::RS, RM = Stage<T, 192, C, M>::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;
    __shared__ __attribute__((aligned(16))) T lds[2 * BUF];

    int slice, b;
    map_block(blockIdx.x, NS, P, slice, b);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int64_t oe = (int64_t)slice * L * E, om = (int64_t)slice * L * M;
    const T *q_ = Q + oe, *k_ = K + oe, *v_ = V + om, *g_ = G + om;
    const float *st = state_in ? state_in + (int64_t)slice * E * M : nullptr;
    if (w == 0 && b < EB)
        bwd_sweep<T, E, M, C, NPF, HILO, kDQ>(q_, k_, v_, g_, st, dQ + oe, L, b, lds);
    else if (w == 1 && b < EB)
        bwd_sweep<T, E, M, C, NPF, HILO, kDK>(q_, k_, v_, g_, st, dK + oe, L, b, lds);
    else if (w == 2 && b < MB)
        bwd_sweep<T, E, M, C, NPF, HILO, kDV>(q_, k_, v_, g_, st, dV + om, L, b, lds);
    else
        bwd_sweep<T, E, M, C, NPF, HILO, kIdle>(q_, k_, v_, g_, st, nullptr, L, b, lds);
}

}  // namespace cp
