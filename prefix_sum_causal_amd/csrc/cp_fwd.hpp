// cp_fwd.hpp -- chunked-scan forward kernel of the causal dot product and of
// normalised causal linear attention, for gfx950.
//
// Method: the causal dot product of "Transformers are RNNs", Algorithm 1, as
// named in the opening post of "Dot Product Computes Wrong Values"
// (triton-lang/triton issue 217): S_i = S_{i-1} + k_i v_i^T, out_i = q_i^T S_i,
// inclusive of token i (the loop excerpt later on that page updates the state
// before reading the row).  Split at chunk boundaries of C tokens this is
//
//     Out_c = (Q_c K_c^T (.) T) V_c + Q_c S_{c-1},   S_c = S_{c-1} + K_c^T V_c
//
// with T the inclusive lower-triangular mask: the prefix sum runs serially
// over chunks and in parallel (as small dense products) inside a chunk.
//
// One wave owns one (n, h) slice and one 16-column block mb of the output.
// It streams Q and K in full (the other column blocks of the slice run on the
// same XCD and take the same rows from L2), V only for its columns, keeps the
// E x 16 block of the state in MFMA accumulators across all chunks, and works
// in the transposed output orientation Out^T = V^T A^T + S^T Q^T so that every
// operand comes either from a natural load, from an LDS transpose read, or
// from an accumulator tile without shuffles (see cp_device.hpp).
//
// Normalised form (NORM): out_i = phi(q_i)^T S_i / (phi(q_i) . z_i + eps) with
// z_i = sum_{j<=i} phi(k_j).  Per chunk, the denominator of token i is the
// masked row sum of the chunk's scores plus phi(q_i) . z_{c-1}; both are one
// extra MFMA row computed next to the numerator, z is carried across chunks
// like S (z_c = z_{c-1} + column sums of phi(K_c)), and the division happens
// in registers before the store.
#pragma once

#include "cp_device.hpp"

namespace cp {

template <typename T, int E, int M, int C>
struct FwdChunk {
    using F = typename Ops<T>::frag;
    static constexpr int EB = E / 16, CB = C / 16;
    F q[CB][EB];  // Q[row0 + 16 I + r][16 eb + 4g + t]
    F k[CB][EB];  // K[row0 + 16 J + r][16 eb + 4g + t]
    F v[CB];      // V[row0 + 16 J + r][16 mb + 4g + t]

    // Rows at or past L (and whole chunks past the end) load as zero.
    __device__ __forceinline__ void load(const T *q_, const T *k_, const T *v_, int row0, int L, int mb) {
        const Rows<T> rq(q_, E, row0, L, C), rk(k_, E, row0, L, C), rv(v_, M, row0, L, C);
#pragma unroll
        for (int b = 0; b < CB; ++b) {
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                q[b][e] = ld_nat<T>(rq, b, e);
                k[b][e] = ld_nat<T>(rk, b, e);
            }
            v[b] = ld_nat<T>(rv, b, mb);
        }
    }
};

template <typename T, int E, int M, int C, int NBUF, bool NORM, bool HILO>
__global__ __launch_bounds__(64) void cp_fwd_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                    const T *__restrict__ V, T *__restrict__ Out,
                                                    float *__restrict__ state_out, int L, int NS,
                                                    float eps, int fmap) {
    static_assert(NBUF >= 2, "the pipeline needs at least two chunk buffers");
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int EB = E / 16, MB = M / 16, CB = C / 16;
    constexpr int RSK = E + O::kPad, RSV = 16 + O::kPad;
    __shared__ __attribute__((aligned(16))) T ldsK[C * RSK];
    __shared__ __attribute__((aligned(16))) T ldsV[C * RSV];

    int slice, mb;
    map_block(blockIdx.x, NS, MB, slice, mb);
    const int g = lane_g(), r = lane_r();
    const T *q_ = Q + (int64_t)slice * L * E;
    const T *k_ = K + (int64_t)slice * L * E;
    const T *v_ = V + (int64_t)slice * L * M;
    T *o_ = Out + (int64_t)slice * L * M;

    f32x4 S[EB];  // S[16 eb + 4g + t][16 mb + r]
    f32x4 z[EB];  // z[16 eb + 4g + t] (same in every lane r)
#pragma unroll
    for (int e = 0; e < EB; ++e) {
        S[e] = zero4();
        z[e] = zero4();
    }

    // The chunk loop is padded to a multiple of NBUF; padded chunks lie past
    // L, load as zero and store nothing, so every step issues the same loads.
    const int nchunks = (L + C - 1) / C;
    const int nsteps = (nchunks + NBUF - 1) / NBUF * NBUF;
    FwdChunk<T, E, M, C> buf[NBUF];
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s) {
        buf[s].load(q_, k_, v_, s * C, L, mb);
        __builtin_amdgcn_sched_barrier(0);  // buffers complete in order
    }

    for (int c0 = 0; c0 < nsteps; c0 += NBUF) {
#pragma unroll
        for (int s = 0; s < NBUF; ++s) {
            const int c = c0 + s;
            const int row0 = c * C;
            FwdChunk<T, E, M, C> &cur = buf[s];
            if constexpr (NORM) {
                if (fmap) {
                    // phi(0) = 1, so rows past L are zeroed again after the map
#pragma unroll
                    for (int b = 0; b < CB; ++b) {
                        const bool valid = row0 + 16 * b + r < L;
#pragma unroll
                        for (int e = 0; e < EB; ++e) {
                            const F pq = phi_frag<T>(cur.q[b][e]), pk = phi_frag<T>(cur.k[b][e]);
                            cur.q[b][e] = valid ? pq : O::zero();
                            cur.k[b][e] = valid ? pk : O::zero();
                        }
                    }
                }
            }
            // natural copies of K (all columns) and V (this block) for the
            // transposed reads of the state update and of V^T A^T
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int e = 0; e < EB; ++e) st_lds<T>(ldsK, RSK, b, e, cur.k[b][e]);
                st_lds<T>(ldsV, RSV, b, 0, cur.v[b]);
            }
            wave_lds_sync();
            F kt[CB][EB], vt[CB];  // K[16 J + 4g + t][16 eb + r], V[16 J + 4g + t][16 mb + r]
#pragma unroll
            for (int b = 0; b < CB; ++b) {
#pragma unroll
                for (int e = 0; e < EB; ++e) kt[b][e] = O::tr_frag(ldsK, RSK, b, e);
                vt[b] = O::tr_frag(ldsV, RSV, b, 0);
            }
            // keep NBUF-1 chunks in flight while this one is computed
            buf[(s + NBUF - 1) % NBUF].load(q_, k_, v_, (c + NBUF - 1) * C, L, mb);
            // keep the prefetch here: sunk towards the loop end it would be
            // the youngest load at the next chunk and stall the pipeline
            __builtin_amdgcn_sched_barrier(0);

            // S_{c-1} (and z_{c-1}) as A operands: A = S^T (rows m, k = e)
            F sh[EB], sl[EB], zh[EB], zl[EB];
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                if constexpr (HILO) O::split(S[e], sh[e], sl[e]);
                else sh[e] = O::cvt(S[e]);
                if constexpr (NORM) O::split(z[e], zh[e], zl[e]);
            }

            const Rows<T> ro(o_, M, row0, L, C);
#pragma unroll
            for (int I = 0; I < CB; ++I) {
                f32x4 o = zero4(), d = zero4();
                // inter-chunk: Out^T += S^T Q_I^T
                dotk<T>(o, 0, EB, [&](int e) { return sh[e]; }, [&](int e) { return cur.q[I][e]; });
                if constexpr (HILO)
                    dotk<T>(o, 0, EB, [&](int e) { return sl[e]; }, [&](int e) { return cur.q[I][e]; });
                if constexpr (NORM) {
                    dotk<T>(d, 0, EB, [&](int e) { return zh[e]; }, [&](int e) { return cur.q[I][e]; });
                    dotk<T>(d, 0, EB, [&](int e) { return zl[e]; }, [&](int e) { return cur.q[I][e]; });
                }
                // intra-chunk scores A^T(J, I) = K_J Q_I^T, causal on the diagonal
                F at[CB];
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    f32x4 a = zero4();
                    dotk<T>(a, 0, EB, [&](int e) { return cur.k[J][e]; }, [&](int e) { return cur.q[I][e]; });
                    if (J == I) a = mask_keys_rows(a);
                    at[J] = O::cvt(a);
                }
                // Out^T += V^T A^T
                dotk<T>(o, 0, I + 1, [&](int J) { return vt[J]; }, [&](int J) { return at[J]; });
                if constexpr (NORM) {
                    dotk<T>(d, 0, I + 1, [&](int) { return O::ones(); }, [&](int J) { return at[J]; });
#pragma unroll
                    for (int t = 0; t < 4; ++t) o[t] = o[t] / (d[t] + eps);
                }
                st_out<T>(ro, I, mb, o);
            }

            // S_c = S_{c-1} + K_c^T V_c  (and z_c = z_{c-1} + K_c^T 1)
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                dotk<T>(S[e], 0, CB, [&](int J) { return kt[J][e]; }, [&](int J) { return vt[J]; });
                if constexpr (NORM)
                    dotk<T>(z[e], 0, CB, [&](int J) { return kt[J][e]; }, [&](int) { return O::ones(); });
            }
            wave_lds_sync();
        }
    }

    if constexpr (!NORM) {
        if (state_out) {
            float *st = state_out + (int64_t)slice * E * M;
#pragma unroll
            for (int e = 0; e < EB; ++e)
#pragma unroll
                for (int t = 0; t < 4; ++t) st[(16 * e + 4 * g + t) * M + 16 * mb + r] = S[e][t];
        }
    }
}

}  // namespace cp
