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
// A workgroup owns one (n, h) slice and one 16-column block mb of the output
// and runs RS waves.  Per chunk, all its threads copy Q, K (all E columns) and
// the V column block into LDS (double buffered, one barrier per chunk) while
// the next chunk's loads are in flight; each wave then keeps the E x 16 block
// of the state in MFMA accumulators (every wave carries the same state, which
// costs a few MFMAs and saves any exchange), and computes the output rows of
// its share of the chunk's 16-row blocks.  The shares are balanced pairs
// (block k and C/16-1-k carry equal causal work), so all workgroups do the
// same work per chunk and the M/16 workgroups of a slice, placed on one XCD,
// stay in step and take the slice's Q and K rows from its L2.  Products run
// in the transposed orientation Out^T = V^T A^T + S^T Q^T so that every
// operand is a natural or transposed LDS read or an accumulator tile.
//
// Normalised form (NORM): out_i = phi(q_i)^T S_i / (phi(q_i) . z_i + eps) with
// z_i = sum_{j<=i} phi(k_j).  phi is applied while the chunk is copied into
// LDS.  The denominator of token i is the masked row sum of the chunk's scores
// plus phi(q_i) . z_{c-1} (one extra MFMA row beside the numerator); z is
// carried like S (z_c = z_{c-1} + column sums of phi(K_c), the running
// inclusive sum of phi(k)); the division happens before the store.
#pragma once

#include "cp_device.hpp"

namespace cp {

// Query row block handled by wave w in round k: a snake over the waves, so
// that each wave gets block k and block C/16-1-k worth of causal work.
template <int RS>
__device__ __forceinline__ int owned_block(int k, int w) {
    return (k & 1) ? k * RS + (RS - 1 - w) : k * RS + w;
}

template <typename T, int E, int M, int C, int RS, int NPF, bool NORM, bool FMAP, bool HILO>
__global__ __launch_bounds__(64 * RS) void cp_fwd_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                         const T *__restrict__ V, T *__restrict__ Out,
                                                         float *__restrict__ state_out, int L, int NS,
                                                         float eps) {
    using O = Ops<T>;
    using F = typename O::frag;
    constexpr int NT = 64 * RS, EB = E / 16, MB = M / 16, CB = C / 16;
    static_assert(CB % RS == 0, "the chunk's row blocks are shared evenly by the waves");
    static_assert(NPF >= 2, "the load ring needs at least two stages");
    using SQ = Stage<T, NT, C, E>;
    using SV = Stage<T, NT, C, 16>;
    constexpr int RQ = SQ::RS, RV = SV::RS;
    constexpr int BUF = 2 * C * RQ + C * RV;  // Q, K, V block
    __shared__ __attribute__((aligned(16))) T lds[2 * BUF];

    int slice, mb;
    map_block(blockIdx.x, NS, MB, slice, mb);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane_g(), r = lane_r();
    const T *q_ = Q + (int64_t)slice * L * E;
    const T *k_ = K + (int64_t)slice * L * E;
    const T *v_ = V + (int64_t)slice * L * M;
    T *o_ = Out + (int64_t)slice * L * M;

    const Diag diag;
    f32x4 S[EB];  // S[16 eb + 4g + t][16 mb + r]
    f32x4 z[EB];  // z[16 eb + 4g + t] (same in every lane r)
#pragma unroll
    for (int e = 0; e < EB; ++e) {
        S[e] = zero4();
        z[e] = zero4();
    }

    // Ring of NPF register stages: NPF-1 chunks are in flight while one is
    // computed.  The step loop is padded to a multiple of NPF; padded chunks
    // lie past L, load as zero and store nothing.
    struct Stages {
        SQ q, k;
        SV v;
        __device__ __forceinline__ void load(const T *q_, const T *k_, const T *v_, int row0, int L, int mb) {
            q.load(Rows<T>(q_, E, row0, L, C), 0);
            k.load(Rows<T>(k_, E, row0, L, C), 0);
            v.load(Rows<T>(v_, M, row0, L, C), 16 * mb);
        }
    };
    Stages st[NPF];
#pragma unroll
    for (int s = 0; s < NPF - 1; ++s) {
        st[s].load(q_, k_, v_, s * C, L, mb);
        __builtin_amdgcn_sched_barrier(0);  // stages complete in order
    }

    constexpr int KB = CB / RS;  // row blocks per wave

    const int nchunks = (L + C - 1) / C;
    const int nsteps = (nchunks + NPF - 1) / NPF * NPF;
    for (int c0 = 0; c0 < nsteps; c0 += NPF) {
#pragma unroll
      for (int s = 0; s < NPF; ++s) {
        const int c = c0 + s;
        const int row0 = c * C;
        T *Qs = lds + (c & 1) * BUF, *Ks = Qs + C * RQ, *Vs = Ks + C * RQ;
        st[s].q.template store<NORM && FMAP>(Qs, row0, L);
        st[s].k.template store<NORM && FMAP>(Ks, row0, L);
        st[s].v.store(Vs);
        __syncthreads();
        st[(s + NPF - 1) % NPF].load(q_, k_, v_, row0 + (NPF - 1) * C, L, mb);
        __builtin_amdgcn_sched_barrier(0);

        // S_{c-1} (and z_{c-1}) as A operands: A = S^T (rows m, k = e)
        F sh[EB], sl[EB], zh[EB], zl[EB];
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            if constexpr (HILO) O::split(S[e], sh[e], sl[e]);
            else sh[e] = O::cvt(S[e]);
            if constexpr (NORM) O::split(z[e], zh[e], zl[e]);
        }

        f32x4 pend[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int I = owned_block<RS>(k, w);
            F qI[EB];  // Q[16 I + r][16 eb + 4g + t]
#pragma unroll
            for (int e = 0; e < EB; ++e) qI[e] = lds_nat<T>(Qs, RQ, I, e);
            f32x4 o = zero4(), d = zero4();
            // inter-chunk: Out^T += S^T Q_I^T
            dotk<T>(o, 0, EB, [&](int e) { return sh[e]; }, [&](int e) { return qI[e]; });
            if constexpr (HILO)
                dotk<T>(o, 0, EB, [&](int e) { return sl[e]; }, [&](int e) { return qI[e]; });
            if constexpr (NORM) {
                dotk<T>(d, 0, EB, [&](int e) { return zh[e]; }, [&](int e) { return qI[e]; });
                dotk<T>(d, 0, EB, [&](int e) { return zl[e]; }, [&](int e) { return qI[e]; });
            }
            // intra-chunk: Out^T += V^T A^T with A^T(J, I) = K_J Q_I^T masked
            // on the diagonal, key blocks J <= I taken in pairs
            for (int J0 = 0; J0 <= I; J0 += 2) {
                f32x4 a0 = nn_tile<T, EB>(Ks, RQ, J0, Qs, RQ, I);
                if (J0 == I) a0 = diag.keys(a0);
                F at1 = O::zero(), vt1 = O::zero();
                if (J0 + 1 <= I) {
                    f32x4 a1 = nn_tile<T, EB>(Ks, RQ, J0 + 1, Qs, RQ, I);
                    if (J0 + 1 == I) a1 = diag.keys(a1);
                    at1 = O::cvt(a1);
                    vt1 = O::tr_frag(Vs, RV, J0 + 1, 0);
                }
                const F at0 = O::cvt(a0);
                O::mma2(o, O::tr_frag(Vs, RV, J0, 0), vt1, at0, at1);
                if constexpr (NORM) O::mma2(d, O::ones(), O::ones(), at0, at1);
            }
            if constexpr (NORM) {
#pragma unroll
                for (int t = 0; t < 4; ++t) o[t] = o[t] / (d[t] + eps);
            }
            pend[k] = o;
        }
        // Stores go after this step's prefetch: memory operations complete in
        // issue order, so the rows waited for at a later step were issued
        // before these stores and never wait for them.
        {
            const Rows<T> ro(o_, M, row0, L, C);
#pragma unroll
            for (int k = 0; k < KB; ++k) st_out<T>(ro, owned_block<RS>(k, w), mb, pend[k]);
        }

        // S_c = S_{c-1} + K_c^T V_c  (and z_c = z_{c-1} + K_c^T 1)
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            dotk<T>(S[e], 0, CB, [&](int J) { return O::tr_frag(Ks, RQ, J, e); },
                    [&](int J) { return O::tr_frag(Vs, RV, J, 0); });
            if constexpr (NORM)
                dotk<T>(z[e], 0, CB, [&](int J) { return O::tr_frag(Ks, RQ, J, e); },
                        [&](int) { return O::ones(); });
        }
      }
    }

    if constexpr (!NORM) {
        if (state_out && w == 0) {
            float *st = state_out + (int64_t)slice * E * M;
#pragma unroll
            for (int e = 0; e < EB; ++e)
#pragma unroll
                for (int t = 0; t < 4; ++t) st[(16 * e + 4 * g + t) * M + 16 * mb + r] = S[e][t];
        }
    }
}

}  // namespace cp
