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
// A workgroup owns one (n, h) slice and a group of NW 16-column blocks of V
// and Out; wave w owns column block w of the group for every row of the
// chunk.  Per chunk all threads copy Q, K (all E columns) and the group's V
// columns into LDS (double buffered, one barrier per chunk) while the next
// chunks' loads are in flight.  Each wave then
//   - reads the chunk's Q and K rows (16-byte natural reads),
//   - forms the causal score tiles A^T(J, I) = K_J Q_I^T, J <= I (every wave
//     forms all of them: cheaper than exchanging them through LDS),
//   - accumulates its output block Out^T = V^T A^T + S^T Q^T, and
//   - updates its E x 16 block of the state, S += K^T V (transposed reads).
// So each row of the inputs enters LDS once per workgroup and the state is
// updated once, by the wave that owns its columns.  Products run in the
// transposed orientation so that every operand is a natural or transposed
// LDS read or an accumulator tile.
//
// Normalised form (NORM): out_i = phi(q_i)^T S_i / (phi(q_i) . z_i + eps) with
// z_i = sum_{j<=i} phi(k_j).  phi is applied while the chunk is copied into
// LDS.  The denominator of token i is the masked column sum of the chunk's
// score tiles plus phi(q_i) . z_{c-1} (one extra MFMA row beside the
// numerator, in every wave); z is carried like S (z_c = z_{c-1} + column sums
// of phi(K_c)) and enters the product as a hi + lo pair of operands; the
// division happens before the store.
#pragma once

#include "cp_device.hpp"

namespace cp {

// The chunk loop of one wave over rows [rb, re) of its slice, for the query
// row blocks of row set H of RS (the row sets of a slice: RSPLIT waves of each
// workgroup times the row groups of workgroups).  Every wave runs the same
// staging and barriers.
//   Numerator waves (DEN = false) own output column block cb of the
//   workgroup's group and carry the state S (by reference) of those columns.
//   Normalised form, with a denominator wave (DW): that wave (DEN = true,
//   one per workgroup) carries z instead: per chunk it forms the score tiles
//   of the workgroup's rows, d_i = phi(q_i) . z_{c-1} + sum_{j<=i in chunk}
//   A(i, j) + eps, and hands d to the numerator waves through LDS; they
//   divide and store their tiles of chunk c one step later, after the next
//   barrier, so the normaliser is computed once per row instead of once per
//   column block.  Without it (!DW: wide heads, where the extra wave's
//   registers would halve the workgroups per CU) every numerator wave also
//   carries z and forms the denominators of its own tiles (z entering the
//   products as a hi + lo pair of operands).
template <typename T, int E, int M, int C, int NW, int RSPLIT, int RS, int NPF, bool NORM, bool FMAP, bool DW,
          bool DEN, int H>
__device__ __forceinline__ void fwd_sweep(const T *q_, const T *k_, const T *v_, T *o_, float *den_, int rb,
                                          int re, int grp, int cb, float eps, lds_t<T> *lds, f32x4 (&S)[E / 16],
                                          f32x4 (&z)[E / 16], int Ea, int Ma) {
    using O = Ops<T>;
    using F = typename O::frag;
    using EO = EOps<T, E>;
    using RF = typename EO::rf;
    constexpr int EB = E / 16, CB = C / 16, KS = EO::STEPS;
    constexpr int NT = 64 * (NW * RSPLIT + (NORM && DW ? 1 : 0)), MW = 16 * NW;
    constexpr bool SELF = NORM && !DW;         // numerator waves form their own denominators
    constexpr bool DELAY = NORM && DW && !DEN;  // numerator waves divide one step later
    // Q: with one row set per workgroup and row groups, only the rows of the
    // workgroup's own row blocks are staged (K and V: every row, for the
    // state update and the scores of earlier key blocks)
    constexpr bool QOWN = RSPLIT == 1 && RS > 1;
    constexpr int CQ = QOWN ? 16 * owned_count<CB, RS>(H) : C;
    using SQ = Stage<T, NT, CQ, E, typename std::conditional<QOWN, OwnedRows<CB, RS, H>, AllRows>::type>;
    using SK = Stage<T, NT, C, E>;
    using SV = Stage<T, NT, C, MW>;
    constexpr int RQ = SK::RS, RV = SV::RS;
    constexpr int BUF = 2 * C * RQ + C * RV;  // Q, K, V columns of the group
    constexpr int JMAX = last_block<CB, RS>(H);  // key blocks this wave scores: J <= JMAX
    static_assert(!DEN || (NORM && DW), "the denominator wave belongs to the normalised form");
    // NORM: the denominators of the last two chunks follow the row buffers
    float *const denbuf = reinterpret_cast<float *>(lds + 2 * BUF);

    const Diag diag;

    // Ring of NPF register stages: NPF-1 chunks are in flight while one is
    // computed.  The step loop is padded to a multiple of NPF; padded chunks
    // lie past re, load as zero and store nothing.
    struct Stages {
        SQ q;
        SK k;
        SV v;
    };
    const int col0 = 16 * grp * NW;
    Stages st[NPF];
#pragma unroll
    for (int s = 0; s < NPF - 1; ++s) {
        st[s].q.load(Rows<T>(q_, Ea, rb + s * C, re, C), 0, Ea);
        st[s].k.load(Rows<T>(k_, Ea, rb + s * C, re, C), 0, Ea);
        st[s].v.load(Rows<T>(v_, Ma, rb + s * C, re, C), col0, Ma);
        __builtin_amdgcn_sched_barrier(0);  // stages complete in order
    }

    // NORM numerator waves: the previous chunk's output tiles, divided by its
    // denominators once they are in LDS
    f32x4 prev[CB];
#pragma unroll
    for (int I = 0; I < CB; ++I) prev[I] = zero4();
    auto finish_prev = [&](int prow0, int pc) {
        if constexpr (DELAY) {
            const float *dn = denbuf + (pc & 1) * C;
            const Rows<T> ro(o_, Ma, prow0, re, C);
#pragma unroll
            for (int I = 0; I < CB; ++I)
                if (owns_block<CB, RS>(H, I)) {
                    const float rcp = 1.f / dn[16 * I + lane_r()];
                    f32x4 o = prev[I];
#pragma unroll
                    for (int t = 0; t < 4; ++t) o[t] *= rcp;
                    st_out<T>(ro, I, grp * NW + cb, o, Ma);
                }
        }
    };

    const int nchunks = (re - rb + C - 1) / C;
    const int nsteps = (nchunks + NPF - 1) / NPF * NPF;
    for (int c0 = 0; c0 < nsteps; c0 += NPF) {
#pragma unroll
        for (int s = 0; s < NPF; ++s) {
            const int c = c0 + s;
            const int row0 = rb + c * C;
            lds_t<T> *Qs = lds + (c & 1) * BUF, *Ks = Qs + C * RQ, *Vs = Ks + C * RQ;
            st[s].q.template store<NORM && FMAP>(Qs, row0, re, Ea);
            st[s].k.template store<NORM && FMAP>(Ks, row0, re, Ea);
            st[s].v.store(Vs);
            __syncthreads();
            // The next chunk's loads are issued one array at a time between
            // the products below, and the output tiles in the middle of the
            // state update, so that the vector memory unit drains while the
            // matrix cores work.  Stores go after the step's loads: memory
            // operations complete in issue order, so the rows waited for at a
            // later step never wait for these stores.
            Stages &nx = st[(s + NPF - 1) % NPF];
            const int nrow0 = row0 + (NPF - 1) * C;
            f32x4 pend[CB];  // this step's output tiles (owned row blocks)
            float pden[CB];  // SELF: their denominators (row 16 I + r)
            int nload = 0;   // arrays of the next chunk whose loads are issued
            auto issue_load = [&]() {
                if (nload == 0) nx.q.load(Rows<T>(q_, Ea, nrow0, re, C), 0, Ea);
                if (nload == 1) nx.k.load(Rows<T>(k_, Ea, nrow0, re, C), 0, Ea);
                if (nload == 2) nx.v.load(Rows<T>(v_, Ma, nrow0, re, C), col0, Ma);
                ++nload;
                __builtin_amdgcn_sched_barrier(0);
            };
            // the step's output tiles (after every owned row block is done)
            auto issue_store = [&]() {
                if constexpr (!NORM || SELF) {
                    const Rows<T> ro(o_, Ma, row0, re, C);
#pragma unroll
                    for (int I = 0; I < CB; ++I)
                        if (owns_block<CB, RS>(H, I)) st_out<T>(ro, I, grp * NW + cb, pend[I], Ma);
                }
                if constexpr (SELF) {  // the denominators, from the first column block's waves
                    if (den_ && grp * NW + cb == 0 && lane_g() == 0) {
                        const Rows<float> rd(den_, 1, row0, re, C);
#pragma unroll
                        for (int I = 0; I < CB; ++I)
                            if (owns_block<CB, RS>(H, I))
                                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, pden[I]), rd.rsrc,
                                                                      (16 * I + lane_r()) * 4, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            issue_load();
            if constexpr (DELAY) {
                // the previous chunk, now that its denominators are in LDS
                if (c > 0) finish_prev(row0 - C, c - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            F vt[CB];  // V_J^T fragments of this wave's columns
            if constexpr (!DEN) {
#pragma unroll
                for (int b = 0; b < CB; ++b) vt[b] = O::tr_frag(Vs, RV, b, cb);
            }

            RF kf[CB][KS];
#pragma unroll
            for (int b = 0; b <= JMAX; ++b)
#pragma unroll
                for (int k = 0; k < KS; ++k) kf[b][k] = EO::load(Ks, RQ, b, k);
            // S_{c-1} (or, in the denominator wave, z_{c-1}) as A operands;
            // SELF: z_{c-1} as a hi + lo pair
            RF sa[KS], zh[KS], zl[KS];
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                sa[k] = EO::state(S, k);
                if constexpr (SELF) EO::state_split(z, k, zh[k], zl[k]);
            }

#pragma unroll
            for (int I = 0; I < CB; ++I) {
                if (!owns_block<CB, RS>(H, I)) continue;
                RF qf[KS];
#pragma unroll
                for (int k = 0; k < KS; ++k) qf[k] = EO::load(Qs, RQ, QOWN ? owned_index<CB, RS>(H, I) : I, k);
                // inter-chunk: Out^T += S^T Q_I^T (denominator: z . q_i in every row)
                f32x4 o = zero4(), d = zero4();
#pragma unroll
                for (int k = 0; k < KS; ++k) EO::mma(o, sa[k], qf[k]);
                if constexpr (SELF) {
#pragma unroll
                    for (int k = 0; k < KS; ++k) {
                        EO::mma(d, zh[k], qf[k]);
                        if constexpr (EO::SPLIT_STATE) EO::mma(d, zl[k], qf[k]);
                    }
                }
                // intra-chunk: Out^T += V^T A^T with A^T(J, I) = K_J Q_I^T
                // masked on the diagonal, key blocks J <= I taken in pairs
                // (denominator: the column sums of A^T)
#pragma unroll
                for (int J0 = 0; J0 <= I; J0 += 2) {
                    f32x4 a0 = zero4();
#pragma unroll
                    for (int k = 0; k < KS; ++k) EO::mma(a0, kf[J0][k], qf[k]);
                    if (J0 == I) a0 = diag.keys(a0);
                    F at1 = O::zero(), vt1 = O::zero();
                    if (J0 + 1 <= I) {
                        f32x4 a1 = zero4();
#pragma unroll
                        for (int k = 0; k < KS; ++k) EO::mma(a1, kf[J0 + 1][k], qf[k]);
                        if (J0 + 1 == I) a1 = diag.keys(a1);
                        at1 = O::cvt(a1);
                        if constexpr (!DEN) vt1 = vt[J0 + 1];
                    }
                    const F at0 = O::cvt(a0);
                    if constexpr (DEN) O::mma2(o, O::ones(), O::ones(), at0, at1);
                    else O::mma2(o, vt[J0], vt1, at0, at1);
                    if constexpr (SELF) O::mma2(d, O::ones(), O::ones(), at0, at1);
                }
                if constexpr (SELF) {
                    // every row of the tile holds the same column sums
                    const float rcp = 1.f / (d[0] + eps);
#pragma unroll
                    for (int t = 0; t < 4; ++t) o[t] *= rcp;
                    pden[I] = d[0] + eps;
                }
                if constexpr (DEN) {
                    // lane (g, r) holds d of query row 16 I + r (every row of
                    // the tile is the same)
                    const float d = o[0] + eps;
                    if (lane_g() == 0) {
                        denbuf[(c & 1) * C + 16 * I + lane_r()] = d;
                        if (den_) {
                            const Rows<float> rd(den_, 1, row0, re, C);
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, d), rd.rsrc,
                                                                  (16 * I + lane_r()) * 4, 0, 0);
                        }
                    }
                }
                pend[I] = o;
                issue_load();
            }
            while (nload < 3) issue_load();

            // S_c = S_{c-1} + K_c^T V_c  (denominator wave: z_c = z_{c-1} + K_c^T 1)
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                if constexpr (DEN)
                    dotk<T>(S[e], 0, CB, [&](int J) { return EO::tr_e(Ks, RQ, J, e); }, [&](int) { return O::ones(); });
                else
                    dotk<T>(S[e], 0, CB, [&](int J) { return EO::tr_e(Ks, RQ, J, e); }, [&](int J) { return vt[J]; });
                if constexpr (SELF)
                    dotk<T>(z[e], 0, CB, [&](int J) { return EO::tr_e(Ks, RQ, J, e); }, [&](int) { return O::ones(); });
                if (e == (EB - 1) / 2) issue_store();
            }
            if constexpr (DELAY) {
#pragma unroll
                for (int I = 0; I < CB; ++I) prev[I] = pend[I];
            }
        }
    }
    if constexpr (NORM && DW) {
        // the last chunk: its denominators become visible after one more barrier
        __syncthreads();
        if constexpr (DELAY) finish_prev(rb + (nsteps - 1) * C, nsteps - 1);
    }
}

// The state increments of the segments of a forward over sequence segments
// (see below): workgroup (slice s, segment g) sums, over the rows of segment
// g, dS = sum_j k_j v_j^T and, for the normalised form, dz = sum_j k_j (k =
// phi of the raw keys when FMAP), and writes them to ws[s][g] (E*M floats of
// dS, row e and column m, then E floats of dz).  Only K and V are read: per
// chunk of C rows all threads copy K and V into LDS (one barrier per chunk,
// NPF-1 chunks in flight), and wave w adds K^T V into the state tiles of its
// CW column blocks of M (and of its share of the E/16 tiles of dz, as K^T 1).
// The segments' increments are independent of each other, so this pass runs
// at the rate of its two input streams; the last segment's increment is never
// needed and not computed.
//
// The first job covers segments first1 .. first1 + nseg - 2 (first1 = 1: the
// backward from the final state, which subtracts the later segments'
// increments from it).  An optional second job (K2 != NULL) runs in the same
// launch, over segments
// 1 .. nseg-1 (the first one's is never needed), into ws2: the backward's
// suffix carries.  Causal product: dR = sum_i q_i dO_i^T (K2 = Q, V2 = dO).
// Normalised form: dR = sum_i phi(q_i) dn_i^T and dr = sum_i dd_i phi(q_i),
// with dn_i = dO_i / den_i and dd_i = -(dO_i . out_i) / den_i formed while dO
// is staged (O2, den2: the forward's output and denominators), dd entering
// the product K2^T dd as a hi + lo pair of operands.
//
// Each segment's increment may be computed in sub parts (consecutive runs of
// whole chunks, the last ones possibly empty) by as many workgroups, into
// consecutive slots: slot seg * sub + u of the slice holds part u of segment
// seg, and a consumer sums the slots of the segments it needs.  (Over few
// slices the increment pass has fewer workgroups than CUs, and the normalised
// backward's second job, which also reads the output and forms dn and dd,
// takes longer than the first: finer parts keep every CU busy.)
template <typename T, int E, int M, int C, int NW, int NPF, bool NORM, bool FMAP>
__global__ __launch_bounds__(64 * NW) void cp_seg_state_kernel(const T *__restrict__ K1, const T *__restrict__ V1,
                                                               float *__restrict__ ws1, const T *__restrict__ K2,
                                                               const T *__restrict__ V2, const T *__restrict__ O2,
                                                               const float *__restrict__ den2,
                                                               float *__restrict__ ws2, int L, int NS, int seg_len,
                                                               int sub, int first1, int Ea, int Ma) {
    using O = Ops<T>;
    using F = typename O::frag;
    using EO = EOps<T, E>;
    constexpr int EB = E / 16, MB = M / 16, CB = C / 16, CW = MB / NW, NT = 64 * NW;
    static_assert(MB % NW == 0, "waves split the column blocks evenly");
    static_assert(NPF >= 2, "the load ring needs at least two stages");
    using SK = Stage<T, NT, C, E>;
    using SV = Stage<T, NT, C, M>;
    constexpr int RK = SK::RS, RV = SV::RS;
    constexpr int BUF = C * RK + C * RV;
    constexpr int WS = E * M + E;
    constexpr int DDE = NORM ? 2 * C * 4 / (int)sizeof(lds_t<T>) : 0;  // two chunks of dd (second job)
    // dz tiles (e-tiles of K^T 1) dealt round robin to the waves
    constexpr int ZT = (EB + NW - 1) / NW;
    __shared__ __attribute__((aligned(16))) lds_t<T> lds[2 * BUF + DDE];

    const int nseg = (L + seg_len - 1) / seg_len, nparts = (nseg - 1) * sub;  // parts per job
    int slice, part;
    map_block(blockIdx.x, NS, (K2 ? 2 : 1) * nparts, slice, part);
    const bool second = part >= nparts;
    const int pj = second ? part - nparts : part;
    const int seg = (second ? 1 : first1) + pj / sub, u = pj % sub;
    const T *K = second ? K2 : K1, *V = second ? V2 : V1;
    float *ws = second ? ws2 : ws1;
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane_g(), r = lane_r();
    const T *k_ = K + (int64_t)slice * L * Ea;
    const T *v_ = V + (int64_t)slice * L * Ma;
    // part u of the segment: a run of whole chunks of this kernel's C (the
    // segment length is a multiple of the sweep's chunk, which may be
    // shorter), cut at the segment's end and empty past it
    const int send = seg * seg_len + seg_len < L ? seg * seg_len + seg_len : L;
    const int plen = ((seg_len + C - 1) / C + sub - 1) / sub * C, pb = seg * seg_len + u * plen;
    const int rb = pb < send ? pb : send, re = pb + plen < send ? pb + plen : send;
    // normalised second job: dn and dd from dO (v_), the output and den
    const bool dnj = NORM && second;
    NormIn<T> nin{nullptr, nullptr, nullptr, nullptr};
    if (dnj) {
        nin.o = O2 + (int64_t)slice * L * Ma;
        nin.den = den2 + (int64_t)slice * L;
    }
    float *const ddbuf = reinterpret_cast<float *>(lds + 2 * BUF);

    f32x4 S[CW][EB], Z[ZT];
#pragma unroll
    for (int x = 0; x < CW; ++x)
#pragma unroll
        for (int e = 0; e < EB; ++e) S[x][e] = zero4();
#pragma unroll
    for (int i = 0; i < ZT; ++i) Z[i] = zero4();

    struct Stages {
        SK k;
        SV v;
        SV o;
        float den[NORM ? SV::NP : 1];
        __device__ __forceinline__ void load(const T *k_, const T *v_, NormIn<T> nin, bool dnj, int row0, int re,
                                             int Ea, int Ma) {
            k.load(Rows<T>(k_, Ea, row0, re, C), 0, Ea);
            v.load(Rows<T>(v_, Ma, row0, re, C), 0, Ma);
            if constexpr (NORM) {
                if (dnj) {
                    o.load(Rows<T>(nin.o, Ma, row0, re, C), 0, Ma);
                    const Rows<float> rd(nin.den, 1, row0, re, C);
#pragma unroll
                    for (int i = 0; i < SV::NP; ++i) {
                        const int p = (int)threadIdx.x + i * NT;
                        den[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                               rd.rsrc, p < SV::P ? 4 * (p / SV::PPR) : kVoid, 0, 0));
                    }
                }
            }
        }
    };
    Stages st[NPF];
#pragma unroll
    for (int i = 0; i < NPF - 1; ++i) {
        st[i].load(k_, v_, nin, dnj, rb + i * C, re, Ea, Ma);
        __builtin_amdgcn_sched_barrier(0);  // stages complete in order
    }
    const int nchunks = (re - rb + C - 1) / C;
    const int nsteps = (nchunks + NPF - 1) / NPF * NPF;
    for (int c0 = 0; c0 < nsteps; c0 += NPF) {
#pragma unroll
        for (int i = 0; i < NPF; ++i) {
            const int c = c0 + i;
            const int row0 = rb + c * C;
            lds_t<T> *Ks = lds + (c & 1) * BUF, *Vs = Ks + C * RK;
            float *dds = ddbuf + (c & 1) * C;
            st[i].k.template store<NORM && FMAP>(Ks, row0, re, Ea);
            if constexpr (NORM) {
                if (dnj) store_dn<T>(st[i].v, st[i].o, st[i].den, Vs, dds);
                else st[i].v.store(Vs);
            } else {
                st[i].v.store(Vs);
            }
            __syncthreads();
            Stages &nx = st[(i + NPF - 1) % NPF];
            nx.load(k_, v_, nin, dnj, row0 + (NPF - 1) * C, re, Ea, Ma);
            __builtin_amdgcn_sched_barrier(0);
            F vt[CW][CB];  // V_J^T fragments of the wave's column blocks
#pragma unroll
            for (int x = 0; x < CW; ++x)
#pragma unroll
                for (int J = 0; J < CB; ++J) vt[x][J] = O::tr_frag(Vs, RV, J, w * CW + x);
            // dz: the ones column; the normalised second job's dr: dd (hi + lo)
            F zh[CB], zl[CB];
            if constexpr (NORM) {
#pragma unroll
                for (int J = 0; J < CB; ++J) {
                    if (dnj) {
                        f32x4 x;
#pragma unroll
                        for (int t = 0; t < 4; ++t) x[t] = dds[16 * J + 4 * g + t];
                        O::split(x, zh[J], zl[J]);
                    } else {
                        zh[J] = O::ones();
                        zl[J] = O::zero();
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < EB; ++e) {
                F kt[CB];  // K^T fragments of e-tile e, shared by the column blocks
#pragma unroll
                for (int J = 0; J < CB; ++J) kt[J] = EO::tr_e(Ks, RK, J, e);
#pragma unroll
                for (int x = 0; x < CW; ++x) dotk<T>(S[x][e], 0, CB, [&](int J) { return kt[J]; }, [&](int J) { return vt[x][J]; });
                if constexpr (NORM)
                    if (e % NW == w) {
                        dotk<T>(Z[e / NW], 0, CB, [&](int J) { return kt[J]; }, [&](int J) { return zh[J]; });
                        if constexpr (sizeof(T) == 2)
                            if (dnj) dotk<T>(Z[e / NW], 0, CB, [&](int J) { return kt[J]; }, [&](int J) { return zl[J]; });
                    }
            }
        }
    }
    float *dS = ws + (((int64_t)slice * nseg + seg) * sub + u) * WS, *dz = dS + E * M;
#pragma unroll
    for (int x = 0; x < CW; ++x)
#pragma unroll
        for (int e = 0; e < EB; ++e)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                dS[(EO::ecol(e) + EO::estride * g + t) * M + 16 * (w * CW + x) + r] = S[x][e][t];
    if constexpr (NORM) {
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < EB; ++e)
                if (e % NW == w)
#pragma unroll
                    for (int t = 0; t < 4; ++t) dz[EO::ecol(e) + EO::estride * g + t] = Z[e / NW][t];
        }
    }
}

// Sequence segments: when slices are too few to fill the GPU, each slice is
// cut into nseg segments of seg_len rows (a multiple of C) and run in two
// launches.  The first (cp_seg_state_kernel) computes each segment's state
// increment dS = sum over its rows of k v^T (and dz = sum of phi(k)) into ws;
// the second starts segment s from the carried-in state (state_in, z_in) plus
// the exclusive sum of the increments of the segments before it (the chunked
// scan's carry, one level up) and sweeps only its own rows.  ws holds, per
// slice and segment, E*M floats of dS (row e, column m) then E floats of dz.
// With one segment, ws is unused (NULL).
//
// Workgroups per (slice, segment): G column groups times RG row groups.  A
// workgroup of row group rg holds RSPLIT waves per column block, of row sets
// rg * RSPLIT + h: the RG * RSPLIT row sets of a slice split each chunk's
// query row blocks (owns_block), so a row of the output is written by the
// waves of one workgroup only, and every workgroup of a slice carries the
// whole state of its column group.  The normalised form (NORM, RSPLIT = 1)
// adds one denominator wave per workgroup.
// waves of a workgroup (DWAVE: with a denominator wave)
template <int M, int G, int RSPLIT, bool DWAVE>
constexpr int fwd_waves() { return (M / 16 / G) * RSPLIT + (DWAVE ? 1 : 0); }

template <typename T, int E, int M, int C, int G, int RSPLIT, int RG, int NPF, bool NORM, bool FMAP, bool DW>
__global__ __launch_bounds__((64 * fwd_waves<M, G, RSPLIT, NORM && DW>())) void cp_fwd_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, T *__restrict__ Out,
    const float *__restrict__ state_in, const float *__restrict__ z_in, float *__restrict__ state_out,
    float *__restrict__ z_out, float *__restrict__ den, const float *__restrict__ ws, int L, int NS, int seg_len,
    int cum, float eps, int Ea, int Ma) {
    using EO = EOps<T, E>;
    constexpr int EB = E / 16, MB = M / 16, CB = C / 16;
    static_assert(MB % G == 0, "column groups split the column blocks evenly");
    static_assert(NPF >= 2, "the load ring needs at least two stages");
    constexpr int RS = RSPLIT * RG;
    static_assert(RS == 1 || (CB % (2 * RS) == 0), "row sets need pairs of row blocks");
    static_assert(RS <= 4, "at most four row sets");
    static_assert(!NORM || !DW || RSPLIT == 1, "a denominator wave serves one row set");
    constexpr bool DWAVE = NORM && DW;
    constexpr int NW = MB / G, NT = 64 * (NW * RSPLIT + (DWAVE ? 1 : 0)), MW = 16 * NW;
    constexpr int RQ = Stage<T, NT, C, E>::RS, RV = Stage<T, NT, C, MW>::RS;
    constexpr int BUF = 2 * C * RQ + C * RV;
    constexpr int DENB = DWAVE ? 2 * C * 4 / (int)sizeof(lds_t<T>) : 0;  // two chunks of denominators
    constexpr int WS = E * M + E;                                // floats per (slice, segment) in ws
    __shared__ __attribute__((aligned(16))) lds_t<T> lds[2 * BUF + DENB];

    const int nseg = (L + seg_len - 1) / seg_len;
    int slice, part;
    map_block(blockIdx.x, NS, G * RG * nseg, slice, part);
    const int grp = part % G, rg = (part / G) % RG, seg = part / (G * RG);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const bool den_wave = DWAVE && w == NW;
    const int cb = den_wave ? 0 : w % NW, h = den_wave ? 0 : w / NW;
    const int mb = grp * NW + cb;
    const int g = lane_g(), r = lane_r();
    // the tensors' own head sizes Ea <= E, Ma <= M (the kernel's tile sizes)
    const T *q_ = Q + (int64_t)slice * L * Ea;
    const T *k_ = K + (int64_t)slice * L * Ea;
    const T *v_ = V + (int64_t)slice * L * Ma;
    T *o_ = Out + (int64_t)slice * L * Ma;
    float *den_ = den ? den + (int64_t)slice * L : nullptr;
    const int rb = seg * seg_len, re = rb + seg_len < L ? rb + seg_len : L;
    const float *ws_slice = ws ? ws + (int64_t)slice * nseg * WS : nullptr;

    // Numerator waves: S[ecol(eb) + estride g + t][16 mb + r], and without a
    // denominator wave also z[ecol(eb) + estride g + t] (the same in every
    // lane r).  Denominator wave: z, in S.
    f32x4 S[EB], z[EB];
    const float *s0 = state_in ? state_in + (int64_t)slice * Ea * Ma : nullptr;
    const float *z0 = z_in ? z_in + (int64_t)slice * Ea : nullptr;
    // The carried-in state plus the increments of the segments before this
    // one (all of one segment's loads issued together).  The element of the
    // increments a lane adds: its S entry, or for the denominator wave its z
    // entry; without a denominator wave numerator waves add z as well.
    constexpr bool SELFZ = NORM && !DW;
#pragma unroll
    for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int row = EO::ecol(e) + EO::estride * g + t;
            float x = 0.f;
            if (den_wave) x = z0 && row < Ea ? z0[row] : 0.f;
            else x = s0 && row < Ea && 16 * mb + r < Ma ? s0[row * Ma + 16 * mb + r] : 0.f;
            S[e][t] = x;
            z[e][t] = SELFZ && z0 && row < Ea ? z0[row] : 0.f;
        }
    // cum: the slots hold inclusive prefix sums (cp_seg_scan_kernel), one read
    for (int p = cum && seg > 0 ? seg - 1 : 0; p < seg; ++p) {
        const float *inc = ws_slice + (int64_t)p * WS;
#pragma unroll
        for (int e = 0; e < EB; ++e)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int row = EO::ecol(e) + EO::estride * g + t;
                S[e][t] += inc[den_wave ? E * M + row : row * M + 16 * mb + r];
                if constexpr (SELFZ) z[e][t] += inc[E * M + row];
            }
    }
    const int H = rg * RSPLIT + h;  // the wave's row set
    if (den_wave) {
        if constexpr (DWAVE) {
#define CP_FWD_SWEEP(HH)                                                                                          \
    fwd_sweep<T, E, M, C, NW, RSPLIT, RS, NPF, NORM, FMAP, DW, true, ((HH) < RS ? (HH) : 0)>(                    \
        q_, k_, v_, o_, den_, rb, re, grp, cb, eps, lds, S, z, Ea, Ma)
            if (H == 0 || RS == 1) CP_FWD_SWEEP(0);
            else if (H == 1 || RS == 2) CP_FWD_SWEEP(1);
            else if (H == 2 || RS == 3) CP_FWD_SWEEP(2);
            else CP_FWD_SWEEP(3);
#undef CP_FWD_SWEEP
        }
    } else {
#define CP_FWD_SWEEP(HH)                                                                                          \
    fwd_sweep<T, E, M, C, NW, RSPLIT, RS, NPF, NORM, FMAP, DW, false, ((HH) < RS ? (HH) : 0)>(                   \
        q_, k_, v_, o_, den_, rb, re, grp, cb, eps, lds, S, z, Ea, Ma)
        if (H == 0 || RS == 1) CP_FWD_SWEEP(0);
        else if (H == 1 || RS == 2) CP_FWD_SWEEP(1);
        else if (H == 2 || RS == 3) CP_FWD_SWEEP(2);
        else CP_FWD_SWEEP(3);
#undef CP_FWD_SWEEP
    }

    if (H == 0 && seg == nseg - 1) {  // the final state of the slice
        if (den_wave) {
            float *zt_ = z_out ? z_out + (int64_t)slice * Ea : nullptr;
            if (zt_ && r == 0 && grp == 0) {
#pragma unroll
                for (int e = 0; e < EB; ++e)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int row = EO::ecol(e) + EO::estride * g + t;
                        if (row < Ea) zt_[row] = S[e][t];
                    }
            }
        } else {
            float *st_ = state_out ? state_out + (int64_t)slice * Ea * Ma : nullptr;
            float *zt_ = NORM && !DW && z_out && mb == 0 ? z_out + (int64_t)slice * Ea : nullptr;
#pragma unroll
            for (int e = 0; e < EB; ++e)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int row = EO::ecol(e) + EO::estride * g + t;
                    if (st_ && row < Ea && 16 * mb + r < Ma) st_[row * Ma + 16 * mb + r] = S[e][t];
                    if (zt_ && r == 0 && row < Ea) zt_[row] = z[e][t];
                }
        }
    }
}

}  // namespace cp
