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
// state S0 (always so for the normalised form with fp32 I/O, where both
// directions sum compensated; see EXACT_PREFIX).  At the end the dV waves hold R_0 = sum_i q_i dO_i^T, the
// gradient of S0.  Carried states keep the
// rows of their contraction index (m or e) in the order of the 16-byte
// natural reads of the other operand (see EOps), so no operand is read twice.
#pragma once

#include "cp_device.hpp"
#include "cp_tune.hpp"

namespace cp {

enum BwdRole { kDQ = 0, kDK = 1, kDV = 2, kIdle = 3 };

// Rows covered by the normalised backward's restart pre-pass (16-bit I/O,
// from the final states; see RESTART in bwd_sweep).
#ifndef CP_RESTART_ROWS
#define CP_RESTART_ROWS 512
#endif
constexpr int kRestartRows = CP_RESTART_ROWS;

// Entry (e, m) of an fp32 [Ea][Ma] state; zero in the padding of a narrower
// head (e >= Ea or m >= Ma).
__device__ __forceinline__ float state_at(const float *s, int e, int m, int Ea, int Ma) {
    return e < Ea && m < Ma ? s[e * Ma + m] : 0.f;
}

// The state carries of a backward over sequence segments, for one slice:
// per segment s, dS[s] = sum over its rows of k v^T and dR[s] = sum of q dO^T
// (E x M floats, row e and column m, at a stride of WS floats), written by
// the segment-increment pass (dS for all but the last segment, dR for all but
// the first).  Segment seg's dQ waves then end at S0 + sum_{s <= seg} dS[s]
// (the last segment at the final state, or at the end of its own pre-pass),
// and its dK, dV waves start from sum_{s > seg} dR[s].  dS == NULL: one
// segment (seg = 0, nseg = 1).
struct SegCarry {
    const float *dS, *dR;
    int seg, nseg, sub;  // sub: increment slots per segment (parts of the increment pass)
};

// The slice's three outputs (dQ, dK: E columns; dV: M columns), for the copy
// waves that store the workgroup's staged output rows (OUTLDS in bwd_sweep).
template <typename T> struct Outs {
    T *dq, *dk, *dv;
};

// A k-contraction into NB accumulators that share one operand: acc(x) is the
// x-th accumulator; fs(i) the shared operand (read once), fo(x, i) the x-th
// own operand.  SHARED_A puts the shared operand on the A side.
template <typename T, int NB, bool SHARED_A, typename FACC, typename FS, typename FO>
__device__ __forceinline__ void dotk_shared(FACC acc, int b0, int b1, FS fs, FO fo) {
    using O = Ops<T>;
    int i = b0;
#pragma unroll
    for (; i + 1 < b1; i += 2) {
        const auto s0 = fs(i), s1 = fs(i + 1);
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            if constexpr (SHARED_A) O::mma2(acc(x), s0, s1, fo(x, i), fo(x, i + 1));
            else O::mma2(acc(x), fo(x, i), fo(x, i + 1), s0, s1);
        }
    }
    if (i < b1) {
        const auto s0 = fs(i);
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            if constexpr (SHARED_A) O::mma1(acc(x), s0, fo(x, i));
            else O::mma1(acc(x), fo(x, i), s0);
        }
    }
}

// The whole sweep of one wave role.  Every role runs the same staging and
// barriers; only the math differs, so each wave's loop is straight-line code.
// The wave owns the NB column blocks b + G x (x = 0 .. NB-1) of its output,
// for the row blocks of each chunk that row group RGI of RG owns
// (owns_block): the RG workgroups of a (slice, column group) split the rows,
// each writing whole rows of its outputs, and all of them carry the states
// over every row.  The chunk's operand tiles and causal tiles are read and
// formed once for all of the wave's column blocks.
template <typename T, int E, int M, int C, int G, int NB, int IDLE, int RG, int RGI, int NPF, bool NORM, bool FMAP,
          int ROLE>
__device__ __forceinline__ void bwd_sweep(const T *q_, const T *k_, const T *v_, const T *g_, const float *s0,
                                          const float *st, NormIn<T> nin, SegCarry sc, Outs<T> outs, T *out_,
                                          float *ds0, float *dz0, int L, int b, lds_t<T> *lds, int Ea, int Ma) {
    using O = Ops<T>;
    using F = typename O::frag;
    using EE = EOps<T, E>;  // contraction over e
    using EM = EOps<T, M>;  // contraction over m
    constexpr int EB = E / 16, MB = M / 16, CB = C / 16;
    constexpr int NT = 64 * bwd_waves<E, M, G, NB, IDLE>();
    using SE = Stage<T, NT, C, E>;
    using SM = Stage<T, NT, C, M>;
    constexpr int RE = SE::RS, RM = SM::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;  // Q, K, V, dO
    constexpr bool PHI = NORM && FMAP;             // phi applied to Q and K on their way into LDS
    // NORM: two buffers of the chunk's dd values follow the row buffers
    float *const ddbuf = reinterpret_cast<float *>(lds + 2 * BUF);
    const int g = lane_g(), r = lane_r();
    const int n = (L + C - 1) / C;
    const Diag diag;
    auto bk = [&](int x) { return b + G * x; };  // the wave's column blocks
    constexpr auto own = [](int I) { return owns_block<C / 16, RG>(RGI, I); };  // the row blocks it writes

    // carried state (fp32 accumulator tiles), per column block bk(x)
    //   dQ: W[x][mt] = S^T[ecol_M(mt) + estride_M g + t][16 bk(x) + r]
    //   dK: W[x][mt] = R^T[ecol_M(mt) + estride_M g + t][16 bk(x) + r]
    //   dV: X[x][et] = R[ecol_E(et) + estride_E g + t][16 bk(x) + r]
    // EXACT_PREFIX (normalised form, fp32 I/O): there dq peaks at the first
    // rows, where the state recovered backwards from the final one is small
    // next to it, so plain fp32 would leave there the rounding error of every
    // later chunk (of the backward and of the forward that produced the final
    // state).  Instead the dQ waves build the final state in their own
    // pre-pass as a compensated sum (W + Wlo) of chunk increments computed
    // exactly as the reverse sweep computes them, and subtract those same
    // increments, compensated, on the way back: the recovered states are then
    // the forward prefix sums up to the increments' own rounding.  bf16 I/O
    // rounds far coarser and keeps the plain update and its registers.
    constexpr bool EXACT_PREFIX = NORM && std::is_same<T, float>::value;
    constexpr bool COMP = EXACT_PREFIX && ROLE == kDQ;
    constexpr int NW = ROLE == kDQ || ROLE == kDK ? NB : 1, NX = ROLE == kDV ? NB : 1;
    f32x4 W[NW][MB], X[NX][EB], Wlo[COMP ? NB : 1][COMP ? MB : 1];
#pragma unroll
    for (int x = 0; x < NW; ++x)
#pragma unroll
        for (int m = 0; m < MB; ++m) W[x][m] = zero4();
#pragma unroll
    for (int x = 0; x < (COMP ? NB : 1); ++x)
#pragma unroll
        for (int m = 0; m < (COMP ? MB : 1); ++m) Wlo[x][m] = zero4();
#pragma unroll
    for (int x = 0; x < NX; ++x)
#pragma unroll
        for (int e = 0; e < EB; ++e) X[x][e] = zero4();
    // NORM: dQ carries zb[x][t] = z[16 bk(x) + 4g + t], from z_{L-1} down to
    // z_{c-1} by subtracting each chunk's column sums of phi(K) (compensated,
    // zlo, with EXACT_PREFIX); dK carries zb[x][t] = r[16 bk(x) + 4g + t]
    // (suffix of dd_i phi(q_i)); same in every lane r
    f32x4 zb[NB], zlo[NB];
#pragma unroll
    for (int x = 0; x < NB; ++x) zb[x] = zlo[x] = zero4();
    // column sums of phi(K_c)[:, bk(x)] from the transposed K fragments
    auto chunk_zsum = [&](const F (&kt)[NB][C / 16], f32x4 (&cs)[NB]) {
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            cs[x] = zero4();
            dotk<T>(cs[x], 0, CB, [&](int J) { return kt[x][J]; }, [&](int) { return O::ones(); });
        }
    };

    // Where the dQ waves get the states before each chunk.  From the final
    // states (state_final with, for the normalised form, z_final): by
    // subtracting the chunks' increments.  Otherwise: from a forward pre-pass
    // over the whole sequence, starting at S0 (z0).
    //
    // RESTART (normalised form, 16-bit I/O, from the final states): the
    // subtraction leaves in every recovered state an absolute error of the
    // order of the final state's rounding (its own and the forward's), and
    // the first rows, whose denominators are smallest and whose dq is a near
    // cancellation of S_i dn_i against dd_i z_i, magnify it most.  So the
    // pre-pass also runs over the first npre chunks (about kRestartRows rows):
    // the dQ waves park those exact-so-far states (S, z after chunk npre - 1)
    // in LDS and take them back when the reverse sweep reaches that chunk,
    // so the early rows never see the final state's rounding.
    constexpr bool RESTART = NORM && !EXACT_PREFIX;
    constexpr int WS = E * M + E;
    const bool last_seg = sc.seg == sc.nseg - 1;
    // the final states given (and used: not with fp32 I/O in the normalised form)
    const bool use_final = st && (!NORM || nin.zf) && !EXACT_PREFIX;
    const bool from_final = (!last_seg || use_final) && !EXACT_PREFIX;
    // Over sequence segments (sc.dS != NULL) the starting states are sums of
    // whole E x M tiles (and E-vectors of z, r): all threads add them up with
    // 16-byte loads into an fp32 tile in LDS (the ring buffers, not in use
    // then), from which each wave takes its fragments.  The dQ waves start at
    // S, z after the segment: with the final states, st, zf minus the later
    // segments' increments (the increment pass then covers segments 1 ..
    // nseg-1, and s0, z0 are not needed); without them, s0, z0 plus the
    // increments up to and including this segment's (segments 0 .. nseg-2),
    // the last segment starting before itself for a pre-pass over it.  The
    // dK and dV waves start at R, r after the segment (the later segments'
    // increments).
    const bool staged = sc.dS != nullptr;
    constexpr int TS = M + 4;  // fp32 row stride of the tile (rows 16 bytes apart mod 128)
    static_assert(E * TS * 4 + E * 4 <= 2 * BUF * (int)sizeof(lds_t<T>), "the carry tile fits the ring buffers");
    auto stage_carries = [&](bool end) {
        float *tile = reinterpret_cast<float *>(lds), *zvec = tile + E * TS;
        const int tid = (int)threadIdx.x;
        const int upto = end ? sc.seg + 1 : sc.seg;
        for (int p = tid; p < E * M / 4 + (NORM ? E / 4 : 0); p += NT) {
            const bool zpart = p >= E * M / 4;  // the z vector's pieces follow the tile's
            const int e = zpart ? 4 * (p - E * M / 4) : p / (M / 4), m = zpart ? 0 : p % (M / 4) * 4;
            const int widx = zpart ? E * M + e : e * M + m;  // in an increment
            const float *st_ = zpart ? nin.zf : st, *s0_ = zpart ? nin.z0 : s0;
            const int64_t off = zpart ? e : (int64_t)e * Ma + m;
            const bool in = e < Ea && m < Ma;
            f32x4 a = zero4();
            // the slots hold cumulative sums (cp_seg_scan_kernel): one read each
            if (use_final) {  // (only ever with end) minus the later segments' sum
                if (in) a = *reinterpret_cast<const f32x4 *>(st_ + off);
                const int s1 = (sc.seg + 1) * sc.sub;
                if (s1 < sc.nseg * sc.sub) a -= *reinterpret_cast<const f32x4 *>(sc.dS + s1 * WS + widx);
            } else {  // plus the earlier segments' sum
                if (s0_ && in) a = *reinterpret_cast<const f32x4 *>(s0_ + off);
                if (upto > 0) a += *reinterpret_cast<const f32x4 *>(sc.dS + (upto * sc.sub - 1) * WS + widx);
            }
            *reinterpret_cast<f32x4 *>(zpart ? zvec + e : tile + e * TS + m) = a;
        }
        __syncthreads();
        if constexpr (ROLE == kDQ) {
#pragma unroll
            for (int x = 0; x < NB; ++x) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        W[x][m][t] = tile[(16 * bk(x) + r) * TS + EM::ecol(m) + EM::estride * g + t];
                if constexpr (NORM) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) zb[x][t] = zvec[16 * bk(x) + 4 * g + t];
                }
            }
        }
        __syncthreads();
        if (!last_seg) {  // (staged once per sweep: with the start or with the end state)
            for (int p = tid; p < E * M / 4 + (NORM ? E / 4 : 0); p += NT) {
                const bool zpart = p >= E * M / 4;
                const int e = zpart ? 4 * (p - E * M / 4) : p / (M / 4), m = zpart ? 0 : p % (M / 4) * 4;
                const int widx = zpart ? E * M + e : e * M + m;
                const f32x4 a = *reinterpret_cast<const f32x4 *>(sc.dR + (sc.seg + 1) * sc.sub * WS + widx);
                *reinterpret_cast<f32x4 *>(zpart ? zvec + e : tile + e * TS + m) = a;
            }
            __syncthreads();
            if constexpr (ROLE == kDK) {
#pragma unroll
                for (int x = 0; x < NB; ++x) {
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            W[x][m][t] = tile[(16 * bk(x) + r) * TS + EM::ecol(m) + EM::estride * g + t];
                    if constexpr (NORM) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) zb[x][t] = zvec[16 * bk(x) + 4 * g + t];
                    }
                }
            } else if constexpr (ROLE == kDV) {
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int e = 0; e < EB; ++e)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            X[x][e][t] = tile[(EE::ecol(e) + EE::estride * g + t) * TS + 16 * bk(x) + r];
            }
            __syncthreads();
        }
    };
    // the last segment without final states: a pre-pass over the segment
    // from the staged states before it
    const bool stage_early = staged && !from_final;
    if (stage_early) stage_carries(false);
    // pre-pass chunks: the whole sequence (segment) without final states; the
    // restart rows at the start of the sequence (RESTART)
    constexpr int kPre = kRestartRows / C > 1 ? kRestartRows / C : 1;
    const int npre = from_final ? (RESTART && sc.seg == 0 ? (n < kPre ? n : kPre) : 0) : n;
    // the wave's parking slots: f32x4 per lane, MB state tiles then z, per block
    f32x4 *const park = RESTART && ROLE == kDQ ? reinterpret_cast<f32x4 *>(ddbuf + 2 * C) +
                                                     (int)(threadIdx.x >> 6) * NB * (MB + 1) * 64  // dQ waves come first
                                               : nullptr;
    if (npre > 0) {
        // forward pre-pass over chunks [0, npre): S^T[:, b] = S0^T[:, b] + the
        // chunks' V^T K[:, b] (NORM: and z = z_{-1} + their column sums)
        if constexpr (ROLE == kDQ) {
            if (s0 && !stage_early) {
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            W[x][m][t] = state_at(s0, 16 * bk(x) + r, EM::ecol(m) + EM::estride * g + t, Ea, Ma);
            }
            if constexpr (NORM) {
                if (nin.z0 && !stage_early) {
#pragma unroll
                    for (int x = 0; x < NB; ++x)
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int f = 16 * bk(x) + 4 * g + t;
                            zb[x][t] = f < Ea ? nin.z0[f] : 0.f;
                        }
                }
            }
        }
        SE sk;
        SM sv;
        sk.load(Rows<T>(k_, Ea, 0, L, C), 0, Ea);
        sv.load(Rows<T>(v_, Ma, 0, L, C), 0, Ma);
        for (int c = 0; c < npre; ++c) {
            lds_t<T> *Ks = lds + (c & 1) * BUF, *Vs = Ks + C * RE;
            sk.template store<PHI>(Ks, c * C, L, Ea);
            sv.store(Vs);
            __syncthreads();
            sk.load(Rows<T>(k_, Ea, (c + 1) * C, L, C), 0, Ea);
            sv.load(Rows<T>(v_, Ma, (c + 1) * C, L, C), 0, Ma);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ROLE == kDQ) {
                F kt[NB][CB];
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int J = 0; J < CB; ++J) kt[x][J] = O::tr_frag(Ks, RE, J, bk(x));
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if constexpr (COMP) {  // the reverse sweep's increment, negated (exactly)
                        f32x4 dw[NB];
#pragma unroll
                        for (int x = 0; x < NB; ++x) dw[x] = zero4();
                        dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return dw[x]; }, 0, CB,
                                                 [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                                                 [&](int x, int J) { return kt[x][J]; });
#pragma unroll
                        for (int x = 0; x < NB; ++x) two_sum_acc(W[x][m], Wlo[x][m], dw[x]);
                    } else {
                        dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return W[x][m]; }, 0, CB,
                                                 [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                                                 [&](int x, int J) { return kt[x][J]; });
                    }
                }
                if constexpr (NORM) {
                    f32x4 cs[NB];
                    chunk_zsum(kt, cs);
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        if constexpr (COMP) two_sum_acc(zb[x], zlo[x], cs[x]);
                        else zb[x] += cs[x];
                    }
                }
            }
        }
        __syncthreads();  // the main sweep reuses the buffers
    }
    if (from_final) {
        if constexpr (RESTART && ROLE == kDQ) {
            if (npre > 0) {
#pragma unroll
                for (int x = 0; x < NB; ++x) {
#pragma unroll
                    for (int m = 0; m < MB; ++m) park[(x * (MB + 1) + m) * 64 + lane_id()] = W[x][m];
                    park[(x * (MB + 1) + MB) * 64 + lane_id()] = zb[x];
                }
            }
        }
        if (staged) {
            stage_carries(true);
        } else if constexpr (ROLE == kDQ) {
#pragma unroll
            for (int x = 0; x < NB; ++x) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        W[x][m][t] = state_at(st, 16 * bk(x) + r, EM::ecol(m) + EM::estride * g + t, Ea, Ma);
                if constexpr (NORM) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int f = 16 * bk(x) + 4 * g + t;
                        zb[x][t] = f < Ea ? nin.zf[f] : 0.f;
                    }
                }
            }
        }
    }

    constexpr int OW = ROLE == kDV ? M : E;

    // OUTLDS (16-bit I/O, two adjacent column blocks per wave, one column
    // group, copy-only waves): the role waves write each chunk's output
    // tiles into an LDS buffer (double buffered, after the ring and the
    // normalised form's buffers) instead of storing them; after the next
    // barrier the copy-only waves store that chunk's dQ, dK and dV rows as
    // whole rows of 16-byte pieces (non-temporal).  A row's 128 bytes then
    // come from one wave and one instruction instead of 32- or 64-byte pieces
    // from several waves.
    constexpr bool OUTLDS = sizeof(T) == 2 && NB == 2 && G == 1 && IDLE > 0;
    constexpr int OWM = E > M ? E : M;              // widest output row (elements)
    constexpr int RSO = OWM + 8;                    // LDS row stride of the staged rows
    constexpr int NOWN = owned_count<CB, RG>(RGI);  // row blocks this row group owns per chunk
    constexpr int OROWS = 16 * NOWN;                // its output rows per chunk and output
    constexpr int EG_ = (EB + G * NB - 1) / (G * NB);  // dQ waves (their parking slots precede)
    lds_t<T> *const outbuf = reinterpret_cast<lds_t<T> *>(ddbuf + 2 * C + (NORM && sizeof(T) == 2 ? EG_ * NB * (MB + 1) * 64 * 4 : 0));
    // the copy-only waves store chunk step ps's rows
    auto flush_rows = [&](int ps) {
        if constexpr (OUTLDS && ROLE == kIdle) {
            constexpr int PPRO = OWM * 2 / 16;  // 16-byte pieces per staged row
            constexpr int NPIECE = 3 * OROWS * PPRO, NI = 64 * IDLE;
            const int il = ((int)(threadIdx.x >> 6) - (NT / 64 - IDLE)) * 64 + lane_id();
            const int prow0 = (n - 1 - ps) * C;
            const lds_t<T> *ob = outbuf + (ps & 1) * 3 * OROWS * RSO;
#pragma unroll
            for (int i = 0; i < (NPIECE + NI - 1) / NI; ++i) {
                const int p = il + i * NI;
                if (NPIECE % NI != 0 && p >= NPIECE) break;
                const int out = p / (OROWS * PPRO), row = p % (OROWS * PPRO) / PPRO, cp = p % PPRO;
                const int wt = out < 2 ? E : M, wa = out < 2 ? Ea : Ma;
                T *base = out == 0 ? outs.dq : out == 1 ? outs.dk : outs.dv;
                const int j = owned_block<CB, RG>(RGI, row / 16);
                const Rows<T> X(base, wa, prow0, L, C);
                const i32x4 v = *reinterpret_cast<const i32x4 *>(ob + (out * OROWS + row) * RSO + cp * 8);
                const int off = cp * 8 < wt && cp * 8 < wa ? ((16 * j + row % 16) * wa + cp * 8) * (int)sizeof(T) : kVoid;
                __builtin_amdgcn_raw_buffer_store_b128(v, X.rsrc, off, 0, 2);
            }
        }
    };

    // Ring of NPF register stages (NPF-1 chunks in flight while one is
    // computed); the step loop is padded to a multiple of NPF with chunks
    // before the start of the sequence, which load as zero and store nothing.
    // NORM: also the forward's output rows and the denominators of the rows
    // of each thread's dO pieces (zero past the sequence).
    struct Stages {
        SE q, k;
        SM v, g;
        SM o;
        float den[NORM ? SM::NP : 1];
        __device__ __forceinline__ void load(const T *q_, const T *k_, const T *v_, const T *g_, NormIn<T> nin,
                                             int row0, int L, int Ea, int Ma) {
            q.load(Rows<T>(q_, Ea, row0, L, C), 0, Ea);
            k.load(Rows<T>(k_, Ea, row0, L, C), 0, Ea);
            v.load(Rows<T>(v_, Ma, row0, L, C), 0, Ma);
            g.load(Rows<T>(g_, Ma, row0, L, C), 0, Ma);
            if constexpr (NORM) {
                o.load(Rows<T>(nin.o, Ma, row0, L, C), 0, Ma);
                const Rows<float> rd(nin.den, 1, row0, L, C);
#pragma unroll
                for (int i = 0; i < SM::NP; ++i) {
                    const int p = (int)threadIdx.x + i * NT;
                    den[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                           rd.rsrc, p < SM::P ? 4 * (p / SM::PPR) : kVoid, 0, 0));
                }
            }
        }
    };
    Stages stg[NPF];
#pragma unroll
    for (int s = 0; s < NPF - 1; ++s) {
        stg[s].load(q_, k_, v_, g_, nin, (n - 1 - s) * C, L, Ea, Ma);
        __builtin_amdgcn_sched_barrier(0);  // stages complete in order
    }
    const int nsteps = (n + NPF - 1) / NPF * NPF;
    for (int sb = 0; sb < nsteps; sb += NPF) {
#pragma unroll
        for (int s = 0; s < NPF; ++s) {
            const int step = sb + s;
            const int row0 = (n - 1 - step) * C;
            lds_t<T> *Qs = lds + (step & 1) * BUF, *Ks = Qs + C * RE, *Vs = Ks + C * RE, *Gs = Vs + C * RM;
            float *dds = ddbuf + (step & 1) * C;  // NORM: dd_i of row row0 + i
            stg[s].q.template store<PHI>(Qs, row0, L, Ea);
            stg[s].k.template store<PHI>(Ks, row0, L, Ea);
            stg[s].v.store(Vs);
            if constexpr (NORM) store_dn<T>(stg[s].g, stg[s].o, stg[s].den, Gs, dds);
            else stg[s].g.store(Gs);
            __syncthreads();
            stg[(s + NPF - 1) % NPF].load(q_, k_, v_, g_, nin, row0 - (NPF - 1) * C, L, Ea, Ma);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (OUTLDS && ROLE == kIdle) {
                if (step > 0) flush_rows(step - 1);
            }

            f32x4 pend[NB][CB];  // this chunk's output tiles (rows 16 I + r) per column block
            if constexpr (ROLE == kDQ) {
                if constexpr (RESTART) {  // S_c, z_c of the pre-pass (see RESTART)
                    if (from_final && npre > 0 && row0 == (npre - 1) * C) {
#pragma unroll
                        for (int x = 0; x < NB; ++x) {
#pragma unroll
                            for (int m = 0; m < MB; ++m) W[x][m] = park[(x * (MB + 1) + m) * 64 + lane_id()];
                            zb[x] = park[(x * (MB + 1) + MB) * 64 + lane_id()];
                        }
                    }
                }
                // W = S_{c-1}^T = S_c^T - V_c^T K_c[:, b]
                F kt[NB][CB];  // K_J[:, b] transposed: lane (g, r) <- K[16 J + 4g + t][16 b + r]
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int J = 0; J < CB; ++J) kt[x][J] = O::tr_frag(Ks, RE, J, bk(x));
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if constexpr (COMP) {  // compensated, see EXACT_PREFIX
                        f32x4 dw[NB];
#pragma unroll
                        for (int x = 0; x < NB; ++x) dw[x] = zero4();
                        dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return dw[x]; }, 0, CB,
                                                 [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                                                 [&](int x, int J) { return O::neg(kt[x][J]); });
#pragma unroll
                        for (int x = 0; x < NB; ++x) two_sum_acc(W[x][m], Wlo[x][m], dw[x]);
                    } else {
                        dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return W[x][m]; }, 0, CB,
                                                 [&](int J) { return EM::tr_e(Vs, RM, J, m); },
                                                 [&](int x, int J) { return O::neg(kt[x][J]); });
                    }
                }
                if constexpr (NORM) {  // z_{c-1} = z_c - the chunk's column sums
                    f32x4 cs[NB];
                    chunk_zsum(kt, cs);
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        if constexpr (COMP) two_sum_acc(zb[x], zlo[x], -cs[x]);
                        else zb[x] -= cs[x];
                    }
                }
                typename EM::rf wa[NB][EM::STEPS], vf[CB][EM::STEPS];
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) wa[x][k] = EM::state(W[x], k);
#pragma unroll
                for (int J = 0; J < CB; ++J)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) vf[J][k] = EM::load(Vs, RM, J, k);
#pragma unroll
                for (int I = 0; I < CB; ++I) {
                    if (!own(I)) continue;
                    typename EM::rf gf[EM::STEPS];
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) gf[k] = EM::load(Gs, RM, I, k);
                    // NORM: the ones column of V' = [V 1] against dd: P'^T(j, i) = P^T(j, i) + dd_i,
                    // and the state's z column: dq_i += dd_i z_{c-1}
                    const float ddi = NORM ? dds[16 * I + r] : 0.f;
                    // P^T(J, I) = V_J dO_I^T, causal on the diagonal (shared by the blocks)
                    F pt[CB];
#pragma unroll
                    for (int J = 0; J <= I; ++J) {
                        f32x4 p = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(p, vf[J][k], gf[k]);
                        if constexpr (NORM) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) p[t] += ddi;
                        }
                        if (J == I) p = diag.keys(p);
                        pt[J] = O::cvt(p);
                    }
                    // dQ^T = S dO_I^T + K^T P^T
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        f32x4 d = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(d, wa[x][k], gf[k]);
                        if constexpr (NORM) {
#pragma unroll
                            for (int t = 0; t < 4; ++t) d[t] += (zb[x][t] + zlo[x][t]) * ddi;
                        }
                        dotk<T>(d, 0, I + 1, [&](int J) { return kt[x][J]; }, [&](int J) { return pt[J]; });
                        if constexpr (PHI) {  // through phi: phi'(x) = min(phi(x), 1)
                            const F ph = lds_nat<T>(Qs, RE, I, bk(x));
#pragma unroll
                            for (int t = 0; t < 4; ++t) d[t] *= fminf(frag_val<T>(ph, t), 1.f);
                        }
                        pend[x][I] = d;
                    }
                }
            } else if constexpr (ROLE == kDK) {
                F qt[NB][CB];  // Q_I[:, b] transposed
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int I = 0; I < CB; ++I) qt[x][I] = O::tr_frag(Qs, RE, I, bk(x));
                typename EM::rf wa[NB][EM::STEPS], gf[CB][EM::STEPS];
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) wa[x][k] = EM::state(W[x], k);  // R_{c+1}
#pragma unroll
                for (int I = 0; I < CB; ++I)
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) gf[I][k] = EM::load(Gs, RM, I, k);
#pragma unroll
                for (int J = 0; J < CB; ++J) {
                    if (!own(J)) continue;
                    typename EM::rf vf[EM::STEPS];
#pragma unroll
                    for (int k = 0; k < EM::STEPS; ++k) vf[k] = EM::load(Vs, RM, J, k);
                    // P(I, J) = dO_I V_J^T for I >= J (shared by the blocks)
                    F pf[CB];
#pragma unroll
                    for (int I = J; I < CB; ++I) {
                        f32x4 p = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(p, gf[I][k], vf[k]);
                        if constexpr (NORM) {  // P'(i, j) = P(i, j) + dd_i
#pragma unroll
                            for (int t = 0; t < 4; ++t) p[t] += dds[16 * I + 4 * g + t];
                        }
                        if (I == J) p = diag.query(p);
                        pf[I] = O::cvt(p);
                    }
                    // dK^T = R_{c+1} V_J^T + Q^T P
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        f32x4 d = zero4();
#pragma unroll
                        for (int k = 0; k < EM::STEPS; ++k) EM::mma(d, wa[x][k], vf[k]);
                        if constexpr (NORM) {  // the ones column of V': dk_j += r_{c+1}
#pragma unroll
                            for (int t = 0; t < 4; ++t) d[t] += zb[x][t];
                        }
                        dotk<T>(d, J, CB, [&](int I) { return qt[x][I]; }, [&](int I) { return pf[I]; });
                        if constexpr (PHI) {
                            const F ph = lds_nat<T>(Ks, RE, J, bk(x));
#pragma unroll
                            for (int t = 0; t < 4; ++t) d[t] *= fminf(frag_val<T>(ph, t), 1.f);
                        }
                        pend[x][J] = d;
                    }
                }
                // R^T += dO_c^T Q_c[:, b]
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return W[x][m]; }, 0, CB,
                                             [&](int I) { return EM::tr_e(Gs, RM, I, m); },
                                             [&](int x, int I) { return qt[x][I]; });
                if constexpr (NORM) {  // r += sum_i dd_i phi(q_i)[b], dd as a hi + lo pair of operands
                    F dh[CB], dl[CB];
#pragma unroll
                    for (int I = 0; I < CB; ++I) {
                        f32x4 x;
#pragma unroll
                        for (int t = 0; t < 4; ++t) x[t] = dds[16 * I + 4 * g + t];
                        O::split(x, dh[I], dl[I]);
                    }
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        dotk<T>(zb[x], 0, CB, [&](int I) { return qt[x][I]; }, [&](int I) { return dh[I]; });
                        if constexpr (sizeof(T) == 2)
                            dotk<T>(zb[x], 0, CB, [&](int I) { return qt[x][I]; }, [&](int I) { return dl[I]; });
                    }
                }
            } else if constexpr (ROLE == kDV) {
                F gt[NB][CB];  // dO_I[:, b] transposed
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int I = 0; I < CB; ++I) gt[x][I] = O::tr_frag(Gs, RM, I, bk(x));
                typename EE::rf xa[NB][EE::STEPS], qf[CB][EE::STEPS];
#pragma unroll
                for (int x = 0; x < NB; ++x)
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) xa[x][k] = EE::state(X[x], k);  // R_{c+1}^T rows
#pragma unroll
                for (int I = 0; I < CB; ++I)
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) qf[I][k] = EE::load(Qs, RE, I, k);
#pragma unroll
                for (int J = 0; J < CB; ++J) {
                    if (!own(J)) continue;
                    typename EE::rf kf[EE::STEPS];
#pragma unroll
                    for (int k = 0; k < EE::STEPS; ++k) kf[k] = EE::load(Ks, RE, J, k);
                    // A(I, J) = Q_I K_J^T for I >= J (shared by the blocks)
                    F af[CB];
#pragma unroll
                    for (int I = J; I < CB; ++I) {
                        f32x4 a = zero4();
#pragma unroll
                        for (int k = 0; k < EE::STEPS; ++k) EE::mma(a, qf[I][k], kf[k]);
                        if (I == J) a = diag.query(a);
                        af[I] = O::cvt(a);
                    }
                    // dV^T = R^T K_J^T + dO^T A
#pragma unroll
                    for (int x = 0; x < NB; ++x) {
                        f32x4 d = zero4();
#pragma unroll
                        for (int k = 0; k < EE::STEPS; ++k) EE::mma(d, xa[x][k], kf[k]);
                        dotk<T>(d, J, CB, [&](int I) { return gt[x][I]; }, [&](int I) { return af[I]; });
                        pend[x][J] = d;
                    }
                }
                // R += Q_c^T dO_c[:, b]
#pragma unroll
                for (int e = 0; e < EB; ++e)
                    dotk_shared<T, NB, true>([&](int x) -> f32x4 & { return X[x][e]; }, 0, CB,
                                             [&](int I) { return EE::tr_e(Qs, RE, I, e); },
                                             [&](int x, int I) { return gt[x][I]; });
            }
            // Stores go after this step's prefetch: memory operations complete
            // in issue order, so the rows waited for at a later step were
            // issued before these stores and never wait for them.
            if constexpr (ROLE != kIdle) {
                const int OWa = ROLE == kDV ? Ma : Ea;
                const Rows<T> rp(out_, OWa, row0, L, C);
                // two-block waves: a row block's two 16-bit tiles as 16-byte
                // pieces (64 contiguous bytes per row with adjacent blocks)
                if constexpr (OUTLDS) {
                    lds_t<T> *ob = outbuf + ((step & 1) * 3 + ROLE) * OROWS * RSO;
                    typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        if (own(j)) {
                            const int row = 16 * owned_index<CB, RG>(RGI, j) + r;
#pragma unroll
                            for (int x = 0; x < NB; ++x)
                                *reinterpret_cast<i32x2 *>(ob + row * RSO + 16 * bk(x) + 4 * g) =
                                    __builtin_bit_cast(i32x2, O::cvt(pend[x][j]));
                        }
                } else if constexpr (sizeof(T) == 2 && NB == 2) {
#pragma unroll
                    for (int j = 0; j < CB; ++j)
                        if (own(j)) st_out_pair<T>(rp, j, bk(0), pend[0][j], j, bk(1), pend[1][j], OWa);
                } else {
#pragma unroll
                    for (int x = 0; x < NB; ++x)
#pragma unroll
                        for (int j = 0; j < CB; ++j)
                            if (own(j)) st_out<T>(rp, j, bk(x), pend[x][j], OWa);
                }
            }
        }
    }
    if constexpr (OUTLDS) {  // the last step's rows
        __syncthreads();
        flush_rows(nsteps - 1);
    }
    // the gradient of the initial z: r_0, held by the dK waves
    if constexpr (NORM && ROLE == kDK && RGI == 0) {
        if (dz0 && r == 0) {
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (16 * bk(x) + 4 * g + t < Ea) dz0[16 * bk(x) + 4 * g + t] = zb[x][t];
        }
    }
    // the gradient of the initial state: R_0 = sum_i q_i dO_i^T, held by the
    // dV waves (column blocks of M) at the end of the reverse sweep
    if constexpr (ROLE == kDV && RGI == 0) {
        if (ds0) {
#pragma unroll
            for (int x = 0; x < NB; ++x)
#pragma unroll
                for (int e = 0; e < EB; ++e)
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int row = EE::ecol(e) + EE::estride * g + t, col = 16 * bk(x) + r;
                        if (row < Ea && col < Ma) ds0[row * Ma + col] = X[x][e][t];
                    }
        }
    }
}

// The wave's role sweep for row group RGI.
template <typename T, int E, int M, int C, int G, int NB, int IDLE, int RG, int RGI, int NPF, bool NORM, bool FMAP>
__device__ __forceinline__ void bwd_role(int role, int b, const T *q_, const T *k_, const T *v_, const T *g_,
                                         const float *s0, const float *st, NormIn<T> nin, SegCarry sc, T *dq_, T *dk_, T *dv_,
                                         float *ds0, float *dz0, int L, lds_t<T> *lds, int Ea, int Ma) {
    constexpr int EB = E / 16, MB = M / 16;
    const Outs<T> outs{dq_, dk_, dv_};
    if (role == kDQ && b < EB)
        bwd_sweep<T, E, M, C, G, NB, IDLE, RG, RGI, NPF, NORM, FMAP, kDQ>(q_, k_, v_, g_, s0, st, nin, sc, outs, dq_, nullptr,
                                                                          nullptr, L, b, lds, Ea, Ma);
    else if (role == kDK && b < EB)
        bwd_sweep<T, E, M, C, G, NB, IDLE, RG, RGI, NPF, NORM, FMAP, kDK>(q_, k_, v_, g_, s0, st, nin, sc, outs, dk_, nullptr,
                                                                          dz0, L, b, lds, Ea, Ma);
    else if (role == kDV && b < MB)
        bwd_sweep<T, E, M, C, G, NB, IDLE, RG, RGI, NPF, NORM, FMAP, kDV>(q_, k_, v_, g_, s0, st, nin, sc, outs, dv_, ds0,
                                                                          nullptr, L, b, lds, Ea, Ma);
    else
        bwd_sweep<T, E, M, C, G, NB, IDLE, RG, RGI, NPF, NORM, FMAP, kIdle>(q_, k_, v_, g_, s0, st, nin, sc, outs, nullptr,
                                                                            nullptr, nullptr, L, 0, lds, Ea, Ma);
}

// NORM (backward of the normalised form, see the launcher): Q, K are the raw
// inputs (phi applied on load when FMAP), Gr is dO, O and den the forward's
// output and denominators, z_final the normaliser after the last row
// (optional: without it, or with fp32 I/O, the dQ waves sum it in their
// pre-pass from z_in), dz_in the gradient of the initial z.
template <typename T, int E, int M, int C, int G, int NB, int IDLE, int RG, int NPF, bool NORM, bool FMAP>
__global__ __launch_bounds__((64 * bwd_waves<E, M, G, NB, IDLE>())) void cp_bwd_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, const T *__restrict__ Gr,
    const float *__restrict__ state_in, const float *__restrict__ state_final, const T *__restrict__ O,
    const float *__restrict__ den, const float *__restrict__ z_in, const float *__restrict__ z_final,
    T *__restrict__ dQ, T *__restrict__ dK, T *__restrict__ dV, float *__restrict__ dstate_in,
    float *__restrict__ dz_in, const float *__restrict__ ws, int L, int NS, int seg_len, int sub, int Ea, int Ma) {
    constexpr int EB = E / 16, MB = M / 16;
    // with several blocks per wave every wave's blocks all exist
    static_assert(NB == 1 || (EB % (G * NB) == 0 && MB % (G * NB) == 0), "blocks per wave");
    constexpr int EG = (EB + G * NB - 1) / (G * NB), MG = (MB + G * NB - 1) / (G * NB);
    constexpr int NT = 64 * bwd_waves<E, M, G, NB, IDLE>();
    static_assert(NT <= 1024, "at most 16 waves per workgroup");
    constexpr int RE = Stage<T, NT, C, E>::RS, RM = Stage<T, NT, C, M>::RS;
    constexpr int BUF = 2 * C * RE + 2 * C * RM;
    // NORM: two dd buffers of C floats; with 16-bit I/O also the dQ waves'
    // parking slots for the restart states
    constexpr int PARK = NORM && sizeof(T) == 2 ? EG * NB * (MB + 1) * 64 * 4 : 0;
    constexpr int DDE = NORM ? (2 * C + PARK) * 4 / (int)sizeof(lds_t<T>) : 0;
    // staged output rows (OUTLDS in bwd_sweep), after the dd buffers
    constexpr bool OUTLDS = sizeof(T) == 2 && NB == 2 && G == 1 && IDLE > 0;
    constexpr int OWM = E > M ? E : M, NOWN0 = owned_count<C / 16, RG>(0), NOWN1 = owned_count<C / 16, RG>(RG - 1);
    constexpr int OUTE = OUTLDS ? (NORM ? 0 : 2 * C * 4 / (int)sizeof(lds_t<T>)) +
                                      2 * 3 * 16 * (NOWN0 > NOWN1 ? NOWN0 : NOWN1) * (OWM + 8)
                                : 0;
    __shared__ __attribute__((aligned(16))) lds_t<T> lds[2 * BUF + DDE + OUTE];

    static_assert(RG >= 1 && RG <= 2 && RG <= C / 16, "row groups");
    const int nseg = (L + seg_len - 1) / seg_len;
    int slice, part;
    map_block(blockIdx.x, NS, G * RG * nseg, slice, part);
    const int grp = part % G, rg = (part / G) % RG, seg = part / (G * RG);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // rows [rb, re) of the slice; the tensors' own head sizes Ea <= E, Ma <= M
    // (the kernel's tile sizes)
    const int rb = seg * seg_len, re = rb + seg_len < L ? rb + seg_len : L;
    const int64_t oe = ((int64_t)slice * L + rb) * Ea, om = ((int64_t)slice * L + rb) * Ma;
    const int64_t os = (int64_t)slice * Ea * Ma;
    const T *q_ = Q + oe, *k_ = K + oe, *v_ = V + om, *g_ = Gr + om;
    const float *s0 = state_in ? state_in + os : nullptr;
    const float *st = state_final ? state_final + os : nullptr;
    NormIn<T> nin{nullptr, nullptr, nullptr, nullptr};
    if constexpr (NORM) {
        nin.o = O + om;
        nin.den = den + (int64_t)slice * L + rb;
        nin.zf = z_final ? z_final + (int64_t)slice * Ea : nullptr;
        nin.z0 = z_in ? z_in + (int64_t)slice * Ea : nullptr;
    }
    // the gradients of the initial states come from the first segment
    float *ds0 = dstate_in && seg == 0 ? dstate_in + os : nullptr;
    float *dz0 = dz_in && seg == 0 ? dz_in + (int64_t)slice * Ea : nullptr;
    constexpr int WS = E * M + E;
    const SegCarry sc{ws ? ws + (int64_t)slice * nseg * sub * WS : nullptr,
                      ws ? ws + ((int64_t)NS + slice) * nseg * sub * WS : nullptr, seg, nseg, sub};
    const int Ls = re - rb;
    // wave w: role, and the first of its NB column blocks (b, b + G, ...)
    const int role = w < EG ? kDQ : w < 2 * EG ? kDK : w < 2 * EG + MG ? kDV : kIdle;
    const int lw = role == kDQ ? w : role == kDK ? w - EG : w - 2 * EG;
    const int b = grp + G * NB * lw;
    if (rg == 0 || RG == 1)
        bwd_role<T, E, M, C, G, NB, IDLE, RG, 0, NPF, NORM, FMAP>(role, b, q_, k_, v_, g_, s0, st, nin, sc, dQ + oe,
                                                                 dK + oe, dV + om, ds0, dz0, Ls, lds, Ea, Ma);
    else
        bwd_role<T, E, M, C, G, NB, IDLE, RG, (RG > 1 ? 1 : 0), NPF, NORM, FMAP>(
            role, b, q_, k_, v_, g_, s0, st, nin, sc, dQ + oe, dK + oe, dV + om, ds0, dz0, Ls, lds, Ea, Ma);
}

}  // namespace cp
