// cp_tune.hpp -- compile-time launch parameters of each kernel instance:
//   FC   forward chunk length (tokens per step of the scan),
//   FG   forward workgroups per (n, h) slice; each owns M/16/FG column blocks
//        of the output, one wave per block,
//   BC   backward chunk length,
//   BG   backward workgroups per (n, h) slice; each owns every BG-th column
//        block of dQ, dK and dV, one wave per block,
//   FRS  forward row sets: waves per output column block, which split the
//        chunk's query row blocks,
//   FRG  forward row groups: workgroups per (slice, column group) that split
//        the chunk's query row blocks, so that every output row is written
//        by one workgroup (whole 128-byte lines stream to HBM at a higher
//        rate than lines whose pieces come from two compute units),
//   FNPF, BNPF  stages of the forward / backward load ring (NPF-1 chunks are
//        in flight while one is computed; BNPF_N for the normalised backward),
//   BNB  backward column blocks per wave (1 or 2): a wave with two blocks
//        reads the chunk's operand tiles and forms its causal tiles once for
//        both,
//   BIDLE  extra backward waves that only help copy, for two-block waves (by
//        default a workgroup of three waves gets a fourth, one per SIMD),
//   BRG  backward row groups: workgroups per (slice, column group) that split
//        the chunk's row blocks (each writes whole rows of dQ, dK and dV);
//        used with two-block waves, whose workgroups then take every column,
// Each value can be overridden when the library is built (-DCP_BF16_FC=32 ...)
// for tuning sweeps.
#pragma once

#ifndef CP_BF16_FC
#define CP_BF16_FC 64
#endif
#ifndef CP_BF16_FG
#define CP_BF16_FG 1
#endif
#ifndef CP_BF16_FRG
#define CP_BF16_FRG 2
#endif
#ifndef CP_BF16_WIDE_FG
#define CP_BF16_WIDE_FG 2
#endif
#ifndef CP_BF16_BC
#define CP_BF16_BC 64
#endif
#ifndef CP_BF16_FRS
#define CP_BF16_FRS 1
#endif
#ifndef CP_BF16_FNPF
#define CP_BF16_FNPF 4  // (3 before the forward staged only its own query rows)
#endif
#ifndef CP_BF16_BNPF
#define CP_BF16_BNPF 4
#endif
#ifndef CP_BF16_BG
#define CP_BF16_BG 2
#endif
#ifndef CP_BF16_BNB
#define CP_BF16_BNB 2
#endif
#ifndef CP_BF16_BRG
#define CP_BF16_BRG 2
#endif
#ifndef CP_BF16_BIDLE
#define CP_BF16_BIDLE -1
#endif
#ifndef CP_BF16_NB2_BC
#define CP_BF16_NB2_BC 64
#endif
#ifndef CP_F32_WIDE_FC
#define CP_F32_WIDE_FC 32
#endif
#ifndef CP_F32_WIDE_BC
#define CP_F32_WIDE_BC 32
#endif
#ifndef CP_F32_BG
#define CP_F32_BG 2
#endif
#ifndef CP_F32_FNPF
#define CP_F32_FNPF 2
#endif
#ifndef CP_F32_BNPF
#define CP_F32_BNPF 3
#endif
#ifndef CP_F32_FC
#define CP_F32_FC 32
#endif
#ifndef CP_F32_FG
#define CP_F32_FG 1
#endif
#ifndef CP_F32_BC
#define CP_F32_BC 32
#endif

namespace cp {

// Waves per role in a backward workgroup of group count G with NB column
// blocks per wave: dQ and dK waves cover the E/16 blocks of E, dV waves the
// M/16 blocks of M; IDLE more waves only help copy.
template <int E, int M, int G, int NB, int IDLE>
constexpr int bwd_waves() {
    return 2 * ((E / 16 + G * NB - 1) / (G * NB)) + (M / 16 + G * NB - 1) / (G * NB) + IDLE;
}

// Backward workgroups per slice: the preferred count, at most one per column
// block, and enough that a workgroup has at most 16 waves.
constexpr int bwd_groups(int E, int M, int pref) {
    const int eb = E / 16, mb = M / 16, most = eb > mb ? eb : mb;
    int g = pref < most ? pref : most;
    while (64 * (2 * ((eb + g - 1) / g) + (mb + g - 1) / g) > 1024) ++g;
    return g;
}

template <typename T, int E, int M> struct Tune;

// 128-wide heads halve the backward chunk so that two workgroups fit a CU's LDS.
template <int E, int M> struct Tune<__bf16, E, M> {
    static constexpr bool wide = E > 64 || M > 64;
    // one-wave workgroups with wide features hold a whole chunk per thread:
    // shorter chunks keep them in registers
    static constexpr int FC = ((M == 16 && E >= 64) || E == 128) && CP_BF16_FC > 32 ? 32 : CP_BF16_FC;
    // 128 output columns: two workgroups of four waves (registers per wave)
    static constexpr int FG0 = M > 64 && CP_BF16_FG < 2 ? CP_BF16_WIDE_FG : CP_BF16_FG;
    static constexpr int FG = FG0 > M / 16 ? M / 16 : FG0;
    static constexpr int BC0 = wide && CP_BF16_BC > 32 ? 32 : CP_BF16_BC;
    // row sets inside a workgroup: two where the workgroup would otherwise
    // be a single wave or spans 128 columns (E = 128: registers)
    static constexpr int FRS = FC >= 64 && E <= 64 ? (M / 16 / FG == 1 || M > 64 ? 2 : CP_BF16_FRS) : 1;
    // row groups of workgroups (whole output rows per workgroup) where the
    // chunk has enough pairs of row blocks
    static constexpr int FRG = M <= 64 && (FC / 16) % (2 * FRS * CP_BF16_FRG) == 0 ? CP_BF16_FRG : 1;
    // the normalised forward: one row set per workgroup (its denominator
    // wave serves the workgroup's rows), row groups as above
    static constexpr int FRG_N = M <= 64 && (FC / 16) % (2 * CP_BF16_FRG) == 0 ? CP_BF16_FRG : 1;
    // a denominator wave per workgroup, but for 128 x 128 heads (its
    // registers would halve the workgroups per CU; there every wave forms
    // its own denominators)
    static constexpr bool FDW = !(E == 128 && M == 128);
    static constexpr int FNPF = E == 128 && CP_BF16_FNPF > 2 ? 2 : CP_BF16_FNPF;  // E = 128: registers
    static constexpr int BNPF = CP_BF16_BNPF;
    // the normalised backward over 128-wide E: its stages also carry the
    // output rows and denominators, and with four of them the twelve-wave
    // workgroup spills (181 VGPRs at its 168 cap); two stages: the L = 16384,
    // E = M = 128 sweep 367 -> 204 us
    static constexpr int BNPF_N = E == 128 && CP_BF16_BNPF > 2 ? 2 : CP_BF16_BNPF;
    // two blocks per wave where they divide evenly and registers allow; such
    // waves run shorter chunks (their per-chunk work is twice as long); with
    // row groups their workgroups take every column and split the rows
    static constexpr bool NB2 = CP_BF16_BNB == 2 && E <= 64 && M <= 64;
    static constexpr int BRG = NB2 && (E / 16) % 2 == 0 && (M / 16) % 2 == 0 ? CP_BF16_BRG : 1;
    static constexpr int BG = BRG > 1 ? 1 : bwd_groups(E, M, CP_BF16_BG);
    static constexpr int BNB = NB2 && (E / 16) % (2 * BG) == 0 && (M / 16) % (2 * BG) == 0 ? 2 : 1;
    static constexpr int BC = BNB == 2 ? CP_BF16_NB2_BC : BC0;
    static constexpr int BIDLE =
        BNB != 2 ? 0 : CP_BF16_BIDLE >= 0 ? CP_BF16_BIDLE : (4 - bwd_waves<E, M, BG, BNB, 0>() % 4) % 4;
};

// fp16 I/O moves and computes exactly like bf16 I/O.
template <int E, int M> struct Tune<_Float16, E, M> : Tune<__bf16, E, M> {};

// fp32 tiles are twice as large in LDS and registers: the forward over the
// widest heads uses shorter chunks.  (The backward over them keeps 32-row
// chunks: 16-row chunks measured 545 us against 447 us on the fp32
// E = 32, M = 128, L = 2048 fwd+bwd workload.)
template <int E, int M> struct Tune<float, E, M> {
    static constexpr bool wide = E > 64 || M > 64;
    static constexpr int FC = wide ? CP_F32_WIDE_FC : CP_F32_FC;
    static constexpr int FG0 = M > 64 && CP_F32_FG < 2 ? 2 : CP_F32_FG;
    static constexpr int FG = FG0 > M / 16 ? M / 16 : FG0;
    static constexpr int BC = wide ? CP_F32_WIDE_BC : CP_F32_BC;
    static constexpr int FRS = 1;
    static constexpr int FRG = 1;
    static constexpr int FRG_N = 1;
    static constexpr bool FDW = !(E == 128 && M == 128);
    static constexpr int FNPF = CP_F32_FNPF;
    // three stages where registers allow (E = 32, M = 128 backward: 278 ->
    // 261 us); two where a third spills (E = 128, or E = 64 with M = 128) and
    // in the normalised backward
    static constexpr int BNPF = E == 128 || (E == 64 && M == 128) ? 2 : CP_F32_BNPF;
    static constexpr int BNPF_N = 2;
    static constexpr int BG = bwd_groups(E, M, CP_F32_BG);
    static constexpr int BNB = 1;
    static constexpr int BRG = 1;
    static constexpr int BIDLE = 0;
};

}  // namespace cp
