// cp_plan.hpp -- host-only launch planning shared by the forward and backward
// launchers: how a call over few slices is cut into sequence segments.  No
// HIP types, so the host tests (under the sanitizers) include it directly.
#pragma once

namespace cp {

// Segments per slice for L rows and NS slices (forward and backward): one,
// unless the slices leave most CUs idle; then enough segments of at least
// kMinSegChunks chunks for about two workgroups per CU.
#ifndef CP_SEG_MIN_CHUNKS
#define CP_SEG_MIN_CHUNKS 4
#endif
#ifndef CP_SEG_WG_PER_CU
#define CP_SEG_WG_PER_CU 2
#endif
#ifndef CP_BWD_SEG_WG_PER_CU
#define CP_BWD_SEG_WG_PER_CU 1
#endif
constexpr int kCUs = 256, kMinSegChunks = CP_SEG_MIN_CHUNKS, kSegWgPerCU = CP_SEG_WG_PER_CU;
constexpr int kBwdSegWgPerCU = CP_BWD_SEG_WG_PER_CU;  // the backward's workgroups hold a CU each
inline int seq_segments(int L, int NS, int groups, int C, int wg_per_cu = kSegWgPerCU) {
    const long long wg = (long long)NS * groups;
    const long long nchunks = ((long long)L + C - 1) / C;
    if (wg >= kCUs || nchunks < 2 * kMinSegChunks) return 1;
    const long long want = ((long long)wg_per_cu * kCUs + wg - 1) / wg;
    const long long most = nchunks / kMinSegChunks;
    return (int)(want < most ? want : most);
}

// The segments of a call: nseg segments of seg_len rows (a whole number of
// C-row chunks; the last one may be shorter, none is empty), or one segment
// of all L rows.  The kernels recover nseg as ceil(L / seg_len).
struct SegPlan {
    int nseg, seg_len;
};
inline SegPlan plan_segments(int L, int NS, int groups, int C, int wg_per_cu = kSegWgPerCU) {
    const int nseg0 = seq_segments(L, NS, groups, C, wg_per_cu);
    if (nseg0 <= 1) return SegPlan{1, L};
    const long long nchunks = ((long long)L + C - 1) / C;
    const long long seg_len = (nchunks + nseg0 - 1) / nseg0 * C;  // < L: nseg0 >= 2, nchunks >= 8
    const long long nseg = ((long long)L + seg_len - 1) / seg_len;
    return nseg > 1 ? SegPlan{(int)nseg, (int)seg_len} : SegPlan{1, L};
}

}  // namespace cp
