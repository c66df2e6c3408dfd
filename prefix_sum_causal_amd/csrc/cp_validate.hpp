// cp_validate.hpp -- argument checks of the C ABI (include/causalprod.h).
// Plain host C++ with no HIP dependency: every check runs before anything is
// enqueued, so a call that fails here has no side effect, and the checks can
// be built and exercised on their own (with sanitizers) on a machine without
// a GPU.
#pragma once

#include <stdint.h>

#include <cmath>
#include <initializer_list>

#include "causalprod.h"

namespace cp {

// Index 0..3 of the kernel tile size {16, 32, 64, 128} that runs a head of
// x features: the smallest one >= x; -1 for x outside [1, 128].  A head
// narrower than its tile is padded with zero columns on load and its padding
// is never stored.
inline int tile_index(int64_t x) {
    return x < 1 ? -1 : x <= 16 ? 0 : x <= 32 ? 1 : x <= 64 ? 2 : x <= 128 ? 3 : -1;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups a launch may give one (n, h) slice: bounds N*H so that grid
// sizes stay in 32 bits.
constexpr int kMaxPartsPerSlice = 128 / 16 * 3;

// Shape checks shared by every entry point.  On success fills the element
// counts of the [N][H][L][E] and [N][H][L][M] tensors.
inline int check_dims(int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype, int64_t &ne, int64_t &nm) {
    if (N <= 0 || H <= 0 || L <= 0 || E <= 0 || M <= 0) return CP_ERR_DIM;
    if (dtype != CP_F32 && dtype != CP_BF16 && dtype != CP_F16) return CP_ERR_UNSUPPORTED;
    // head sizes up to 128 whose rows are whole 16-byte pieces
    const int64_t es = dtype == CP_F32 ? 4 : 2;
    if (tile_index(E) < 0 || tile_index(M) < 0 || (E * es) % 16 != 0 || (M * es) % 16 != 0) return CP_ERR_UNSUPPORTED;
    if (L > INT32_MAX) return CP_ERR_DIM;
    // N*H slices, each launched as up to kMaxPartsPerSlice workgroups
    if (N > INT32_MAX / H) return CP_ERR_DIM;
    const int64_t NS = N * H;
    if (NS > INT32_MAX / kMaxPartsPerSlice) return CP_ERR_DIM;
    // element counts in bytes must fit in int64
    const int64_t limit = INT64_MAX / 8 / 128;
    if (NS > limit / L) return CP_ERR_DIM;
    ne = NS * L * E;
    nm = NS * L * M;
    return CP_OK;
}

inline int check_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (!p) return CP_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned16(p)) return CP_ERR_ALIGN;
    return CP_OK;
}

// Optional pointers (may be NULL): when given, 16-byte aligned.
inline int check_opt_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return CP_ERR_ALIGN;
    return CP_OK;
}

// Every output must be disjoint from every input and from the other outputs
// (a NULL optional pointer has an empty range and overlaps nothing).  A
// caller's workspace (ws, ws_bytes) counts as an output.
inline int check_alias(std::initializer_list<Range> ins, std::initializer_list<Range> outs) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range &i : ins)
            if (overlap(*o, i)) return CP_ERR_ALIAS;
        for (auto p = o + 1; p != outs.end(); ++p)
            if (overlap(*o, *p)) return CP_ERR_ALIAS;
    }
    return CP_OK;
}

// The byte range of a buffer (a NULL pointer: the empty range); a range
// that would run past the end of the address space ends there.
inline Range span(const void *p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (!p || bytes <= 0) return Range{0, 0};
    const uintptr_t b = static_cast<uintptr_t>(bytes);
    return Range{a, a > UINTPTR_MAX - b ? UINTPTR_MAX : a + b};
}

inline int64_t elem_bytes(int dtype) { return dtype == CP_F32 ? 4 : 2; }

inline int validate_fwd(const void *Q, const void *K, const void *V, const void *Out, const float *state_in,
                        const float *state_out, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                        const void *ws = nullptr, int64_t ws_bytes = 0) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, ne, nm);
    if (st != CP_OK) return st;
    st = check_ptrs({Q, K, V, Out});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, state_out, ws});
    if (st != CP_OK) return st;
    const int64_t es = elem_bytes(dtype), ns = N * H * E * M * 4;
    return check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(state_in, ns)},
                       {span(Out, nm * es), span(state_out, ns), span(ws, ws_bytes)});
}

inline int validate_bwd(const void *Q, const void *K, const void *V, const void *dOut, const float *state_in,
                        const float *state_final, const void *dQ, const void *dK, const void *dV,
                        const float *dstate_in, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                        const void *ws = nullptr, int64_t ws_bytes = 0) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, ne, nm);
    if (st != CP_OK) return st;
    st = check_ptrs({Q, K, V, dOut, dQ, dK, dV});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, state_final, dstate_in, ws});
    if (st != CP_OK) return st;
    const int64_t es = elem_bytes(dtype), ns = N * H * E * M * 4;
    return check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(dOut, nm * es),
                        span(state_in, ns), span(state_final, ns)},
                       {span(dQ, ne * es), span(dK, ne * es), span(dV, nm * es), span(dstate_in, ns), span(ws, ws_bytes)});
}

inline int validate_linattn_fwd(const void *Q, const void *K, const void *V, const void *Out, const float *state_in,
                                const float *z_in, const float *state_out, const float *z_out, const float *den_out,
                                int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, float eps, int feature_map,
                                int dtype,
                                const void *ws = nullptr, int64_t ws_bytes = 0) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, ne, nm);
    if (st != CP_OK) return st;
    if (feature_map != 0 && feature_map != 1) return CP_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return CP_ERR_UNSUPPORTED;
    st = check_ptrs({Q, K, V, Out});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, z_in, state_out, z_out, den_out, ws});
    if (st != CP_OK) return st;
    const int64_t es = elem_bytes(dtype), ns = N * H * E * M * 4, nz = N * H * E * 4, nd = N * H * L * 4;
    return check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(state_in, ns), span(z_in, nz)},
                       {span(Out, nm * es), span(state_out, ns), span(z_out, nz), span(den_out, nd), span(ws, ws_bytes)});
}

inline int validate_linattn_bwd(const void *Q, const void *K, const void *V, const void *Out, const void *dOut,
                                const float *den, const float *state_in, const float *z_in, const float *state_final,
                                const float *z_final, const void *dQ, const void *dK, const void *dV,
                                const float *dstate_in, const float *dz_in, int64_t N, int64_t H, int64_t L, int64_t E,
                                int64_t M, int feature_map, int dtype,
                                const void *ws = nullptr, int64_t ws_bytes = 0) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, ne, nm);
    if (st != CP_OK) return st;
    if (feature_map != 0 && feature_map != 1) return CP_ERR_UNSUPPORTED;
    st = check_ptrs({Q, K, V, Out, dOut, den, dQ, dK, dV});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, z_in, state_final, z_final, dstate_in, dz_in, ws});
    if (st != CP_OK) return st;
    const int64_t es = elem_bytes(dtype), ns = N * H * E * M * 4, nz = N * H * E * 4, nd = N * H * L * 4;
    return check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(Out, nm * es),
                        span(dOut, nm * es), span(den, nd), span(state_in, ns), span(z_in, nz),
                        span(state_final, ns), span(z_final, nz)},
                       {span(dQ, ne * es), span(dK, ne * es), span(dV, nm * es), span(dstate_in, ns),
                        span(dz_in, nz), span(ws, ws_bytes)});
}

}  // namespace cp
