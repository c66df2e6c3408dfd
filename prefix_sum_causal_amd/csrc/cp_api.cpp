// cp_api.cpp -- the C ABI declared in include/causalprod.h: argument
// validation, kernel selection by (dtype, E, M) and launch on the caller's
// stream.  Validation runs before any HIP call, so invalid calls have no side
// effect and need no device.
#include "causalprod.h"

#include <hip/hip_runtime.h>

#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "cp_launch.hpp"

namespace {

constexpr int kAbiMajor = 4, kAbiMinor = 0;  // 3.0: carried state, normalised backward; 3.1: fp16 I/O;
                                             // 4.0: cp_timing_end bounded by the caller's buffer

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.  On success fills the element
// counts of the [N][H][L][E] and [N][H][L][M] tensors.
int check_dims(int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype, int parts_per_slice_max,
               int64_t &ne, int64_t &nm) {
    if (N <= 0 || H <= 0 || L <= 0 || E <= 0 || M <= 0) return CP_ERR_DIM;
    if (dtype != CP_F32 && dtype != CP_BF16 && dtype != CP_F16) return CP_ERR_UNSUPPORTED;
    // head sizes up to 128 whose rows are whole 16-byte pieces
    const int64_t es = dtype == CP_F32 ? 4 : 2;
    if (cp::tile_index(E) < 0 || cp::tile_index(M) < 0 || (E * es) % 16 != 0 || (M * es) % 16 != 0)
        return CP_ERR_UNSUPPORTED;
    if (L > INT32_MAX) return CP_ERR_DIM;
    // N*H slices, each launched as up to parts_per_slice_max workgroups
    if (N > INT32_MAX / H) return CP_ERR_DIM;
    const int64_t NS = N * H;
    if (NS > INT32_MAX / parts_per_slice_max) return CP_ERR_DIM;
    // element counts in bytes must fit in int64
    const int64_t limit = INT64_MAX / 8 / 128;
    if (NS > limit / L) return CP_ERR_DIM;
    ne = NS * L * E;
    nm = NS * L * M;
    return CP_OK;
}

int check_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (!p) return CP_ERR_NULL;
    for (const void *p : ptrs)
        if (!aligned16(p)) return CP_ERR_ALIGN;
    return CP_OK;
}

// Optional pointers (may be NULL): when given, 16-byte aligned.
int check_opt_ptrs(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return CP_ERR_ALIGN;
    return CP_OK;
}

// Every output must be disjoint from every input and from the other outputs
// (a NULL optional pointer has an empty range and overlaps nothing).
int check_alias(std::initializer_list<Range> ins, std::initializer_list<Range> outs) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range &i : ins)
            if (overlap(*o, i)) return CP_ERR_ALIAS;
        for (auto p = o + 1; p != outs.end(); ++p)
            if (overlap(*o, *p)) return CP_ERR_ALIAS;
    }
    return CP_OK;
}

Range span(const void *p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return p ? Range{a, a + static_cast<uintptr_t>(bytes)} : Range{0, 0};
}

cp::fwd_fn pick_fwd(int dtype, int E, int M, bool norm) {
    return dtype == CP_BF16 ? cp::fwd_bf16(E, M, norm) : dtype == CP_F16 ? cp::fwd_f16(E, M, norm) : cp::fwd_f32(E, M, norm);
}

cp::bwd_fn pick_bwd(int dtype, int E, int M, bool norm) {
    return dtype == CP_BF16 ? cp::bwd_bf16(E, M, norm) : dtype == CP_F16 ? cp::bwd_f16(E, M, norm) : cp::bwd_f32(E, M, norm);
}

int launch_status(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

// Per-thread kernel timing (cp_timing_begin / cp_timing_end).
struct Timing {
    bool on = false;
    int used = 0;
    std::vector<hipEvent_t> start, stop;
    void release() {
        for (hipEvent_t e : start) (void)hipEventDestroy(e);
        for (hipEvent_t e : stop) (void)hipEventDestroy(e);
        start.clear();
        stop.clear();
        on = false;
        used = 0;
    }
};
thread_local Timing timing;

}  // namespace

namespace cp {

hipError_t launch_kernel(const void *kernel, dim3 grid, dim3 block, void **args, hipStream_t stream) {
    if (timing.on && timing.used < (int)timing.start.size()) {
        const int i = timing.used++;
        return hipExtLaunchKernel(kernel, grid, block, args, 0, stream, timing.start[i], timing.stop[i], 0);
    }
    return hipLaunchKernel(kernel, grid, block, args, 0, stream);
}

}  // namespace cp

extern "C" {

int cp_abi_version(void) { return (kAbiMajor << 16) | kAbiMinor; }

int cp_timing_begin(int capacity) {
    if (capacity < 1 || capacity > 65536) return CP_ERR_DIM;
    timing.release();
    timing.start.reserve(capacity);
    timing.stop.reserve(capacity);
    for (int i = 0; i < capacity; ++i) {
        hipEvent_t a = nullptr, b = nullptr;
        if (hipEventCreate(&a) != hipSuccess) {
            timing.release();
            return CP_ERR_HIP;
        }
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            timing.release();
            return CP_ERR_HIP;
        }
        timing.start.push_back(a);
        timing.stop.push_back(b);
    }
    timing.on = true;
    return CP_OK;
}

int cp_timing_end(float *ms, int ms_capacity, int *count) {
    if (!ms || !count || !timing.on) return CP_ERR_NULL;
    if (ms_capacity < 1) return CP_ERR_DIM;
    int st = CP_OK;
    const int n = timing.used < ms_capacity ? timing.used : ms_capacity;
    for (int i = 0; i < n && st == CP_OK; ++i) {
        if (hipEventSynchronize(timing.stop[i]) != hipSuccess ||
            hipEventElapsedTime(&ms[i], timing.start[i], timing.stop[i]) != hipSuccess)
            st = CP_ERR_HIP;
    }
    *count = st == CP_OK ? n : 0;
    timing.release();
    return st;
}

const char *cp_status_string(int status) {
    switch (status) {
        case CP_OK: return "success";
        case CP_ERR_NULL: return "a required pointer is NULL";
        case CP_ERR_DIM: return "invalid size: N, H, L, E, M must be > 0, L <= 2^31-1, and the sizes must not overflow";
        case CP_ERR_UNSUPPORTED: return "unsupported argument: E and M must be at most 128 with rows of whole 16-byte pieces (multiples of 8 for 16-bit types, of 4 for fp32); dtype, feature_map or eps out of range";
        case CP_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case CP_ERR_ALIAS: return "an output overlaps an input or another output";
        case CP_ERR_HIP: return "the HIP runtime reported an error when launching the kernel";
        default: return "unknown status";
    }
}

int causal_product_fwd(const void *Q, const void *K, const void *V, void *Out, const float *state_in,
                       float *state_out, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                       void *stream) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, 128 / 16 * 3, ne, nm);
    if (st != CP_OK) return st;
    st = check_ptrs({Q, K, V, Out});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, state_out});
    if (st != CP_OK) return st;
    const int64_t es = dtype == CP_F32 ? 4 : 2, ns = N * H * E * M * 4;
    st = check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(state_in, ns)},
                     {span(Out, nm * es), span(state_out, ns)});
    if (st != CP_OK) return st;

    cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, false);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::FwdArgs a{Q,      K,      V, Out, state_in, nullptr, state_out, nullptr, nullptr, (int)L, (int)(N * H), 0.f,
                  0,      (int)E, (int)M};
    return launch_status(fn(a, static_cast<hipStream_t>(stream)));
}

int causal_product_bwd(const void *Q, const void *K, const void *V, const void *dOut, const float *state_in,
                       const float *state_final, void *dQ, void *dK, void *dV, float *dstate_in, int64_t N,
                       int64_t H, int64_t L, int64_t E, int64_t M, int dtype, void *stream) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, 128 / 16 * 3, ne, nm);
    if (st != CP_OK) return st;
    st = check_ptrs({Q, K, V, dOut, dQ, dK, dV});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, state_final, dstate_in});
    if (st != CP_OK) return st;
    const int64_t es = dtype == CP_F32 ? 4 : 2, ns = N * H * E * M * 4;
    st = check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(dOut, nm * es),
                      span(state_in, ns), span(state_final, ns)},
                     {span(dQ, ne * es), span(dK, ne * es), span(dV, nm * es), span(dstate_in, ns)});
    if (st != CP_OK) return st;

    cp::bwd_fn fn = pick_bwd(dtype, (int)E, (int)M, false);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::BwdArgs a{Q,   K,    V,       dOut,    state_in, state_final, dQ, dK, dV, dstate_in, (int)L, (int)(N * H),
                  nullptr, nullptr, nullptr, nullptr, 0, (int)E, (int)M};
    return launch_status(fn(a, static_cast<hipStream_t>(stream)));
}

int linear_attn_fwd(const void *Q, const void *K, const void *V, void *Out, const float *state_in,
                    const float *z_in, float *state_out, float *z_out, float *den_out, int64_t N, int64_t H,
                    int64_t L, int64_t E, int64_t M, float eps, int feature_map, int dtype, void *stream) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, 128 / 16 * 3, ne, nm);
    if (st != CP_OK) return st;
    if (feature_map != 0 && feature_map != 1) return CP_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return CP_ERR_UNSUPPORTED;
    st = check_ptrs({Q, K, V, Out});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, z_in, state_out, z_out, den_out});
    if (st != CP_OK) return st;
    const int64_t es = dtype == CP_F32 ? 4 : 2, ns = N * H * E * M * 4, nz = N * H * E * 4, nd = N * H * L * 4;
    st = check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(state_in, ns), span(z_in, nz)},
                     {span(Out, nm * es), span(state_out, ns), span(z_out, nz), span(den_out, nd)});
    if (st != CP_OK) return st;

    cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, true);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::FwdArgs a{Q,           K,      V,     Out, state_in, z_in, state_out, z_out, den_out, (int)L, (int)(N * H), eps,
                  feature_map, (int)E, (int)M};
    return launch_status(fn(a, static_cast<hipStream_t>(stream)));
}

int linear_attn_bwd(const void *Q, const void *K, const void *V, const void *Out, const void *dOut,
                    const float *den, const float *state_in, const float *z_in, const float *state_final,
                    void *dQ, void *dK, void *dV, float *dstate_in, float *dz_in, int64_t N,
                    int64_t H, int64_t L, int64_t E, int64_t M, int feature_map, int dtype, void *stream) {
    int64_t ne = 0, nm = 0;
    int st = check_dims(N, H, L, E, M, dtype, 128 / 16 * 3, ne, nm);
    if (st != CP_OK) return st;
    if (feature_map != 0 && feature_map != 1) return CP_ERR_UNSUPPORTED;
    st = check_ptrs({Q, K, V, Out, dOut, den, dQ, dK, dV});
    if (st != CP_OK) return st;
    st = check_opt_ptrs({state_in, z_in, state_final, dstate_in, dz_in});
    if (st != CP_OK) return st;
    const int64_t es = dtype == CP_F32 ? 4 : 2, ns = N * H * E * M * 4, nz = N * H * E * 4, nd = N * H * L * 4;
    st = check_alias({span(Q, ne * es), span(K, ne * es), span(V, nm * es), span(Out, nm * es), span(dOut, nm * es),
                      span(den, nd), span(state_in, ns), span(z_in, nz), span(state_final, ns)},
                     {span(dQ, ne * es), span(dK, ne * es), span(dV, nm * es), span(dstate_in, ns),
                      span(dz_in, nz)});
    if (st != CP_OK) return st;

    cp::bwd_fn fn = pick_bwd(dtype, (int)E, (int)M, true);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::BwdArgs a{Q, K,    V,       dOut,    state_in, state_final, dQ, dK, dV, dstate_in, (int)L, (int)(N * H),
                  Out, den, z_in, dz_in, feature_map, (int)E, (int)M};
    return launch_status(fn(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
