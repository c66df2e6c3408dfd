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
#include <mutex>
#include <vector>

#include "cp_launch.hpp"
#include "cp_validate.hpp"

// Scratch of causal_product_fwd_noalloc: the per-segment state increments of
// a forward over sequence segments live in this file-scope device array
// instead of stream-ordered allocations.  Each GPU the library runs on holds
// its own copy until the process ends; in host code `scratch` only names the
// symbol, so the entry point uses the device address that
// hipGetSymbolAddress returns for it, looked up once per device (with that
// device current) and kept in scratch_dev.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kAbiMajor = 6, kAbiMinor = 0;  // 3.0: carried state, normalised backward; 3.1: fp16 I/O;
                                             // 4.0: cp_timing_end bounded by the caller's buffer;
                                             // 4.1: causal_product_fwd_noalloc;
                                             // 5.0: linear_attn_bwd takes z_final, no scratch unsplit;
                                             // 6.0: caller workspaces, cp_workspace_size

cp::fwd_fn pick_fwd(int dtype, int E, int M, bool norm) {
    return dtype == CP_BF16 ? cp::fwd_bf16(E, M, norm) : dtype == CP_F16 ? cp::fwd_f16(E, M, norm) : cp::fwd_f32(E, M, norm);
}

cp::bwd_fn pick_bwd(int dtype, int E, int M, bool norm) {
    return dtype == CP_BF16 ? cp::bwd_bf16(E, M, norm) : dtype == CP_F16 ? cp::bwd_f16(E, M, norm) : cp::bwd_f32(E, M, norm);
}

int launch_status(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

// A call with the caller's workspace: the bytes it needs (host arithmetic,
// nothing launched), then the call itself on that workspace.  Without a
// workspace the launcher allocates what it needs.
template <typename Fn, typename Args>
int run_with_workspace(Fn fn, Args a, void *ws, int64_t ws_bytes, hipStream_t stream) {
    if (ws) {
        size_t need = 0;
        a.ws_need = &need;
        if (fn(a, stream) != hipSuccess) return CP_ERR_HIP;
        if (ws_bytes < 0 || need > (uint64_t)ws_bytes) return CP_ERR_SCRATCH;
        a.ws_need = nullptr;
        a.ws = static_cast<float *>(ws);
        a.ws_bytes = (size_t)ws_bytes;
    }
    return launch_status(fn(a, stream));
}

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

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the device that runs `stream` (the
// current device for the NULL stream).
int scratch_address(hipStream_t stream, void **addr) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return CP_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return CP_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return CP_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return CP_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return CP_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return CP_ERR_HIP;
        scratch_dev[dev] = p;
    }
    *addr = scratch_dev[dev];
    return CP_OK;
}

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
        case CP_ERR_SCRATCH: return "the workspace is smaller than the call needs (cp_workspace_size), or the call needs more scratch than the no-allocation entry point holds (16 MiB)";
        default: return "unknown status";
    }
}

int cp_workspace_size(int op, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype, int64_t *bytes) {
    if (!bytes) return CP_ERR_NULL;
    if (op < CP_OP_CAUSAL_FWD || op > CP_OP_LINATTN_BWD) return CP_ERR_UNSUPPORTED;
    int64_t ne = 0, nm = 0;
    const int st = cp::check_dims(N, H, L, E, M, dtype, ne, nm);
    if (st != CP_OK) return st;
    const bool norm = op == CP_OP_LINATTN_FWD || op == CP_OP_LINATTN_BWD;
    size_t need = 0;
    hipError_t e = hipSuccess;
    if (op == CP_OP_CAUSAL_FWD || op == CP_OP_LINATTN_FWD) {
        cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, norm);
        if (!fn) return CP_ERR_UNSUPPORTED;
        cp::FwdArgs a{};
        a.L = (int)L, a.NS = (int)(N * H), a.Ea = (int)E, a.Ma = (int)M, a.ws_need = &need;
        e = fn(a, nullptr);
    } else {
        cp::bwd_fn fn = pick_bwd(dtype, (int)E, (int)M, norm);
        if (!fn) return CP_ERR_UNSUPPORTED;
        cp::BwdArgs a{};
        a.L = (int)L, a.NS = (int)(N * H), a.Ea = (int)E, a.Ma = (int)M, a.ws_need = &need;
        e = fn(a, nullptr);
    }
    if (e != hipSuccess) return CP_ERR_HIP;
    *bytes = (int64_t)need;
    return CP_OK;
}

int causal_product_fwd(const void *Q, const void *K, const void *V, void *Out, const float *state_in,
                       float *state_out, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                       void *workspace, int64_t workspace_bytes, void *stream) {
    const int st = cp::validate_fwd(Q, K, V, Out, state_in, state_out, N, H, L, E, M, dtype, workspace,
                                    workspace_bytes);
    if (st != CP_OK) return st;
    cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, false);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::FwdArgs a{Q,      K,      V, Out, state_in, nullptr, state_out, nullptr, nullptr, (int)L, (int)(N * H), 0.f,
                  0,      (int)E, (int)M};
    return run_with_workspace(fn, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int causal_product_fwd_noalloc(const void *Q, const void *K, const void *V, void *Out, const float *state_in,
                               float *state_out, int64_t N, int64_t H, int64_t L, int64_t E, int64_t M, int dtype,
                               void *stream) {
    int st = cp::validate_fwd(Q, K, V, Out, state_in, state_out, N, H, L, E, M, dtype);
    if (st != CP_OK) return st;
    cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, false);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::FwdArgs a{Q,      K,      V, Out, state_in, nullptr, state_out, nullptr, nullptr, (int)L, (int)(N * H), 0.f,
                  0,      (int)E, (int)M};
    // the scratch this call needs (host arithmetic only, nothing is launched)
    size_t need = 0;
    a.ws_need = &need;
    if (fn(a, static_cast<hipStream_t>(stream)) != hipSuccess) return CP_ERR_HIP;
    if (need > kScratchBytes) return CP_ERR_SCRATCH;
    void *ws = nullptr;
    st = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (st != CP_OK) return st;
    a.ws_need = nullptr;
    a.ws = static_cast<float *>(ws);
    a.ws_bytes = kScratchBytes;
    a.noalloc = true;
    return launch_status(fn(a, static_cast<hipStream_t>(stream)));
}

int causal_product_bwd(const void *Q, const void *K, const void *V, const void *dOut, const float *state_in,
                       const float *state_final, void *dQ, void *dK, void *dV, float *dstate_in, int64_t N,
                       int64_t H, int64_t L, int64_t E, int64_t M, int dtype, void *workspace,
                       int64_t workspace_bytes, void *stream) {
    const int st = cp::validate_bwd(Q, K, V, dOut, state_in, state_final, dQ, dK, dV, dstate_in, N, H, L, E, M, dtype,
                                    workspace, workspace_bytes);
    if (st != CP_OK) return st;
    cp::bwd_fn fn = pick_bwd(dtype, (int)E, (int)M, false);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::BwdArgs a{Q,       K,       V,       dOut,    state_in, state_final, dQ,     dK,    dV, dstate_in, (int)L,
                  (int)(N * H), nullptr, nullptr, nullptr, nullptr, nullptr, 0, (int)E, (int)M};
    return run_with_workspace(fn, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int linear_attn_fwd(const void *Q, const void *K, const void *V, void *Out, const float *state_in,
                    const float *z_in, float *state_out, float *z_out, float *den_out, int64_t N, int64_t H,
                    int64_t L, int64_t E, int64_t M, float eps, int feature_map, int dtype, void *workspace,
                    int64_t workspace_bytes, void *stream) {
    const int st = cp::validate_linattn_fwd(Q, K, V, Out, state_in, z_in, state_out, z_out, den_out, N, H, L, E, M, eps,
                                            feature_map, dtype, workspace, workspace_bytes);
    if (st != CP_OK) return st;
    cp::fwd_fn fn = pick_fwd(dtype, (int)E, (int)M, true);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::FwdArgs a{Q,           K,      V,     Out, state_in, z_in, state_out, z_out, den_out, (int)L, (int)(N * H), eps,
                  feature_map, (int)E, (int)M};
    return run_with_workspace(fn, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int linear_attn_bwd(const void *Q, const void *K, const void *V, const void *Out, const void *dOut,
                    const float *den, const float *state_in, const float *z_in, const float *state_final,
                    const float *z_final, void *dQ, void *dK, void *dV, float *dstate_in, float *dz_in, int64_t N,
                    int64_t H, int64_t L, int64_t E, int64_t M, int feature_map, int dtype, void *workspace,
                    int64_t workspace_bytes, void *stream) {
    const int st = cp::validate_linattn_bwd(Q, K, V, Out, dOut, den, state_in, z_in, state_final, z_final, dQ, dK,
                                            dV, dstate_in, dz_in, N, H, L, E, M, feature_map, dtype, workspace,
                                            workspace_bytes);
    if (st != CP_OK) return st;
    cp::bwd_fn fn = pick_bwd(dtype, (int)E, (int)M, true);
    if (!fn) return CP_ERR_UNSUPPORTED;
    cp::BwdArgs a{Q,      K,      V,     dOut,  state_in, state_final, dQ,  dK, dV, dstate_in, (int)L, (int)(N * H),
                  Out,    den,    z_in,  z_final, dz_in, feature_map, (int)E, (int)M};
    return run_with_workspace(fn, a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
