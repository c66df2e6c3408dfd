// cp_launch.hpp -- host-side launch table between the C ABI and the kernels.
// Each dtype/direction lives in its own translation unit; the C ABI picks a
// launcher by (dtype, E, M) and passes sizes already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cp_validate.hpp"

namespace cp {

struct FwdArgs {
    const void *Q, *K, *V;
    void *Out;
    const float *state_in, *z_in;  // optional initial S and z
    float *state_out, *z_out;      // optional final S and z
    float *den_out;                // optional denominators (normalised form) [NS][L]
    int L, NS;
    float eps;
    int fmap;
    int Ea, Ma;  // head sizes of the tensors (the kernel runs the next tile size up)
    // Scratch of a forward over sequence segments.  ws_need != NULL: only
    // report the bytes the call needs (0 without segments) and launch
    // nothing.  ws != NULL: use ws_bytes bytes at ws (a call that needs more
    // fails) and allocate nothing; with ws == NULL and noalloc set, a call
    // that needs scratch fails; otherwise it comes from the stream-ordered
    // allocator.
    size_t *ws_need = nullptr;
    float *ws = nullptr;
    size_t ws_bytes = 0;
    bool noalloc = false;
};

struct BwdArgs {
    const void *Q, *K, *V, *G;
    const float *state_in;     // optional initial state S0
    const float *state_final;  // optional final state S_{L-1}
    void *dQ, *dK, *dV;
    float *dstate_in;  // optional gradient of S0
    int L, NS;
    // backward of the normalised form only
    const void *Out;    // the forward's output
    const float *den;   // the forward's denominators [NS][L]
    const float *z_in;     // optional initial z
    const float *z_final;  // optional z after the last row (with state_final)
    float *dz_in;
    int fmap;
    int Ea, Ma;  // head sizes of the tensors (the kernel runs the next tile size up)
};

// Each launcher enqueues one kernel on stream and returns hipSuccess or the
// launch error.  NULL when (E, M) is not instantiated.
typedef hipError_t (*fwd_fn)(const FwdArgs &, hipStream_t);
typedef hipError_t (*bwd_fn)(const BwdArgs &, hipStream_t);

fwd_fn fwd_f32(int E, int M, bool norm);
fwd_fn fwd_bf16(int E, int M, bool norm);
fwd_fn fwd_f16(int E, int M, bool norm);
bwd_fn bwd_f32(int E, int M, bool norm);
bwd_fn bwd_bf16(int E, int M, bool norm);
bwd_fn bwd_f16(int E, int M, bool norm);

// Launch a kernel on stream: hipLaunchKernel, or, while the calling thread
// has a timing in progress (cp_timing_begin), hipExtLaunchKernel with the
// next pair of timing events.
hipError_t launch_kernel(const void *kernel, dim3 grid, dim3 block, void **args, hipStream_t stream);

}  // namespace cp
