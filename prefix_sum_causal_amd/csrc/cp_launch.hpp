// cp_launch.hpp -- host-side launch table between the C ABI and the kernels.
// Each dtype/direction lives in its own translation unit; the C ABI picks a
// launcher by (dtype, E, M) and passes sizes already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "cp_plan.hpp"
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
    // nothing (the pointers are not read).  ws != NULL: use ws_bytes bytes at
    // ws (a call that needs more fails) and allocate nothing; with ws == NULL
    // and noalloc set, a call that needs scratch fails; otherwise it comes
    // from the stream-ordered allocator.
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
    // Scratch of a backward over sequence segments, as for FwdArgs (no
    // noalloc flag: every backward either gets ws or may allocate).
    size_t *ws_need = nullptr;
    float *ws = nullptr;
    size_t ws_bytes = 0;
};

// stages of the load ring of the segment-increment pass, and its waves (at
// most CP_SEG_MAXW, each owning M/16/waves column blocks of the increment)
#ifndef CP_SEG_NPF
#define CP_SEG_NPF 4
#endif
#ifndef CP_SEG_MAXW
#define CP_SEG_MAXW 8  // (8 rather than 4: the L = 16384, 128-wide passes 103 -> 84 us and 36 -> 31 us)
#endif
template <int M>
constexpr int seg_state_waves() { return M / 16 >= CP_SEG_MAXW ? CP_SEG_MAXW : M / 16; }

// Each launcher enqueues one kernel on stream and returns hipSuccess or the
// launch error.  NULL when (E, M) is not instantiated.
typedef hipError_t (*fwd_fn)(const FwdArgs &, hipStream_t);
typedef hipError_t (*bwd_fn)(const BwdArgs &, hipStream_t);

// The backward's segment-increment pass (cp_seg_state_kernel with two jobs:
// the prefix increments, sum k v^T (and of k), over segments first1 ..
// first1 + nseg-2 into ws1; the suffix increments, sum q dO^T (normalised form: of phi(q)
// dn^T, and of dd phi(q), from the output O2 and den2), over segments
// 1 .. nseg-1 into ws2); its instances live with the forward's.
struct SegArgs {
    const void *K1, *V1;
    float *ws1;
    const void *K2, *V2, *O2;
    const float *den2;
    float *ws2;
    int L, NS, seg_len, sub, first1, Ea, Ma;  // sub: parts (workgroups, slots) per segment increment
    bool norm, fmap;
};
typedef hipError_t (*seg_fn)(const SegArgs &, hipStream_t);
seg_fn seg_f32(int E, int M);
seg_fn seg_bf16(int E, int M);
seg_fn seg_f16(int E, int M);

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
