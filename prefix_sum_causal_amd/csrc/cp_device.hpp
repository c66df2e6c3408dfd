// cp_device.hpp -- wave-level building blocks of the causal-product kernels
// for gfx950 (CDNA4): 16x16 MFMA tiles, operand fragments and their loads.
//
// Every kernel in this library runs one 64-lane wave per workgroup and splits
// lane l into g = l / 16 (0..3) and r = l % 16.  All matrix products are
// 16 x 16 output tiles D += A * B computed by MFMA:
//   bf16 I/O: v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, fp32 accumulate)
//   fp32 I/O: v_mfma_f32_16x16x4_f32   (A 16x4,  B 4x16)
// with these lane layouts (checked on gfx950):
//   A operand: lane (g, r) holds row r of A,
//   B operand: lane (g, r) holds column r of B,
//   D result : lane (g, r) holds D[4g + t][r], t = 0..3.
//
// The contraction index k is cut into blocks of 16.  A "fragment" is the four
// values lane (g, r) holds for one k-block: k = 16 b + 4g + t, t = 0..3.  The
// bf16 MFMA consumes two k-blocks (8 values per lane), the fp32 MFMA one
// value per lane four times.  Since the result of a tile holds exactly the
// rows 4g + t in lane (g, r), a result tile D can be fed back without any
// lane shuffle: as a B operand it is D itself, as an A operand it is D^T.
//
// Three fragment sources are used:
//   natural  (ld_nat):  lane (g, r) <- X[row0 + 16 rb + r][16 cb + 4g + t]
//            4 consecutive elements of one row, read straight from HBM with
//            a buffer load.
//            As an A operand this is X, as a B operand X^T.
//   transposed (tr_frag): lane (g, r) <- X[16 tb + 4g + t][16 cb + r]
//            4 consecutive rows of one column, read from a natural copy of
//            the chunk in LDS (bf16: one ds_read_b64_tr_b16, which hands lane
//            i of each 16-lane group element i of the four 16-element rows
//            addressed by lanes 4a..4a+3).  As an A operand this is X^T, as a
//            B operand X.
//   result tiles, as above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cp {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16))));
typedef bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int lane_g() { return (threadIdx.x >> 4) & 3; }
__device__ __forceinline__ int lane_r() { return threadIdx.x & 15; }

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

template <typename T> struct Ops;

// bf16 I/O: fragments are 4 bf16; MFMA over two k-blocks at a time.
template <> struct Ops<bf16> {
    using frag = bf16x4;
    static constexpr int kPad = 8;  // LDS row padding (elements)

    __device__ static __forceinline__ frag zero() {
        s16x4 z = {0, 0, 0, 0};
        return __builtin_bit_cast(frag, z);
    }
    __device__ static __forceinline__ frag ones() {
        s16x4 o = {0x3F80, 0x3F80, 0x3F80, 0x3F80};
        return __builtin_bit_cast(frag, o);
    }
    __device__ static __forceinline__ void mma2(f32x4 &acc, frag a0, frag a1, frag b0, frag b1) {
        bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    __device__ static __forceinline__ void mma1(f32x4 &acc, frag a0, frag b0) {
        mma2(acc, a0, zero(), b0, zero());
    }
    __device__ static __forceinline__ frag cvt(f32x4 x) {
        frag f;
#pragma unroll
        for (int t = 0; t < 4; ++t) f[t] = (bf16)x[t];
        return f;
    }
    // x ~= hi + lo with both halves in bf16 (16 significant bits in total).
    __device__ static __forceinline__ void split(f32x4 x, frag &hi, frag &lo) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            hi[t] = (bf16)x[t];
            lo[t] = (bf16)(x[t] - (float)hi[t]);
        }
    }
    __device__ static __forceinline__ frag neg(frag a) {
        s16x4 s = __builtin_bit_cast(s16x4, a);
        s16x4 m = {(short)0x8000, (short)0x8000, (short)0x8000, (short)0x8000};
        return __builtin_bit_cast(frag, s ^ m);
    }
    __device__ static __forceinline__ f32x4 widen(frag a) {
        f32x4 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = (float)a[t];
        return x;
    }
    // lane (g, r) <- X[16 tb + 4g + t][16 cb + r] from a natural LDS copy
    // with row stride rs (elements).
    __device__ static __forceinline__ frag tr_frag(const bf16 *lds, int rs, int tb, int cb) {
        const int g = lane_g(), i = lane_r();
        const bf16 *p = lds + (16 * tb + 4 * g + (i >> 2)) * rs + 16 * cb + 4 * (i & 3);
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)((__attribute__((address_space(3))) char *)(p)));
        return __builtin_bit_cast(frag, v);
    }
};

// fp32 I/O: fragments are 4 floats; the fp32 MFMA takes one k value per lane,
// so a k-block is four MFMAs (t = 0..3 pairs k = 4g + t on both operands).
template <> struct Ops<float> {
    using frag = f32x4;
    static constexpr int kPad = 4;

    __device__ static __forceinline__ frag zero() { return zero4(); }
    __device__ static __forceinline__ frag ones() {
        f32x4 o = {1.f, 1.f, 1.f, 1.f};
        return o;
    }
    __device__ static __forceinline__ void mma1(f32x4 &acc, frag a, frag b) {
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc, 0, 0, 0);
    }
    __device__ static __forceinline__ void mma2(f32x4 &acc, frag a0, frag a1, frag b0, frag b1) {
        mma1(acc, a0, b0);
        mma1(acc, a1, b1);
    }
    __device__ static __forceinline__ frag cvt(f32x4 x) { return x; }
    __device__ static __forceinline__ void split(f32x4 x, frag &hi, frag &lo) {
        hi = x;
        lo = zero4();
    }
    __device__ static __forceinline__ frag neg(frag a) { return -a; }
    __device__ static __forceinline__ f32x4 widen(frag a) { return a; }
    __device__ static __forceinline__ frag tr_frag(const float *lds, int rs, int tb, int cb) {
        const int g = lane_g(), r = lane_r();
        f32x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = lds[(16 * tb + 4 * g + t) * rs + 16 * cb + r];
        return v;
    }
};

// acc += sum over k-blocks b in [b0, b1) of A_b * B_b.  For bf16 the blocks
// go to the MFMA in pairs; an odd count is padded with a zero block.
template <typename T, typename FA, typename FB>
__device__ __forceinline__ void dotk(f32x4 &acc, int b0, int b1, FA fa, FB fb) {
    using O = Ops<T>;
    int b = b0;
#pragma unroll
    for (; b + 1 < b1; b += 2) O::mma2(acc, fa(b), fa(b + 1), fb(b), fb(b + 1));
    if (b < b1) O::mma1(acc, fa(b), fb(b));
}

// A chunk of C rows of one row-major slice (leading dimension ld elements),
// addressed through a buffer resource whose range ends at row L: loads past
// the range return zero and stores past it are dropped by the hardware, so
// every access is issued unconditionally (no divergent branches around
// memory operations, which keeps the load pipeline's wait counts exact) and
// rows outside [0, L) never touch memory.
constexpr int kBufferDword3 = 0x00020000;  // gfx9-family raw buffer, no swizzle

template <typename T>
struct Rows {
    __amdgpu_buffer_rsrc_t rsrc;
    int ld;
    // rows [row0, row0 + C) of the slice at base; rows < 0 or >= L are void
    __device__ __forceinline__ Rows(const T *base, int ld_, int row0, int L, int C) : ld(ld_) {
        int n = (row0 < 0) ? 0 : L - row0;
        n = n < 0 ? 0 : (n > C ? C : n);
        // the range is the same for every lane: keep it in scalar registers
        n = __builtin_amdgcn_readfirstlane(n);
        const T *p = base + (int64_t)(row0 > 0 ? row0 : 0) * ld;
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(p), (short)0, n * ld * (int)sizeof(T),
                                                 kBufferDword3);
    }
};

// Natural fragment of the 16-row block rb: lane (g, r) <- X[16 rb + r][16 cb + 4g + t].
template <typename T>
__device__ __forceinline__ typename Ops<T>::frag ld_nat(const Rows<T> &X, int rb, int cb) {
    const int off = ((16 * rb + lane_r()) * X.ld + 16 * cb + 4 * lane_g()) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
        auto v = __builtin_amdgcn_raw_buffer_load_b64(X.rsrc, off, 0, 0);
        return __builtin_bit_cast(typename Ops<T>::frag, v);
    } else {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(X.rsrc, off, 0, 0);
        return __builtin_bit_cast(typename Ops<T>::frag, v);
    }
}

// Store a transposed result tile: lane (g, r) holds X[16 rb + r][16 cb + 4g + t].
template <typename T>
__device__ __forceinline__ void st_out(const Rows<T> &X, int rb, int cb, f32x4 v) {
    const int off = ((16 * rb + lane_r()) * X.ld + 16 * cb + 4 * lane_g()) * (int)sizeof(T);
    if constexpr (sizeof(T) == 2) {
        typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, Ops<T>::cvt(v)), X.rsrc, off, 0, 0);
    } else {
        typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), X.rsrc, off, 0, 0);
    }
}

// Store a natural fragment into an LDS copy of the chunk (row stride rs).
template <typename T>
__device__ __forceinline__ void st_lds(T *lds, int rs, int rb, int cb, typename Ops<T>::frag f) {
    *reinterpret_cast<typename Ops<T>::frag *>(lds + (16 * rb + lane_r()) * rs + 16 * cb + 4 * lane_g()) = f;
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data and vice versa.  A workgroup here is a single wave, so this is all the
// synchronisation LDS needs (no s_barrier, no wait on global loads).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Causal mask of a diagonal tile in the layout D[j][i] (rows = keys j,
// columns = queries i): keep j <= i, i.e. 4g + t <= r.
__device__ __forceinline__ f32x4 mask_keys_rows(f32x4 a) {
    const int g = lane_g(), r = lane_r();
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (4 * g + t > r) a[t] = 0.f;
    return a;
}

// Causal mask of a diagonal tile in the layout D[i][j] (rows = queries i,
// columns = keys j): keep j <= i, i.e. r <= 4g + t.
__device__ __forceinline__ f32x4 mask_query_rows(f32x4 a) {
    const int g = lane_g(), r = lane_r();
#pragma unroll
    for (int t = 0; t < 4; ++t)
        if (r > 4 * g + t) a[t] = 0.f;
    return a;
}

// Workgroup id -> (slice, part).  The P parts of one (n, h) slice read the
// same rows of the inputs, so they are kept on one XCD (workgroups are
// dispatched to the 8 XCDs round robin by id) where they share its L2.
__device__ __forceinline__ void map_block(int b, int NS, int P, int &slice, int &part) {
    if ((NS & 7) == 0) {
        const int x = b & 7, u = b >> 3;
        slice = x * (NS >> 3) + u / P;
        part = u % P;
    } else {
        slice = b / P;
        part = b % P;
    }
}

// phi(x) = elu(x) + 1 = x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <typename T>
__device__ __forceinline__ typename Ops<T>::frag phi_frag(typename Ops<T>::frag f) {
    f32x4 x = Ops<T>::widen(f);
#pragma unroll
    for (int t = 0; t < 4; ++t) x[t] = phi(x[t]);
    return Ops<T>::cvt(x);
}

}  // namespace cp
