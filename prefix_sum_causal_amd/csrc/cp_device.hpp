// cp_device.hpp -- wave-level building blocks of the causal-product kernels
// for gfx950 (CDNA4): 16x16 MFMA tiles, operand fragments, and the staging of
// chunks of the inputs through LDS.
//
// Lane l of a 64-lane wave is split into g = l / 16 (0..3) and r = l % 16.
// All matrix products are 16 x 16 output tiles D += A * B computed by MFMA:
//   bf16 I/O: v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, fp32 accumulate)
//   fp16 I/O: v_mfma_f32_16x16x32_f16 (same shapes and lane layouts)
//   fp32 I/O: the same MFMA on split hi + lo bf16 operands (see Ops<float>),
//             or v_mfma_f32_16x16x4_f32 (A 16x4, B 4x16)
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
// Inputs reach the waves through LDS: every thread of a workgroup copies
// 16-byte pieces of a chunk of rows from HBM (buffer loads, kept in registers
// while the previous chunk is computed) into a natural row-major copy in LDS.
// Fragments are then read from that copy in two ways:
//   natural  (lds_nat): lane (g, r) <- X[16 rb + r][16 cb + 4g + t]
//            (four consecutive elements of one row).  As an A operand this is
//            X, as a B operand X^T.
//   transposed (tr_frag): lane (g, r) <- X[16 tb + 4g + t][16 cb + r]
//            (four consecutive rows of one column; bf16: one
//            ds_read_b64_tr_b16, which hands lane i of each 16-lane group
//            element i of the four 16-element rows addressed by lanes
//            4a..4a+3).  As an A operand this is X^T, as a B operand X.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace cp {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16))));
typedef bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ int lane_g() { return (threadIdx.x >> 4) & 3; }
__device__ __forceinline__ int lane_r() { return threadIdx.x & 15; }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

template <typename T> struct Ops;

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((__vector_size__(4 * sizeof(f16))));
typedef f16 f16x8 __attribute__((__vector_size__(8 * sizeof(f16))));

// The two 16-bit I/O types: their fragment vectors and MFMA (16x16x32, fp32
// accumulate).  Everything else about them is the same.
template <typename H> struct Half16;
template <> struct Half16<bf16> {
    using x4 = bf16x4;
    using x8 = bf16x8;
    static constexpr short one = 0x3F80;  // 1.0
    __device__ static __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Half16<f16> {
    using x4 = f16x4;
    using x8 = f16x8;
    static constexpr short one = 0x3C00;  // 1.0
    __device__ static __forceinline__ f32x4 mfma(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// 16-bit I/O (bf16 or fp16): fragments are 4 values; MFMA over two k-blocks
// at a time.
template <typename H> struct Ops16 {
    using frag = typename Half16<H>::x4;
    using frag8 = typename Half16<H>::x8;

    __device__ static __forceinline__ frag zero() {
        s16x4 z = {0, 0, 0, 0};
        return __builtin_bit_cast(frag, z);
    }
    __device__ static __forceinline__ frag ones() {
        constexpr short o1 = Half16<H>::one;
        s16x4 o = {o1, o1, o1, o1};
        return __builtin_bit_cast(frag, o);
    }
    __device__ static __forceinline__ void mma2(f32x4 &acc, frag a0, frag a1, frag b0, frag b1) {
        frag8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        frag8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc = Half16<H>::mfma(a, b, acc);
    }
    __device__ static __forceinline__ void mma1(f32x4 &acc, frag a0, frag b0) {
        mma2(acc, a0, zero(), b0, zero());
    }
    __device__ static __forceinline__ frag cvt(f32x4 x) {
        frag f;
#pragma unroll
        for (int t = 0; t < 4; ++t) f[t] = (H)x[t];
        return f;
    }
    // x ~= hi + lo with both halves in the 16-bit type (bf16: 16 significant
    // bits in total; fp16: 22, within its exponent range).
    __device__ static __forceinline__ void split(f32x4 x, frag &hi, frag &lo) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            hi[t] = (H)x[t];
            lo[t] = (H)(x[t] - (float)hi[t]);
        }
    }
    // -a: the sign bits flipped, one 32-bit xor per pair of values
    __device__ static __forceinline__ frag neg(frag a) {
        typedef unsigned u32x2 __attribute__((__vector_size__(2 * sizeof(unsigned))));
        const u32x2 m = {0x80008000u, 0x80008000u};
        return __builtin_bit_cast(frag, __builtin_bit_cast(u32x2, a) ^ m);
    }
    // lane (g, r) <- X[16 tb + 4g + t][16 cb + r] from a natural LDS copy
    // with row stride rs (elements).
    __device__ static __forceinline__ frag tr_frag(const H *lds, int rs, int tb, int cb) {
        const int g = lane_g(), i = lane_r();
        const H *p = lds + (16 * tb + 4 * g + (i >> 2)) * rs + 16 * cb + 4 * (i & 3);
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)((__attribute__((address_space(3))) char *)(p)));
        return __builtin_bit_cast(frag, v);
    }
};
template <> struct Ops<bf16> : Ops16<bf16> {};
template <> struct Ops<f16> : Ops16<f16> {};

// fp32 I/O: products run as split bf16.  Each fp32 operand x is cut into
// hi = bf16(x) and lo = bf16(x - hi), 16 significant bits together, and a
// product keeps hi*hi + hi*lo + lo*hi (the dropped lo*lo term is below 2^-16
// of it): three bf16 MFMAs of 16x16x32 with fp32 accumulation instead of
// eight fp32 MFMAs of 16x16x4 -- gfx950's fp32 matrix rate is a sixteenth of
// its bf16 rate.  Values with at most 16 significant bits (small integers
// among them) are split exactly, so their products are exact.
//
// The inputs are split once, while a chunk is staged: the LDS copy of an
// fp32 row of W values is a row of 2W bf16, the W hi values then the W lo
// values (lds_t<float> = bf16), so that every read of an operand is a bf16
// read of each half and no wave splits what it reads.  A fragment is the pair
// of bf16 fragments; accumulator tiles fed back as operands are split when
// converted (cvt).
struct F32S {
    bf16x4 h, l;
};

// Offset (elements) of the lo half of an fp32 LDS row of stride rs: rows of
// W >= 16 values are 2W bf16 plus a 16-element pad (lds_stride).
__device__ __forceinline__ int lo_half(int rs) { return (rs - 16) >> 1; }

template <> struct Ops<float> {
    using frag = F32S;
    using B = Ops16<bf16>;

    __device__ static __forceinline__ frag zero() { return {B::zero(), B::zero()}; }
    __device__ static __forceinline__ frag ones() { return {B::ones(), B::zero()}; }
    __device__ static __forceinline__ void mma2(f32x4 &acc, frag a0, frag a1, frag b0, frag b1) {
        B::mma2(acc, a0.l, a1.l, b0.h, b1.h);
        B::mma2(acc, a0.h, a1.h, b0.l, b1.l);
        B::mma2(acc, a0.h, a1.h, b0.h, b1.h);
    }
    __device__ static __forceinline__ void mma1(f32x4 &acc, frag a, frag b) { mma2(acc, a, zero(), b, zero()); }
    __device__ static __forceinline__ frag cvt(f32x4 x) {
        frag f;
        B::split(x, f.h, f.l);
        return f;
    }
    // (fp32 states enter the products as one split operand)
    __device__ static __forceinline__ void split(f32x4 x, frag &hi, frag &lo) {
        hi = cvt(x);
        lo = zero();
    }
    __device__ static __forceinline__ frag neg(frag a) { return {B::neg(a.h), B::neg(a.l)}; }
    __device__ static __forceinline__ frag tr_frag(const bf16 *lds, int rs, int tb, int cb) {
        return {B::tr_frag(lds, rs, tb, cb), B::tr_frag(lds + lo_half(rs), rs, tb, cb)};
    }
    // value t of a fragment
    __device__ static __forceinline__ float val(frag a, int t) { return (float)a.h[t] + (float)a.l[t]; }
};

// The element type of the LDS copies of a chunk (see Ops<float>).
template <typename T> struct LdsOf {
    using type = T;
};
template <> struct LdsOf<float> {
    using type = bf16;
};
template <typename T> using lds_t = typename LdsOf<T>::type;

// value t of a 16-bit fragment
template <typename T>
__device__ __forceinline__ float frag_val(typename Ops<T>::frag a, int t) {
    if constexpr (std::is_same<T, float>::value) return Ops<float>::val(a, t);
    else return (float)a[t];
}

// lane (g, r) <- X[16 rb + r][16 cb + 4g + t] from a natural LDS copy with
// row stride rs (elements).
template <typename T>
__device__ __forceinline__ typename Ops<T>::frag lds_nat(const lds_t<T> *lds, int rs, int rb, int cb) {
    const lds_t<T> *p = lds + (16 * rb + lane_r()) * rs + 16 * cb + 4 * lane_g();
    if constexpr (std::is_same<T, float>::value) {
        return {*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + lo_half(rs))};
    } else {
        return *reinterpret_cast<const typename Ops<T>::frag *>(p);
    }
}

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

// (hi, lo) += d with the rounding error kept in lo (Knuth's two-sum, then a
// renormalisation so that hi stays the fp32 value nearest hi + lo).  Needs
// IEEE evaluation as written (no reassociation).
__device__ __forceinline__ void two_sum_acc(f32x4 &hi, f32x4 &lo, const f32x4 &d) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float s = hi[t] + d[t];
        const float bb = s - hi[t];
        const float err = (hi[t] - (s - bb)) + (d[t] - bb);
        const float l = lo[t] + err;
        const float h = s + l;
        lo[t] = l - (h - s);
        hi[t] = h;
    }
}

// phi(x) = elu(x) + 1 = x + 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

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

// A byte offset past every buffer range: loads there read zero, stores are
// dropped.
constexpr int kVoid = 0x7FFFFFF0;

// Store a transposed result tile: lane (g, r) holds X[16 rb + r][16 cb + 4g + t].
// Columns at or past wa (the row's width; a multiple of 4) are not stored.
template <typename T>
__device__ __forceinline__ void st_out(const Rows<T> &X, int rb, int cb, f32x4 v, int wa) {
    const int col = 16 * cb + 4 * lane_g();
    const int off = col < wa ? ((16 * rb + lane_r()) * X.ld + col) * (int)sizeof(T) : kVoid;
    if constexpr (sizeof(T) == 2) {
        typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, Ops<T>::cvt(v)), X.rsrc, off, 0, 0);
    } else {
        typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), X.rsrc, off, 0, 0);
    }
}

// Store two transposed 16-bit result tiles, A at (row block rbA, column
// block cbA) and B at (rbB, cbB), as 16-byte pieces: each lane holds 4
// columns of each tile (st_out's layout); the lane pairs (g, g ^ 1) of a row
// swap halves through ds_bpermute so that lanes with even g hold 8
// consecutive columns of A and lanes with odd g 8 of B.  For two adjacent
// column blocks of one row block this writes 64 contiguous bytes per row in
// one instruction (two st_out calls: 32-byte pieces in two), half the memory
// requests: the headline backward's stores measured 114 -> 100 us.  (Pairing
// two row blocks of one column block halves only the instructions and
// measured no change.)  wa: the row's width, a multiple of 8.
template <typename T>
__device__ __forceinline__ void st_out_pair(const Rows<T> &X, int rbA, int cbA, f32x4 va, int rbB, int cbB, f32x4 vb,
                                            int wa) {
    static_assert(sizeof(T) == 2, "16-bit tiles");
    typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));
    typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
    const int g = lane_g();
    const i32x2 a = __builtin_bit_cast(i32x2, Ops<T>::cvt(va)), b = __builtin_bit_cast(i32x2, Ops<T>::cvt(vb));
    const bool even = (g & 1) == 0;
    const i32x2 send = even ? b : a;  // what the partner keeps
    const int src = ((int)threadIdx.x ^ 16) << 2;
    const int r0 = __builtin_amdgcn_ds_bpermute(src, send[0]), r1 = __builtin_amdgcn_ds_bpermute(src, send[1]);
    const i32x4 v = even ? i32x4{a[0], a[1], r0, r1} : i32x4{r0, r1, b[0], b[1]};
    const int col = even ? 16 * cbA + 4 * g : 16 * cbB + 4 * (g - 1);
    const int row = 16 * (even ? rbA : rbB) + lane_r();
    const int off = col < wa ? (row * X.ld + col) * (int)sizeof(T) : kVoid;
    // non-temporal (aux bit 1, nt): these rows are not read again by the call
    // and written as whole 64-byte pieces; leaving them dirty in the caches
    // made the next kernel write them back (headline: that forward 63.7 ->
    // 54.7 us, this backward 104.5 -> 105.7, the step 187 -> 182 us).  (The
    // 32-byte pieces of st_out measured far slower with nt.)
    __builtin_amdgcn_raw_buffer_store_b128(v, X.rsrc, off, 0, 2);
}

// Row stride (16-bit elements) of the LDS copy of a W-column chunk, a
// multiple of 16 bytes so that every row starts 16-byte aligned.  Measured on
// gfx950 (16 rows read as 16-byte pieces at one column, and 4 x 4 rows read
// as 8-byte pieces by the transposing read): strides of 32 bytes modulo 64
// run both at full rate (about 250 and 225 bytes per clock per CU), strides
// of 16 or 48 bytes modulo 64 at half of it and multiples of 64 bytes at a
// quarter or less.  Rows are therefore padded to 32 modulo 64 bytes (fp32
// rows, stored as their bf16 hi and lo halves, by 32 bytes: lo_half relies
// on it).
template <typename T, int W>
constexpr int lds_stride() {
    constexpr int bytes = W * (int)sizeof(T);  // a row of 16-bit values, or the hi + lo halves of fp32 ones
    return (bytes + (96 - bytes % 64) % 64) / 2;
}

typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));

// Row maps of a chunk copy: staged row r is row RM::map(r) of the chunk.
struct AllRows {
    __device__ static constexpr int map(int r) { return r; }
};

// One thread's share of a chunk copy: C rows (rows RM::map(0 .. C-1) of the
// chunk at row0; all of them by default) and columns [col0, col0 + W) of a
// row-major slice, as 16-byte pieces spread over the NT threads of the
// workgroup (piece p = staged row * W*sizeof(T)/16 + column piece).
// load() issues the buffer loads (rows outside [0, L) and columns at or past
// the row's width wa read as zero: a narrower head is padded to W columns);
// store() writes the pieces into the LDS copy, optionally through phi (the
// elementwise feature map, with rows at or past L and padded columns kept
// zero).
template <typename T, int NT, int C, int W, typename RM = AllRows>
struct Stage {
    static constexpr int NT_ = NT;
    static constexpr int PPR = W * (int)sizeof(T) / 16;  // pieces per row
    static constexpr int P = C * PPR;
    static constexpr int NP = (P + NT - 1) / NT;
    static constexpr int RS = lds_stride<T, W>();
    static_assert(W * (int)sizeof(T) % 16 == 0, "rows must be whole 16-byte pieces");
    static_assert(sizeof(T) == 2 || W % 16 == 0, "fp32 rows of whole 16-value blocks (lo_half)");
    i32x4 v[NP];

    static constexpr int VEC = 16 / (int)sizeof(T);  // elements per piece

    __device__ __forceinline__ void load(const Rows<T> &X, int col0, int wa) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int p = (int)threadIdx.x + i * NT;
            const int row = RM::map(p / PPR), cp = p % PPR;
            int off = (row * X.ld + col0) * (int)sizeof(T) + cp * 16;
            if constexpr (P % NT != 0) off = p < P ? off : kVoid;  // past the range: zero
            off = col0 + cp * VEC < wa ? off : kVoid;                // padded column: zero
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(X.rsrc, off, 0, 0);
        }
    }

    template <bool PHI = false>
    __device__ __forceinline__ void store(lds_t<T> *lds, int row0 = 0, int L = 0, int wa = W) const {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int p = (int)threadIdx.x + i * NT;
            const int row = p / PPR, cp = p % PPR;
            if (P % NT != 0 && p >= P) continue;
            i32x4 x = v[i];
            if constexpr (PHI) {
                constexpr int n = 16 / (int)sizeof(T);
                typedef T tn __attribute__((__vector_size__(16)));
                tn e = __builtin_bit_cast(tn, x);
#pragma unroll
                for (int j = 0; j < n; ++j) e[j] = (T)phi((float)e[j]);
                x = __builtin_bit_cast(i32x4, e);
                // rows at or past L and padding columns were loaded as zero,
                // and phi(0) = 1: such a piece is zeroed again, a select per
                // 32-bit word rather than a branch
                const bool keep = row0 + RM::map(row) < L && cp * VEC < wa;
#pragma unroll
                for (int d = 0; d < 4; ++d) x[d] = keep ? x[d] : 0;
            }
            if constexpr (std::is_same<T, float>::value) {
                // the hi and lo halves of the four values
                F32S f = Ops<float>::cvt(__builtin_bit_cast(f32x4, x));
                bf16 *dst = lds + row * RS + cp * 4;
                *reinterpret_cast<bf16x4 *>(dst) = f.h;
                *reinterpret_cast<bf16x4 *>(dst + W) = f.l;
            } else {
                *reinterpret_cast<i32x4 *>(lds + row * RS + cp * (16 / (int)sizeof(T))) = x;
            }
        }
    }
};

// The normalised form's extra inputs of one slice: the forward's output and
// denominators (the backward turns dO into dn = dO / den and dd = -(dO . out)
// / den while staging it), the final normaliser z_{L-1} (optional) and the
// initial one z_{-1} (optional).
template <typename T> struct NormIn {
    const T *o;
    const float *den;
    const float *zf, *z0;
};

// The dn rows of a staged dO chunk and their dd: the pieces of dO and of the
// forward's output (same layout), and the denominators of the pieces' rows
// (zero past the sequence).  The PPR lanes of a row (consecutive lanes of one
// wave) reduce dO . out across the row; dd goes to dds[row], dn to the LDS
// copy.
template <typename T, typename SG>
__device__ __forceinline__ void store_dn(const SG &g, const SG &o, const float (&den)[SG::NP], lds_t<T> *Gs,
                                         float *dds) {
    constexpr int VEC = 16 / (int)sizeof(T), PPR = SG::PPR, NT = SG::NT_;
    static_assert(NT % PPR == 0 && 64 % PPR == 0, "a row's pieces lie in one wave");
    typedef T tv __attribute__((__vector_size__(16)));
    SG dn = g;
#pragma unroll
    for (int i = 0; i < SG::NP; ++i) {
        const int p = (int)threadIdx.x + i * NT;
        const tv gv = __builtin_bit_cast(tv, g.v[i]), ov = __builtin_bit_cast(tv, o.v[i]);
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc += (float)gv[j] * (float)ov[j];
#pragma unroll
        for (int x = PPR / 2; x >= 1; x >>= 1) acc += __shfl_xor(acc, x, PPR);
        const float inv = den[i] != 0.f ? 1.f / den[i] : 0.f;
        tv nv;
#pragma unroll
        for (int j = 0; j < VEC; ++j) nv[j] = (T)((float)gv[j] * inv);
        dn.v[i] = __builtin_bit_cast(i32x4, nv);
        if (p % PPR == 0 && (SG::P % NT == 0 || p < SG::P)) dds[p / PPR] = -acc * inv;
    }
    dn.store(Gs);
}

// Causal masks of a diagonal 16x16 tile.  Lane (g, r) holds rows 4g + t of
// column r; the keep-predicates depend on the lane only and are computed once.
struct Diag {
    bool keys_rows[4];   // layout D[j][i] (rows = keys, columns = queries): keep j <= i
    bool query_rows[4];  // layout D[i][j] (rows = queries, columns = keys): keep j <= i
    __device__ __forceinline__ Diag() {
        const int g = lane_g(), r = lane_r();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            keys_rows[t] = 4 * g + t <= r;
            query_rows[t] = r <= 4 * g + t;
        }
    }
    __device__ __forceinline__ f32x4 keys(f32x4 a) const {
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = keys_rows[t] ? a[t] : 0.f;
        return a;
    }
    __device__ __forceinline__ f32x4 query(f32x4 a) const {
#pragma unroll
        for (int t = 0; t < 4; ++t) a[t] = query_rows[t] ? a[t] : 0.f;
        return a;
    }
};

// Operands contracted over the feature index e (E columns of Q or K rows).
// A k-step is one MFMA's worth of features: bf16 with E >= 32 takes 32 per
// step as 8 consecutive elements per lane (one 16-byte LDS read), bf16 with
// E = 16 takes 16 (four per lane, padded with zeros), fp32 takes 16 (four per
// lane, four MFMAs).  Lane (g, r) of step s holds features
//     e = col0(s) + estride * g + v,   v < 8 (bf16, E >= 32) or v < 4.
// Carried states S (E x 16 column block) are kept as E/16 accumulator tiles
// whose rows follow the same order: tile eb holds, in lane (g, r), rows
//     e = ecol(eb) + estride * g + t,   t = 0..3,
// so the tiles of step s, converted, are directly that step's operand.  The
// transposed read tr_e() produces the matching K^T fragments for updating
// those tiles.
template <typename T, int E> struct EOps;

template <typename H, int E> struct EOps16 {
    static constexpr bool SPLIT_STATE = true;  // states enter as hi + lo bf16 pairs where accuracy needs it
    static constexpr int EB = E / 16;
    static constexpr bool WIDE = EB >= 2;
    static constexpr int STEPS = WIDE ? EB / 2 : 1;
    static constexpr int estride = WIDE ? 8 : 4;
    using x4 = typename Half16<H>::x4;
    using rf = typename std::conditional<WIDE, typename Half16<H>::x8, x4>::type;

    __device__ static __forceinline__ int ecol(int eb) { return WIDE ? 32 * (eb >> 1) + 4 * (eb & 1) : 16 * eb; }
    __device__ static __forceinline__ rf zero_rf() {
        rf z;
#pragma unroll
        for (int i = 0; i < (int)(sizeof(rf) / sizeof(H)); ++i) z[i] = (H)0.f;
        return z;
    }
    // lane (g, r) <- X[16 rb + r][features of step s]
    __device__ static __forceinline__ rf load(const H *lds, int rs, int rb, int s) {
        const H *p = lds + (16 * rb + lane_r()) * rs + (WIDE ? 32 * s : 0) + estride * lane_g();
        return *reinterpret_cast<const rf *>(p);
    }
    __device__ static __forceinline__ void mma(f32x4 &acc, rf a, rf b) {
        if constexpr (WIDE) {
            acc = Half16<H>::mfma(a, b, acc);
        } else {
            Ops16<H>::mma1(acc, a, b);
        }
    }
    // operand of step s from the state tiles
    __device__ static __forceinline__ rf state(const f32x4 *tiles, int s) {
        if constexpr (WIDE) {
            const x4 lo = Ops16<H>::cvt(tiles[2 * s]), hi = Ops16<H>::cvt(tiles[2 * s + 1]);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            return Ops16<H>::cvt(tiles[0]);
        }
    }
    __device__ static __forceinline__ void state_split(const f32x4 *tiles, int s, rf &hi, rf &lo) {
        if constexpr (WIDE) {
            x4 h0, l0, h1, l1;
            Ops16<H>::split(tiles[2 * s], h0, l0);
            Ops16<H>::split(tiles[2 * s + 1], h1, l1);
            hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
            lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            Ops16<H>::split(tiles[0], hi, lo);
        }
    }
    // lane (g, r) <- X[16 tb + 4g + t][ecol(eb) + estride * (r / 4) + r % 4]:
    // K^T fragment (rows e in state-tile order, k = tokens of block tb).
    __device__ static __forceinline__ x4 tr_e(const H *lds, int rs, int tb, int eb) {
        const int g = lane_g(), i = lane_r();
        const H *p = lds + (16 * tb + 4 * g + (i >> 2)) * rs + ecol(eb) + estride * (i & 3);
        s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)((__attribute__((address_space(3))) char *)(p)));
        return __builtin_bit_cast(x4, v);
    }
};
template <int E> struct EOps<bf16, E> : EOps16<bf16, E> {};
template <int E> struct EOps<f16, E> : EOps16<f16, E> {};

// fp32: the same feature order as the 16-bit operands, each a hi + lo pair.
template <int E> struct EOps<float, E> {
    using B = EOps16<bf16, E>;
    static constexpr int EB = B::EB;
    static constexpr bool WIDE = B::WIDE;
    static constexpr int STEPS = B::STEPS;
    static constexpr int estride = B::estride;
    // fp32 states enter the products as one split operand
    static constexpr bool SPLIT_STATE = false;
    struct rf {
        typename B::rf h, l;
    };

    __device__ static __forceinline__ int ecol(int eb) { return B::ecol(eb); }
    __device__ static __forceinline__ rf load(const bf16 *lds, int rs, int rb, int s) {
        return {B::load(lds, rs, rb, s), B::load(lds + lo_half(rs), rs, rb, s)};
    }
    __device__ static __forceinline__ void mma(f32x4 &acc, rf x, rf y) {
        B::mma(acc, x.l, y.h);
        B::mma(acc, x.h, y.l);
        B::mma(acc, x.h, y.h);
    }
    __device__ static __forceinline__ rf state(const f32x4 *tiles, int s) {
        rf x;
        B::state_split(tiles, s, x.h, x.l);
        return x;
    }
    __device__ static __forceinline__ void state_split(const f32x4 *tiles, int s, rf &hi, rf &lo) {
        hi = state(tiles, s);
        lo.h = B::zero_rf();
        lo.l = B::zero_rf();
    }
    __device__ static __forceinline__ F32S tr_e(const bf16 *lds, int rs, int tb, int eb) {
        return {B::tr_e(lds, rs, tb, eb), B::tr_e(lds + lo_half(rs), rs, tb, eb)};
    }
};

// Query row blocks of a chunk of CB row blocks owned by row set h of RS:
// where the chunk holds whole pairs for every set, the blocks are taken in
// balanced pairs (k, CB-1-k) -- equal causal work -- dealt round robin to the
// row sets; otherwise block I goes to set I % RS.
template <int CB, int RS>
constexpr bool owns_block(int h, int I) {
    if constexpr (RS == 1) {
        return true;
    } else if constexpr (CB % (2 * RS) == 0) {
        const int k = I < CB / 2 ? I : CB - 1 - I;
        return k % RS == h;
    } else {
        return I % RS == h;
    }
}
template <int CB, int RS>
constexpr int last_block(int h) {
    int last = -1;
    for (int I = 0; I < CB; ++I)
        if (owns_block<CB, RS>(h, I)) last = I;
    return last;
}

// The k-th row block (k from 0) of a chunk's CB that row group h of RG owns
// (owns_block), the position of block j among them, and how many it owns.
template <int CB, int RG>
constexpr int owned_block(int h, int k) {
    for (int I = 0; I < CB; ++I)
        if (owns_block<CB, RG>(h, I) && k-- == 0) return I;
    return -1;
}
template <int CB, int RG>
constexpr int owned_index(int h, int j) {
    int k = 0;
    for (int I = 0; I < j; ++I) k += owns_block<CB, RG>(h, I) ? 1 : 0;
    return k;
}
template <int CB, int RG>
constexpr int owned_count(int h) {
    return owned_index<CB, RG>(h, CB);
}

// Stage row map of the row blocks that row set H of RS owns, in order:
// staged row r is chunk row 16 owned_block(H, r / 16) + r % 16.
template <int CB, int RS, int H>
struct OwnedRows {
    __device__ static int map(int r) {
        const int j = r >> 4;
        int b = 0;
#pragma unroll
        for (int k = 0; k < owned_count<CB, RS>(H); ++k) b = j == k ? owned_block<CB, RS>(H, k) : b;
        return 16 * b + (r & 15);
    }
};

// The increment slots of a call over sequence segments made cumulative, in
// place, so that each sweep reads one slot per carried state instead of
// summing a run of them: per slice (nslot slots of E*M + E floats), ws1 (the
// prefix state's increments) becomes inclusive suffix sums over slots
// [lo1, nslot) when the sweeps start from the final state (suffix1), else
// inclusive prefix sums over [0, hi1); with a second job (ws2, the
// backward's suffix state's increments) inclusive suffix sums over
// [lo2, nslot).  One thread per 16-byte piece of a slice's increment and per
// job.
template <int E, int M>
__global__ __launch_bounds__(256) void cp_seg_scan_kernel(float *__restrict__ ws1, float *__restrict__ ws2, int NS,
                                                          int nslot, int lo1, int hi1, int suffix1, int lo2) {
    constexpr int WS = E * M + E, NP = WS / 4;
    static_assert(WS % 4 == 0, "whole 16-byte pieces");
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (ws2 ? 2 : 1) * (int64_t)NS * NP) return;
    const bool second = t >= (int64_t)NS * NP;
    const int64_t q = second ? t - (int64_t)NS * NP : t;
    const int slice = (int)(q / NP), p = (int)(q % NP);
    f32x4 *x = reinterpret_cast<f32x4 *>((second ? ws2 : ws1) + (int64_t)slice * nslot * WS) + p;
    // slots [lo, hi) in scan order (downwards for suffix sums), eight at a
    // time: the eight loads are issued together, then summed and stored
    const bool down = second || suffix1;
    const int lo = down ? (second ? lo2 : lo1) : 0, hi = down ? nslot : hi1;
    f32x4 acc = zero4();
    for (int b = 0; b < hi - lo; b += 8) {
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = down ? hi - 1 - (b + i) : lo + b + i;
            v[i] = b + i < hi - lo ? x[(int64_t)s * NP] : zero4();
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = down ? hi - 1 - (b + i) : lo + b + i;
            acc += v[i];
            if (b + i < hi - lo) x[(int64_t)s * NP] = acc;
        }
    }
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



}  // namespace cp
