// cp_bwd_launch.hpp -- host side of the backward launches (causal product and
// normalised form), shared by the bf16, fp16 and fp32 translation units.
#pragma once

#include <algorithm>

#include "cp_bwd.hpp"
#include "cp_launch.hpp"
#include "cp_tune.hpp"

namespace cp {

// Per-chunk terms of the backward of the normalised form out_i = n_i / d_i,
// for chunk c (rows cC .. cC+C-1) of one slice:
//     dn_i = dO_i / d_i              (stored in the I/O type, like dO)
//     dd_i = -(dO_i . out_i) / d_i   (= -(dO_i . n_i) / d_i^2; fp32)
//     cs_c = sum over the chunk's rows of phi(k_i)   (fp32)
// Rows are read and dn written in 16-byte pieces: TPM lanes per row of dO
// (M, the tile width, of them; lanes past the head's Ma columns idle), the
// dot product reduced across them; dd has zeros in rows L .. Lpad-1.  The
// column sums read K the same way, TPR lanes per row, and apply phi rounded
// to the I/O type, as the sweeps see it; the sums of padding columns (past
// Ea) are zero.
template <typename T, int E, int M, int C, bool FMAP>
__device__ __forceinline__ void lin_prep_chunk(const T *dO, const T *Out, const T *K, const float *den, T *dn,
                                               float *dd, float *cs, int c, int L, float (*red)[E + 1], int Ea,
                                               int Ma) {
    constexpr int VEC = 16 / sizeof(T), TPM = M / VEC, RPM = 256 / TPM, TPR = E / VEC, P = 256 / TPR;
    typedef T tv __attribute__((__vector_size__(16)));
    const int t = threadIdx.x;
    {
        const int cm = t % TPM, pr = t / TPM;
        const bool mv = cm * VEC < Ma;
#pragma unroll
        for (int ii = pr; ii < C; ii += RPM) {
            const int i = c * C + ii;
            const bool live = i < L && mv;
            const float d = i < L ? den[i] : 1.f;
            float acc = 0.f;
            if (live) {
                const int64_t off = (int64_t)i * Ma + cm * VEC;
                const tv gv = *reinterpret_cast<const tv *>(dO + off);
                const tv ov = *reinterpret_cast<const tv *>(Out + off);
                tv nv;
#pragma unroll
                for (int j = 0; j < VEC; ++j) {
                    acc += (float)gv[j] * (float)ov[j];
                    nv[j] = (T)((float)gv[j] / d);
                }
                *reinterpret_cast<tv *>(dn + off) = nv;
            }
#pragma unroll
            for (int x = TPM / 2; x >= 1; x >>= 1) acc += __shfl_xor(acc, x, TPM);
            if (cm == 0) dd[i] = i < L ? -acc / d : 0.f;
        }
    }
    const int cg = t % TPR, p = t / TPR;
    const bool ev = cg * VEC < Ea;
    float acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = 0.f;
    if (ev) {
        for (int i = c * C + p; i < (c + 1) * C && i < L; i += P) {
            const tv x = *reinterpret_cast<const tv *>(K + (int64_t)i * Ea + cg * VEC);
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] += FMAP ? (float)(T)phi((float)x[j]) : (float)x[j];
        }
    }
#pragma unroll
    for (int j = 0; j < VEC; ++j) red[p][cg * VEC + j] = acc[j];
    __syncthreads();
    if (t < E) {
        float sum = 0.f;
        for (int q = 0; q < P; ++q) sum += red[q][t];
        cs[(int64_t)c * E + t] = sum;
    }
    __syncthreads();  // red is rewritten by the next chunk
}

// One workgroup per (slice, chunk), grid-strided.  dd is [NS][Lpad], cs
// [NS][Lpad / C][E].
template <typename T, int E, int M, int C, bool FMAP>
__global__ __launch_bounds__(256) void cp_lin_prep_kernel(const T *__restrict__ dO, const T *__restrict__ Out,
                                                          const T *__restrict__ K, const float *__restrict__ den,
                                                          T *__restrict__ dn, float *__restrict__ dd,
                                                          float *__restrict__ cs, int L, int Lpad, int NS, int Ea,
                                                          int Ma) {
    constexpr int VEC = 16 / sizeof(T), TPR = E / VEC, P = 256 / TPR, TPM = M / VEC;
    static_assert(E % VEC == 0 && 256 % TPR == 0 && M % VEC == 0 && TPM <= 64 && 256 % TPM == 0 && C % 16 == 0,
                  "prep layout");
    __shared__ float red[P][E + 1];
    const int nch = Lpad / C;
    for (int64_t blk = blockIdx.x; blk < (int64_t)nch * NS; blk += gridDim.x) {
        const int64_t sl = blk / nch;
        lin_prep_chunk<T, E, M, C, FMAP>(dO + sl * L * Ma, Out + sl * L * Ma, K + sl * L * Ea, den + sl * L,
                                         dn + sl * L * Ma, dd + sl * Lpad, cs + sl * nch * E, (int)(blk % nch), L,
                                         red, Ea, Ma);
    }
}

// Exclusive prefix over the chunk sums of one slice, in place (E columns
// including any padding; z_in holds Ea):
// zc_c = z_{-1} + sum of cs_c' for c' < c, the normaliser before chunk c,
// summed forward in fp32 (recovering early prefixes from the final z by
// subtraction would lose most of their bits).  Lane (p, e) scans a contiguous
// range of chunks; the range totals are combined through LDS.
template <int E>
__device__ __forceinline__ void lin_zscan_slice(const float *z_in, float *zc, int nch, float (*tot)[E], int Ea) {
    constexpr int P = 256 / E;
    const int e = threadIdx.x % E, p = threadIdx.x / E;
    const int c0 = (int)((int64_t)nch * p / P), c1 = (int)((int64_t)nch * (p + 1) / P);
    float *col = zc + e;
    // (the loads of both passes are independent of the running sum: unrolled
    // so that several are in flight)
    float sum = 0.f;
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += col[(int64_t)c * E];
    tot[p][e] = sum;
    __syncthreads();
    float z = z_in && e < Ea ? z_in[e] : 0.f;
    for (int q = 0; q < p; ++q) z += tot[q][e];
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
        const float x = col[(int64_t)c * E];
        col[(int64_t)c * E] = z;
        z += x;
    }
    __syncthreads();  // tot is rewritten by the next slice
}

// One workgroup per slice, grid-strided.
template <int E>
__global__ __launch_bounds__(256) void cp_lin_zscan_kernel(const float *__restrict__ z_in, float *__restrict__ zc,
                                                           int nch, int NS, int Ea) {
    __shared__ float tot[256 / E][E];
    for (int64_t sl = blockIdx.x; sl < NS; sl += gridDim.x)
        lin_zscan_slice<E>(z_in ? z_in + sl * Ea : nullptr, zc + sl * nch * E, nch, tot, Ea);
}

template <typename T, int E, int M, bool NORM, bool FMAP>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
    using P = Tune<T, E, M>;
    constexpr int C = P::BC;
    const T *q = static_cast<const T *>(a.Q), *k = static_cast<const T *>(a.K), *v = static_cast<const T *>(a.V),
            *g = static_cast<const T *>(a.G);
    const float *s0 = a.state_in, *st = a.state_final;
    T *dq = static_cast<T *>(a.dQ), *dk = static_cast<T *>(a.dK), *dv = static_cast<T *>(a.dV);
    float *ds0 = a.dstate_in, *dz0 = a.dz_in;
    int L = a.L, NS = a.NS, Ea = a.Ea, Ma = a.Ma;
    int Lpad = (L + C - 1) / C * C;
    float *dd = nullptr, *zc = nullptr;
    void *scratch = nullptr;
    hipError_t e = hipSuccess;
    if constexpr (NORM) {
        // scratch: dn [NS][L][M] in the I/O type, dd [NS][Lpad] and zc [NS][Lpad / C][E] fp32
        const size_t dn_bytes = ((size_t)NS * L * M * sizeof(T) + 255) / 256 * 256;
        const size_t dd_bytes = ((size_t)NS * Lpad * sizeof(float) + 255) / 256 * 256;
        const size_t bytes = dn_bytes + dd_bytes + (size_t)NS * (Lpad / C) * E * sizeof(float);
        e = hipMallocAsync(&scratch, bytes, s);
        if (e != hipSuccess) return e;
        T *dn = static_cast<T *>(scratch);
        dd = reinterpret_cast<float *>(static_cast<char *>(scratch) + dn_bytes);
        zc = reinterpret_cast<float *>(static_cast<char *>(scratch) + dn_bytes + dd_bytes);
        const T *out = static_cast<const T *>(a.Out);
        const float *den = a.den;
        const float *z0 = a.z_in;
        int nch = Lpad / C;
        auto prep = cp_lin_prep_kernel<T, E, M, C, FMAP>;
        void *pargs[] = {&g, &out, &k, &den, &dn, &dd, &zc, &L, &Lpad, &NS, &Ea, &Ma};
        const int64_t blocks = std::min<int64_t>((int64_t)NS * nch, 1 << 20);
        e = launch_kernel(reinterpret_cast<const void *>(prep), dim3((unsigned)blocks), dim3(256), pargs, s);
        g = dn;  // the sweeps take dn in place of dO
        if (e == hipSuccess) {
            auto scan = cp_lin_zscan_kernel<E>;
            void *sargs[] = {&z0, &zc, &nch, &NS, &Ea};
            e = launch_kernel(reinterpret_cast<const void *>(scan), dim3((unsigned)std::min(NS, 1 << 20)), dim3(256),
                              sargs, s);
        }
    }
    if (e == hipSuccess) {
        auto kern = cp_bwd_kernel<T, E, M, C, P::BG, P::BNB, P::BIDLE, P::BRG, P::BNPF, NORM, FMAP>;
        void *args[] = {&q, &k, &v, &g, &s0, &st, &zc, &dd, &Lpad, &dq, &dk, &dv, &ds0, &dz0, &L, &NS, &Ea, &Ma};
        e = launch_kernel(reinterpret_cast<const void *>(kern), dim3(NS * P::BG * P::BRG),
                          dim3(64 * bwd_waves<E, M, P::BG, P::BNB, P::BIDLE>()),
                          args, s);
    }
    if (scratch) {
        const hipError_t f = hipFreeAsync(scratch, s);
        if (e == hipSuccess) e = f;
    }
    return e;
}

template <typename T, int E, int M, bool NORM>
hipError_t launch_bwd_fm(const BwdArgs &a, hipStream_t s) {
    if (NORM && a.fmap) return launch_bwd_t<T, E, M, NORM, true>(a, s);
    return launch_bwd_t<T, E, M, NORM, false>(a, s);
}

template <typename T, bool NORM>
bwd_fn pick_bwd(int E, int M) {
    static const bwd_fn table[4][4] = {
        {launch_bwd_fm<T, 16, 16, NORM>, launch_bwd_fm<T, 16, 32, NORM>, launch_bwd_fm<T, 16, 64, NORM>,
         launch_bwd_fm<T, 16, 128, NORM>},
        {launch_bwd_fm<T, 32, 16, NORM>, launch_bwd_fm<T, 32, 32, NORM>, launch_bwd_fm<T, 32, 64, NORM>,
         launch_bwd_fm<T, 32, 128, NORM>},
        {launch_bwd_fm<T, 64, 16, NORM>, launch_bwd_fm<T, 64, 32, NORM>, launch_bwd_fm<T, 64, 64, NORM>,
         launch_bwd_fm<T, 64, 128, NORM>},
        {launch_bwd_fm<T, 128, 16, NORM>, launch_bwd_fm<T, 128, 32, NORM>, launch_bwd_fm<T, 128, 64, NORM>,
         launch_bwd_fm<T, 128, 128, NORM>},
    };
    const int ie = tile_index(E), im = tile_index(M);
    return (ie < 0 || im < 0) ? nullptr : table[ie][im];
}

}  // namespace cp
