// cp_tune.hpp -- compile-time launch parameters of each kernel instance:
// chunk length C (tokens per step of the scan), NBUF (register buffers of
// the load pipeline: NBUF-1 chunks are in flight while one is computed) and
// HILO (carried states enter the bf16 MFMA as a hi + lo pair of bf16 values,
// 16 significant bits instead of 8).  Each value can be overridden when the
// library is built (-DCP_BF16_C=64 ...) for tuning sweeps.
#pragma once

#ifndef CP_BF16_C
#define CP_BF16_C 32
#endif
#ifndef CP_BF16_NBUF
#define CP_BF16_NBUF 2
#endif
#ifndef CP_BF16_HILO
#define CP_BF16_HILO 1
#endif
#ifndef CP_F32_C
#define CP_F32_C 32
#endif
#ifndef CP_F32_C_WIDE
#define CP_F32_C_WIDE 16
#endif
#ifndef CP_F32_NBUF
#define CP_F32_NBUF 2
#endif

namespace cp {

template <typename T, int E, int M> struct Tune;

template <int E, int M> struct Tune<__bf16, E, M> {
    static constexpr int C = CP_BF16_C;
    static constexpr int NBUF = CP_BF16_NBUF;
    static constexpr bool HILO = CP_BF16_HILO != 0;
};

template <int E, int M> struct Tune<float, E, M> {
    static constexpr int C = (E > 64 || M > 64) ? CP_F32_C_WIDE : CP_F32_C;
    static constexpr int NBUF = CP_F32_NBUF;
    static constexpr bool HILO = false;
};

}  // namespace cp
