// cp_tune.hpp -- compile-time launch parameters of each kernel instance:
// chunk length C (tokens per step of the scan), NBUF (register buffers of
// the load pipeline: NBUF-1 chunks are in flight while one is computed) and
// HILO (carried states enter the bf16 MFMA as a hi + lo pair of bf16 values,
// 16 significant bits instead of 8).
#pragma once

namespace cp {

template <typename T, int E, int M> struct Tune;

template <int E, int M> struct Tune<__bf16, E, M> {
    static constexpr int C = 32;
    static constexpr int NBUF = 2;
    static constexpr bool HILO = true;
};

template <int E, int M> struct Tune<float, E, M> {
    static constexpr int C = (E > 64 || M > 64) ? 16 : 32;
    static constexpr int NBUF = 2;
    static constexpr bool HILO = false;
};

}  // namespace cp
