// Device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tq {

typedef int8_t i8x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Compile-time loop: calls f(std::integral_constant<int, I>) for I = 0..N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Work-group barrier over LDS traffic only: it waits for this wave's LDS operations but not
// for its vector-memory loads, so loads issued earlier (direct-to-LDS or into registers)
// stay in flight (a __syncthreads() would drain them all). Only for code whose cross-wave
// communication goes through ordinary LDS reads and writes.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Estimator scale constants of one call, passed by value.
struct ScoreScale {
    double inv_sqrt_d[2];  // 1/sqrt(d_g)
    double qjl;            // sqrt(pi/2)/m
};

}  // namespace tq
