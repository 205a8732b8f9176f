// Device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace tq {

typedef int8_t i8x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer resources (raw, untyped access): the fourth descriptor dword, whose data-format
// field must be non-zero (32-bit) on gfx9 parts. Accesses past the byte range are dropped.
constexpr int BUF_DWORD3 = 0x00020000;
// cache-policy bits of a memory instruction on gfx950: sc0, nt, sc1
constexpr int CPOL_SC0 = 1, CPOL_NT = 2, CPOL_SC1 = 16;

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

// Stored norms: float32, or the bits of an IEEE binary16 value (the 16-bit norm format;
// v_cvt_f16_f32 rounds to nearest even, the widening back is exact).
__device__ __forceinline__ float norm_f32(float v) { return v; }
__device__ __forceinline__ float norm_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_binary16(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }

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

// ---- cross-lane reductions on the VALU (DPP and gfx950 row swaps; no LDS round trip) ----
// DPP controls: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2), and the
// rotations by 4 and 8 lanes inside each row of 16.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp_mov_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_mov_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// x[lane] and x[lane ^ 16] (ROWS = 16) or x[lane ^ 32] (ROWS = 32), as the two outputs of a
// row swap (which output holds which depends only on the lane, the same for both halves of a
// 64-bit value)
template <int ROWS>
__device__ __forceinline__ void swap_pair(uint32_t x, uint32_t &a, uint32_t &b) {
    if constexpr (ROWS == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        a = p[0], b = p[1];
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        a = p[0], b = p[1];
    }
}
template <int ROWS>
__device__ __forceinline__ float rows_max_f32(float x) {
    uint32_t a, b;
    swap_pair<ROWS>(__float_as_uint(x), a, b);
    return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
template <int ROWS>
__device__ __forceinline__ float rows_sum_f32(float x) {
    uint32_t a, b;
    swap_pair<ROWS>(__float_as_uint(x), a, b);
    return __uint_as_float(a) + __uint_as_float(b);
}
template <int ROWS>
__device__ __forceinline__ double rows_sum_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    uint32_t a0, b0, a1, b1;
    swap_pair<ROWS>((uint32_t)u, a0, b0);
    swap_pair<ROWS>((uint32_t)(u >> 32), a1, b1);
    return __builtin_bit_cast(double, ((uint64_t)a1 << 32) | a0) + __builtin_bit_cast(double, ((uint64_t)b1 << 32) | b0);
}
// Sum over consecutive groups of N lanes (N a power of two, at most 64), by a fixed pairwise
// tree (lane ^ 1, lane ^ 2, mirrors inside half-rows and rows, row swaps): every lane of a
// group ends with the same value, the one a lane ^ 1, ^ 2, ^ 4, ... butterfly gives.
template <int N>
__device__ __forceinline__ float group_sum_f32(float x) {
    if constexpr (N >= 2) x += dpp_mov_f32<DPP_XOR1>(x);
    if constexpr (N >= 4) x += dpp_mov_f32<DPP_XOR2>(x);
    if constexpr (N >= 8) x += dpp_mov_f32<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp_mov_f32<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x = rows_sum_f32<16>(x);
    if constexpr (N >= 64) x = rows_sum_f32<32>(x);
    return x;
}
// Max and fp64 sum over the lanes congruent to this one modulo S (S a power of two below 64)
// across the wave; lane 0 (and, for the max, every lane) holds the full result.
template <int S>
__device__ __forceinline__ float stride_max_f32(float x) {
    if constexpr (S <= 8) x = fmaxf(x, dpp_mov_f32<0x120 + 8>(x));
    if constexpr (S <= 4) x = fmaxf(x, dpp_mov_f32<0x120 + 4>(x));
    if constexpr (S <= 2) x = fmaxf(x, dpp_mov_f32<0x120 + 2>(x));
    if constexpr (S <= 1) x = fmaxf(x, dpp_mov_f32<0x120 + 1>(x));
    if constexpr (S <= 16) x = rows_max_f32<16>(x);
    return rows_max_f32<32>(x);
}
template <int S>
__device__ __forceinline__ double stride_sum_f64(double x) {
    if constexpr (S <= 8) x += dpp_mov_f64<0x120 + 8>(x);
    if constexpr (S <= 4) x += dpp_mov_f64<0x120 + 4>(x);
    if constexpr (S <= 2) x += dpp_mov_f64<0x120 + 2>(x);
    if constexpr (S <= 1) x += dpp_mov_f64<0x120 + 1>(x);
    if constexpr (S <= 16) x = rows_sum_f64<16>(x);
    return rows_sum_f64<32>(x);
}
// Over the lanes that share lane % 4 inside each row of 16 (4 lanes): every one of them ends
// with the same result.
__device__ __forceinline__ float quad_stride_max_f32(float x) {
    x = fmaxf(x, dpp_mov_f32<DPP_ROR8>(x));
    return fmaxf(x, dpp_mov_f32<DPP_ROR4>(x));
}
__device__ __forceinline__ double quad_stride_sum_f64(double x) {
    x += dpp_mov_f64<DPP_ROR8>(x);
    return x + dpp_mov_f64<DPP_ROR4>(x);
}
// Over the whole wave; every lane ends with the same result.
__device__ __forceinline__ float dpp_wave_max_f32(float x) {
    x = fmaxf(x, dpp_mov_f32<DPP_XOR1>(x));
    x = fmaxf(x, dpp_mov_f32<DPP_XOR2>(x));
    x = quad_stride_max_f32(x);
    return rows_max_f32<32>(rows_max_f32<16>(x));
}
__device__ __forceinline__ double dpp_wave_sum_f64(double x) {
    x += dpp_mov_f64<DPP_XOR1>(x);
    x += dpp_mov_f64<DPP_XOR2>(x);
    x = quad_stride_sum_f64(x);
    return rows_sum_f64<32>(rows_sum_f64<16>(x));
}

// Estimator scale constants of one call, passed by value.
struct ScoreScale {
    double inv_sqrt_d[2];  // 1/sqrt(d_g)
    double qjl;            // sqrt(pi/2)/m
};

}  // namespace tq
