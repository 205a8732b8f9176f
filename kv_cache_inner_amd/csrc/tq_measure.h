// Measurement kernels: fp32 logits against unquantized keys (the 32-bit-key baseline
// that the tambur.pub article compares 4-bit TurboQuant keys with) and a device copy
// (achievable HBM bandwidth; calibration of the traffic counters).
#pragma once
#include "tq_device.h"

namespace tq {

// scores[b][g][i] = sum_c q[b][g][c] * keys[b][i][c]. A work-group stages TK keys in LDS
// with 16-byte coalesced loads, then each thread takes one (key, query) pair at a time.
template <int TK>
__global__ __launch_bounds__(256) void fp32_logits_kernel(const float *__restrict__ keys, long n, int d,
                                                          const float *__restrict__ q, int G,
                                                          float *__restrict__ scores, int tiles) {
    extern __shared__ __align__(16) float lds[];
    const int ld = d + 1;
    float *K = lds;            // [TK][d+1]
    float *Q = lds + TK * ld;  // [G][d]
    const long bank = blockIdx.x / tiles;
    const int tile = blockIdx.x % tiles, tid = threadIdx.x;
    const long key0 = (long)tile * TK;
    const float *kb = keys + ((size_t)bank * n + key0) * d;
    const int nvec = TK * d / 4;
    for (int e = tid; e < nvec; e += 256) {
        const int i = (4 * e) / d, c = (4 * e) % d;
        f32x4 v = {0, 0, 0, 0};
        if (key0 + i < n) v = *reinterpret_cast<const f32x4 *>(kb + (size_t)i * d + c);
        K[i * ld + c + 0] = v[0];
        K[i * ld + c + 1] = v[1];
        K[i * ld + c + 2] = v[2];
        K[i * ld + c + 3] = v[3];
    }
    const float *qb = q + (size_t)bank * G * d;
    for (int e = tid; e < G * d; e += 256) Q[e] = qb[e];
    __syncthreads();
    for (int pair = tid; pair < TK * G; pair += 256) {
        const int i = pair % TK, g = pair / TK;
        const float *kr = K + i * ld, *qr = Q + g * d;
        float s = 0.0f;
        for (int c = 0; c < d; ++c) s = fmaf(kr[c], qr[c], s);
        if (key0 + i < n) scores[((size_t)bank * G + g) * n + key0 + i] = s;
    }
}

inline int launch_fp32_logits(const float *keys, int64_t banks, int64_t n, int32_t d, const float *q, int32_t G,
                              float *scores, hipStream_t st) {
    constexpr int TK = 64;
    const int64_t tiles = (n + TK - 1) / TK;
    if (banks * tiles > INT32_MAX) return 1;
    const size_t smem = (size_t)(TK * (d + 1) + G * d) * 4;
    (void)hipFuncSetAttribute((const void *)fp32_logits_kernel<TK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL(fp32_logits_kernel<TK>, dim3((unsigned)(banks * tiles)), dim3(256), smem, st, keys, (long)n,
                       (int)d, q, (int)G, scores, (int)tiles);
    return hipGetLastError() != hipSuccess;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t nvec) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) dst[i] = src[i];
}

inline int launch_copy(const void *src, void *dst, size_t bytes, hipStream_t st) {
    const size_t nvec = bytes / 16;
    size_t blocks = (nvec + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4 *)src, (u32x4 *)dst, nvec);
    return hipGetLastError() != hipSuccess;
}

}  // namespace tq
