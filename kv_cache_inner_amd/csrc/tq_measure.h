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

// The same logits for d = 128 and G <= 4, streaming: every wave load instruction reads
// 1 KiB of consecutive key bytes (two keys; lane l holds channels 4(l % 32) .. 4(l % 32) + 3
// of key l / 32), the lane's 4 x G query values stay in registers, and each lane forms 4G
// partial sums per load. After the 8 loads of a 16-key tile a lane holds 8 keys x 4 queries
// = 32 partials; five exchange-and-halve steps over the 32 lanes of each half-wave (lane
// pairs at distance 1, 2 inside quads, mirrored inside 8 and 16 lanes, then the two rows)
// leave each lane with the full sum of one (key, query). Tiles are double-buffered in
// registers, so the next tile's loads are in flight while one is reduced.
constexpr int F32L_WAVES = 8;

// one exchange-and-halve step: x[0..N) -> x[0..N/2), keeping the half this lane owns
template <int N, int CTRL>
__device__ __forceinline__ void fold_dpp(float (&x)[32], bool upper) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = upper ? x[i] : x[i + N / 2];
        const float keep = upper ? x[i + N / 2] : x[i];
        x[i] = keep + dpp_mov_f32<CTRL>(send);
    }
}
template <int N>
__device__ __forceinline__ void fold_rows(float (&x)[32], bool upper) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = upper ? x[i] : x[i + N / 2];
        const float keep = upper ? x[i + N / 2] : x[i];
        uint32_t a, b;
        swap_pair<16>(__float_as_uint(send), a, b);
        // the row swap returns this lane's own value in one output and the partner's in the
        // other; which is which depends on the row
        x[i] = keep + __uint_as_float(upper ? a : b);
    }
}

__global__ __launch_bounds__(F32L_WAVES * 64) void fp32_logits_stream_kernel(
    const float *__restrict__ keys, long banks, long n, const float *__restrict__ q, int G,
    float *__restrict__ scores, int n_tiles, int tiles_per_wave, int waves_per_bank) {
    const int lane = threadIdx.x & 63, h = lane >> 5, c4 = lane & 31;
    const long wave = (long)blockIdx.x * F32L_WAVES + (threadIdx.x >> 6);
    const long bank = wave / waves_per_bank;
    const int t0 = (int)(wave % waves_per_bank) * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, n_tiles);
    if (bank >= banks || t0 >= t1) return;  // the grid's last work-group may run past the last bank
    f32x4 qv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
        qv[g] = g < G ? *reinterpret_cast<const f32x4 *>(q + ((size_t)bank * G + g) * 128 + 4 * c4) : f32x4{0, 0, 0, 0};
    const float *kb = keys + (size_t)bank * n * 128;
    const long last = n * 32 - 1;  // last float4 of the bank (clamped loads past n are discarded)
    auto load = [&](f32x4 (&v)[8], int t) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const long e = min((long)t * 512 + r * 64 + lane, last);
            v[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(kb) + e);
        }
    };
    // one tile: lane (h, c4) ends with the sum of partial index c4 = 4 r + g, i.e. key 2 r + h
    // of the tile against query g (each fold keeps the upper half on the lanes whose bit is
    // set, so the kept index is 16 b4 + 8 b3 + 4 b2 + 2 b1 + b0 = c4)
    auto reduce_store = [&](const f32x4 (&v)[8], int t) {
        float x[32];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float s = v[r][0] * qv[g][0];
                s = fmaf(v[r][1], qv[g][1], s);
                s = fmaf(v[r][2], qv[g][2], s);
                x[4 * r + g] = fmaf(v[r][3], qv[g][3], s);
            }
        fold_rows<32>(x, (c4 & 16) != 0);            // partner: lane ^ 16 (row swap)
        fold_dpp<16, 0x140>(x, (c4 & 8) != 0);       // partner: mirror inside the row of 16
        fold_dpp<8, 0x141>(x, (c4 & 4) != 0);        // partner: mirror inside the half-row
        fold_dpp<4, DPP_XOR2>(x, (c4 & 2) != 0);     // partner: lane ^ 2
        fold_dpp<2, DPP_XOR1>(x, (c4 & 1) != 0);     // partner: lane ^ 1
        const int r = c4 >> 2, g = c4 & 3;
        const long key = (long)t * 16 + 2 * r + h;
        if (g < G && key < n) scores[((size_t)bank * G + g) * n + key] = x[0];
    };
    f32x4 A[8], B[8];
    load(A, t0);
    for (int t = t0; t < t1; t += 2) {
        if (t + 1 < t1) load(B, t + 1);
        reduce_store(A, t);
        if (t + 1 >= t1) break;
        if (t + 2 < t1) load(A, t + 2);
        reduce_store(B, t + 1);
    }
}

inline int launch_fp32_logits(const float *keys, int64_t banks, int64_t n, int32_t d, const float *q, int32_t G,
                              float *scores, hipStream_t st) {
    if (d == 128 && G <= 4 && ((uintptr_t)keys & 15) == 0 && ((uintptr_t)q & 15) == 0) {
        const int64_t n_tiles = (n + 15) / 16;
        // about 16 waves per compute unit over the whole launch
        int64_t wpb = (256 * 16 + banks - 1) / banks;
        if (wpb > n_tiles) wpb = n_tiles;
        const int64_t tpw = (n_tiles + wpb - 1) / wpb;
        wpb = (n_tiles + tpw - 1) / tpw;
        const int64_t waves = banks * wpb;
        if ((waves + F32L_WAVES - 1) / F32L_WAVES > INT32_MAX || n_tiles > INT32_MAX) return 1;
        hipLaunchKernelGGL(fp32_logits_stream_kernel, dim3((unsigned)((waves + F32L_WAVES - 1) / F32L_WAVES)),
                           dim3(F32L_WAVES * 64), 0, st, keys, (long)banks, (long)n, q, (int)G, scores, (int)n_tiles,
                           (int)tpw, (int)wpb);
        return hipGetLastError() != hipSuccess;
    }
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
