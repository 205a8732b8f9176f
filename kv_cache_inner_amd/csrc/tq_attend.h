// Decompression of stored vectors and decode attention over packed keys and values.
//
// turboquant-pytorch write-up (discuss.pytorch.kr), usage example and two-stage section: the
// MSE quantiser's decompression of one stored vector is, per channel group g,
//     x_hat_g = (nu_g / sqrt(d_g)) R_g^T c_g[idx_g],
// put back in channel order. In a decode step the keys (inner-product quantiser) give the
// logits through the estimator and the values (MSE quantiser) enter through x_hat; one
// query head's output is o = sum_i p_i x_hat_i with p = softmax(scale * logits). R_g^T is
// linear, so it leaves the sum:
//     o = P^T blockdiag(R_g)^T o_rot,  o_rot[j] = sum_i p_i (nu_{g,i} / sqrt(d_g)) c_g[idx_ij],
// and the kernels accumulate o_rot (rotated, group order) and rotate once per query.
//
// o_rot as an integer matrix product. For a symmetric codebook (c[L-1-k] = -c[k]) only the
// odd Walsh terms survive: with sign variables s_p = 2 b_p - 1 of the code bits b_p,
//     1 bit:  c = a0 s0;   2 bits: c = a0 s0 + a1 s1;   3 bits: c = a0 s0 + a1 s1 + a2 s2 + a3 s0 s1 s2,
// and s0 s1 s2 = 2 (b0 ^ b1 ^ b2) - 1. So c = sum_P 2 a_P B_P - sum_P a_P over bit planes B_P
// (the stored planes, plus their XOR for 3 bits). Then
//     sum_i w_i c[idx_ij] = sum_P 2 a_P (sum_i w_i B_P(i, j)) - (sum_P a_P) sum_i w_i,
// with w_i = e^(z_i - max) nu_i: each inner sum is weights times a 0/1 matrix. The weights are
// rounded to 30-bit fixed point per (chunk, query, group) and split into four signed 8-bit
// limbs; the bits enter v_mfma_i32_16x16x64_i8 as bytes {0, 2^t} (one shift t per product,
// 2^7 read as -128), so every product and sum is exact in int32 and the limbs recombine
// exactly. A 16-row operand holds 4 queries x 4 limbs; a 16-column operand holds one
// 32-coordinate word of the four planes (4 planes x 4 bytes), the shift t selecting the
// coordinate 8 * byte + t inside each byte.
#pragma once
#include "tq_device.h"

namespace tq {

constexpr int AT_THREADS = 256;                // four waves
constexpr int AT_STEP = 64;                    // keys per product: four 16-key tiles
constexpr int AT_CHUNK = 1024;                 // keys per work-group
constexpr int AT_STEPS = AT_CHUNK / AT_STEP;
constexpr int AT_DMAX = 128;                   // value dimension: one 32-coordinate word per wave

struct AttnArgs {
    int d, ng, W;                  // value dimension, channel groups, stored words per value
    int gdim[2], goff[2], gbits[2], gword[2];
    double coef[2][4];             // 2 a_P per group, planes: bit 0, bit 1, bit 2, xor of the three
    double bias[2];                // sum_P a_P per group
    double inv_sqrt_d[2];
};

__device__ __forceinline__ float at_wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double at_wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint64_t at_wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// 4 x 4 byte transpose: out[b] byte k = in[k] byte b.
__device__ __forceinline__ u32x4 at_transpose_bytes(u32x4 x) {
    const uint32_t t0 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
    const uint32_t t1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
    const uint32_t t2 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
    u32x4 y;
    y[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    y[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    y[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    y[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
    return y;
}

// Partial attention of one chunk of AT_CHUNK keys for four queries of one bank.
// grid (banks * chunks, ceil(G / 4)), AT_THREADS threads. Wave q computes the weights of
// query 4 * blockIdx.y + q; wave w accumulates coordinate word w (32 coordinates, group
// order) for the four queries.
// part [bank][G][chunks][2 + d] floats: scaled maximum, sum of e^(z - max), then o_rot
// (un-normalised, relative to that maximum).
__global__ __launch_bounds__(AT_THREADS) void attn_chunk_kernel(
    const float *__restrict__ scores, const uint32_t *__restrict__ vbits, const float *__restrict__ vnorms, long n,
    int n_tiles, int G, int chunks, float scale, AttnArgs a, float *__restrict__ part) {
    __shared__ __align__(16) uint8_t s_a[2][16][AT_CHUNK];     // [group][row 4q + limb][key]: weight limbs
    __shared__ __align__(16) uint32_t s_b[4][16][AT_STEP / 4];  // [wave][column 4P + byte][4 keys]
    __shared__ int s_F[2][4];
    __shared__ double s_vsum[2][4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long bank = blockIdx.x / chunks;
    const int ch = blockIdx.x % chunks;
    const int q0 = 4 * blockIdx.y;
    const long k0 = (long)ch * AT_CHUNK;
    const long n_pad = (long)n_tiles * 16;
    const int PS = 2 + a.d;

    // ---- 1. weights of query q0 + wv for every key of the chunk (lane = key within a step)
    {
        const int qg = q0 + wv;
        const bool qlive = qg < G;
        const float *srow = scores + ((size_t)bank * G + (qlive ? qg : 0)) * n;
        float e[AT_STEPS];
        float mx = -INFINITY;
#pragma unroll
        for (int s = 0; s < AT_STEPS; ++s) {
            const long key = k0 + AT_STEP * s + lane;
            e[s] = (qlive && key < n) ? scale * srow[key] : -INFINITY;
            mx = fmaxf(mx, e[s]);
        }
        mx = at_wave_max(mx);
        double esum = 0.0;
#pragma unroll
        for (int s = 0; s < AT_STEPS; ++s) {
            e[s] = e[s] == -INFINITY ? 0.0f : expf(e[s] - mx);
            esum += (double)e[s];
        }
        esum = at_wave_sum(esum);
        if (qlive && lane == 0) {
            float *pp = part + (((size_t)bank * G + qg) * chunks + ch) * PS;
            pp[0] = mx;
            pp[1] = (float)esum;
        }
        for (int g = 0; g < a.ng; ++g) {
            float w[AT_STEPS];
            float wm = 0.0f;
#pragma unroll
            for (int s = 0; s < AT_STEPS; ++s) {
                const long key = k0 + AT_STEP * s + lane;
                const float nu = key < n ? vnorms[((size_t)bank * n_pad + key) * a.ng + g] : 0.0f;
                w[s] = e[s] * nu;
                wm = fmaxf(wm, w[s]);
            }
            wm = at_wave_max(wm);
            // fixed point: w 2^F < 2^30 for every weight of the chunk
            int E = 0;
            if (wm > 0.0f) frexpf(wm, &E);
            const int F = wm > 0.0f ? 30 - E : 0;
            uint64_t vsum = 0;
#pragma unroll
            for (int s = 0; s < AT_STEPS; ++s) {
                const uint32_t V = (uint32_t)__float2int_rn(ldexpf(w[s], F));
                vsum += V;
                // balanced base-256 digits: bytes of V + 0x80808080, each minus 128
                const uint32_t L = (V + 0x80808080u) ^ 0x80808080u;
#pragma unroll
                for (int l = 0; l < 4; ++l) s_a[g][4 * wv + l][AT_STEP * s + lane] = (uint8_t)(L >> (8 * l));
            }
            vsum = at_wave_sum_u64(vsum);
            if (lane == 0) {
                s_F[g][wv] = F;
                s_vsum[g][wv] = (double)vsum;
            }
        }
    }
    __syncthreads();

    // ---- 2. wave wv: coordinate word wv of the four queries
    const int nwords = a.d >> 5;
    if (wv >= nwords) return;
    const int g = (a.ng > 1 && 32 * wv >= a.gdim[0]) ? 1 : 0;
    const int gb = a.gbits[g];
    const int wl = wv - (a.goff[g] >> 5);
    const int pstride = a.gdim[g] >> 5;
    const int wbase = a.gword[g] + wl;
    // staging role of this lane: tile T of the step, keys 4 s4 .. 4 s4 + 3, plane P
    const int T = lane >> 4, s4 = (lane >> 2) & 3, P = lane & 3;
    const int t_first = (int)(k0 >> 4);
    const uint32_t *vb = vbits + (size_t)bank * n_tiles * a.W * 16;

    // Every lane issues three loads a step, XORed only when the step is used (so the loads
    // stay in flight across the products): a stored plane P loads its word three times
    // (a ^ a ^ a = a), the XOR plane loads planes 0, 1, 2, and unused columns (coefficient
    // 0) load plane 0. Tiles past the bank's end re-read its last tile: their keys carry
    // zero weight.
    const int pa = P < gb ? P : 0;
    const int pb = P < gb ? P : (P == 3 && gb == 3 ? 1 : 0);
    const int pc = P < gb ? P : (P == 3 && gb == 3 ? 2 : 0);
    const size_t o0 = (size_t)(wbase + pa * pstride) * 16 + 4 * s4;
    const size_t o1 = (size_t)(wbase + pb * pstride) * 16 + 4 * s4;
    const size_t o2 = (size_t)(wbase + pc * pstride) * 16 + 4 * s4;
    struct Planes {
        u32x4 x0, x1, x2;
    };
    auto load_step = [&](int s) -> Planes {
        const int tile = min(t_first + 4 * s + T, n_tiles - 1);
        const uint32_t *tw = vb + (size_t)tile * a.W * 16;
        Planes r;
        r.x0 = *(const u32x4 *)(tw + o0);
        r.x1 = *(const u32x4 *)(tw + o1);
        r.x2 = *(const u32x4 *)(tw + o2);
        return r;
    };

    i32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = i32x4{0, 0, 0, 0};
    const int col = lane & 15, kg = lane >> 4;
    Planes x = load_step(0);
    for (int s = 0; s < AT_STEPS; ++s) {
        const u32x4 y = at_transpose_bytes(x.x0 ^ x.x1 ^ x.x2);
#pragma unroll
        for (int b = 0; b < 4; ++b) s_b[wv][4 * P + b][4 * T + s4] = y[b];
        const i8x16 A = *(const i8x16 *)&s_a[g][col][AT_STEP * s + 16 * kg];
        const u32x4 B = *(const u32x4 *)&s_b[wv][col][4 * kg];
        if (s + 1 < AT_STEPS) x = load_step(s + 1);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const u32x4 bt = B & (0x01010101u << t);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, __builtin_bit_cast(i8x16, bt), acc[t], 0, 0, 0);
        }
    }

    // ---- 3. lane (query c, column 4P + b): recombine limbs, weight the planes, add them up
    const int c = lane >> 4, Pc = col >> 2, bc = col & 3;
    const double coef = Pc < 4 ? a.coef[g][Pc] : 0.0;
    const int qg = q0 + c;
    const double fscale = ldexp(a.inv_sqrt_d[g], -s_F[g][c]);
    const double bterm = a.bias[g] * s_vsum[g][c];
    float *prow = part + (((size_t)bank * G + (qg < G ? qg : 0)) * chunks + ch) * PS + 2;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t v = (int64_t)acc[t][0] + ((int64_t)acc[t][1] << 8) + ((int64_t)acc[t][2] << 16) +
                          ((int64_t)acc[t][3] << 24);
        double xv = (double)v * coef * (t == 7 ? -1.0 / 128.0 : 1.0 / (double)(1 << t));
        xv += __shfl_xor(xv, 4, 64);
        xv += __shfl_xor(xv, 8, 64);
        if (Pc == 0 && qg < G) prow[32 * wv + 8 * bc + t] = (float)((xv - bterm) * fscale);
    }
}

// Merge of the chunks and the rotation back: one work-group per (bank, query), one thread
// per output channel. out [bank][G][d] float32 in channel order.
__global__ __launch_bounds__(AT_DMAX) void attn_combine_kernel(const float *__restrict__ part, int chunks,
                                                               const float *__restrict__ rot,
                                                               const int *__restrict__ chan, AttnArgs a,
                                                               float *__restrict__ out) {
    __shared__ double s_o[AT_DMAX];
    const int tid = threadIdx.x;
    const int PS = 2 + a.d;
    const float *pb = part + (size_t)blockIdx.x * chunks * PS;
    double mx = -INFINITY;
    for (int c = 0; c < chunks; ++c) mx = fmax(mx, (double)pb[(size_t)c * PS]);
    double tot = 0.0, v = 0.0;
    for (int c = 0; c < chunks; ++c) {
        const double f = exp((double)pb[(size_t)c * PS] - mx);
        tot += f * (double)pb[(size_t)c * PS + 1];
        if (tid < a.d) v += f * (double)pb[(size_t)c * PS + 2 + tid];
    }
    if (tid < a.d) s_o[tid] = v / tot;
    __syncthreads();
    // o[chan[off_g + k]] = sum_j R_g[j][k] o_rot[off_g + j]
    if (tid < a.d) {
        const int g = (a.ng > 1 && tid >= a.gdim[0]) ? 1 : 0;
        const int dg = a.gdim[g], off = a.goff[g], k = tid - off;
        const float *R = rot + (g ? (size_t)a.gdim[0] * a.gdim[0] : 0);
        double r = 0.0;
        for (int j = 0; j < dg; ++j) r += (double)R[(size_t)j * dg + k] * s_o[off + j];
        const int cc = chan ? chan[tid] : tid;
        out[(size_t)blockIdx.x * a.d + cc] = (float)r;
    }
}

// ---------------------------------------------------------------------------------------
// Decompression of a packed bank: x_hat per stored vector, channel order.
// One work-group per (bank, 16-key tile); the scaled centroids of the tile go to LDS
// (16 x d floats, group order), then thread k forms output channel k of the 16 vectors.
// ---------------------------------------------------------------------------------------
struct DecArgs {
    int d, ng, W;
    int gdim[2], goff[2], gbits[2], gword[2];
    float cent[2][8];
    float inv_sqrt_d[2];
};

__global__ __launch_bounds__(256) void decode_kernel(const uint32_t *__restrict__ bits, const float *__restrict__ norms,
                                                     long n, int n_tiles, const float *__restrict__ rot,
                                                     const int *__restrict__ chan, DecArgs a, float *__restrict__ out) {
    extern __shared__ float s_c[];  // [16][d]
    const long bank = blockIdx.x / n_tiles;
    const int t = blockIdx.x % n_tiles;
    const long n_pad = (long)n_tiles * 16;
    const uint32_t *tw = bits + ((size_t)bank * n_tiles + t) * a.W * 16;
    for (int e = threadIdx.x; e < 16 * a.d; e += blockDim.x) {
        const int i = e / a.d, j = e % a.d;
        const int g = (a.ng > 1 && j >= a.gdim[0]) ? 1 : 0;
        const int jj = j - a.goff[g];
        int idx = 0;
        for (int p = 0; p < a.gbits[g]; ++p)
            idx |= (int)((tw[(size_t)(a.gword[g] + p * (a.gdim[g] >> 5) + (jj >> 5)) * 16 + i] >> (jj & 31)) & 1u) << p;
        const float nu = norms[((size_t)bank * n_pad + 16 * t + i) * a.ng + g];
        s_c[i * a.d + j] = a.cent[g][idx] * (nu * a.inv_sqrt_d[g]);
    }
    __syncthreads();
    for (int k = threadIdx.x; k < a.d; k += blockDim.x) {
        const int g = (a.ng > 1 && k >= a.gdim[0]) ? 1 : 0;
        const int dg = a.gdim[g], off = a.goff[g], kk = k - off;
        const float *R = rot + (g ? (size_t)a.gdim[0] * a.gdim[0] : 0);
        float acc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
        for (int j = 0; j < dg; ++j) {
            const float r = R[(size_t)j * dg + kk];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf(r, s_c[i * a.d + off + j], acc[i]);
        }
        const int cc = chan ? chan[k] : k;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const long key = 16L * t + i;
            if (key < n) out[((size_t)bank * n + key) * a.d + cc] = acc[i];
        }
    }
}

}  // namespace tq
