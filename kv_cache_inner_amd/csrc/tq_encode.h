// Encoder kernels (stage 1: rotate + per-coordinate Lloyd-Max; stage 2: residual sign
// sketch), for gfx950.
//
// turboquant-pytorch write-up (discuss.pytorch.kr), two-stage algorithm section:
// each key is rotated by a random orthogonal matrix, every rotated coordinate is
// quantised on its own against a codebook precomputed for the normal distribution,
// then the stage-1 residual is projected by a Gaussian matrix and only the signs of
// the projections are kept.
//
// One work-group (4 wave64) encodes one 16-key tile of one bank:
//   1. keys -> LDS (float32, channels in group order), per-group norms in fp64;
//   2. Y_g = X_g R_g^T on MFMA (v_mfma_f32_16x16x4f32, fp32 products and sums);
//      z = sqrt(d_g) Y / |x_g|, bucket = #thresholds <= z, rotated residual
//      u = Y - (|x_g|/sqrt(d_g)) c[bucket] -> LDS;
//   3. P = U S'^T on MFMA with S' = S P_chan blockdiag(R_g)^T (prepared once per call),
//      which equals S times the residual taken in the original basis; sign = [P >= 0];
//      rho = |u| in fp64;
//   4. bit-planes and sign words packed from LDS, written as the bank tile
//      [W][16] (one coalesced store per word row).
#pragma once
#include "tq_device.h"

namespace tq {

struct EncArgs {
    int d, m, ng;
    int gdim[2], gbits[2], goff[2];
    int gword[2];  // first stored word of each group
    int sword;     // first sign word
    int W;         // stored words per key
    float cent[2][16];
    float thr[2][15];
    double sqrt_d[2];
};

// S'[i][pos] for pos = goff[g] + j: sum_k S[i][chan[goff[g]+k]] * R_g[j][k]  (fp64 sums)
__global__ __launch_bounds__(256) void enc_prep_proj_kernel(const float *__restrict__ S, const float *__restrict__ rot,
                                                            const int *__restrict__ chan, EncArgs a,
                                                            float *__restrict__ sp) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long)a.m * a.d) return;
    const int i = (int)(idx / a.d), pos = (int)(idx % a.d);
    const int g = (a.ng > 1 && pos >= a.gdim[0]) ? 1 : 0;
    const int dg = a.gdim[g], off = a.goff[g], j = pos - off;
    const float *R = rot + (g ? (long)a.gdim[0] * a.gdim[0] : 0) + (long)j * dg;
    double s = 0.0;
    for (int k = 0; k < dg; ++k) {
        const int c = chan ? chan[off + k] : off + k;
        s += (double)S[(long)i * a.d + c] * (double)R[k];
    }
    sp[(long)i * a.d + pos] = (float)s;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Gather the bits of one 32-element word from a byte array (one element per byte):
// bit t of the result = bit p of bytes[t].
__device__ __forceinline__ uint32_t pack_plane(const uint8_t *bytes, int p) {
    const uint32_t *w = reinterpret_cast<const uint32_t *>(bytes);
    uint32_t out = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t x = (w[q] >> p) & 0x01010101u;
        // bit 0 of each byte moved to bits 24..27 (no carries between the partial products)
        const uint32_t nib = ((x * 0x01020408u) >> 24) & 0xFu;
        out |= nib << (4 * q);
    }
    return out;
}

template <typename KT>
__device__ __forceinline__ float load_key(const KT *p);
template <>
__device__ __forceinline__ float load_key<float>(const float *p) {
    return *p;
}
template <>
__device__ __forceinline__ float load_key<uint16_t>(const uint16_t *p) {
    return bf16_to_f32(*p);
}

constexpr int ENC_KEYS = 16;

// Dynamic LDS: X[16][d+2] f32, U[16][d+2] f32, IDX[16][d] u8, SG[16][m] u8.
inline size_t enc_smem_bytes(int d, int m) {
    return (size_t)2 * ENC_KEYS * (d + 2) * 4 + (size_t)ENC_KEYS * d + (size_t)ENC_KEYS * m;
}

template <typename KT>
__global__ __launch_bounds__(256) void encode_kernel(const KT *__restrict__ keys, long n, int n_tiles,
                                                     const float *__restrict__ rot, const float *__restrict__ sp,
                                                     const int *__restrict__ chan, EncArgs a,
                                                     uint32_t *__restrict__ bits, float *__restrict__ norms,
                                                     float *__restrict__ rnorms) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float s_inv[ENC_KEYS][2], s_coef[ENC_KEYS][2], s_cent[2][16];
    const int d = a.d, m = a.m, ld = d + 2;
    float *X = reinterpret_cast<float *>(smem);
    float *U = X + ENC_KEYS * ld;
    uint8_t *IDX = reinterpret_cast<uint8_t *>(U + ENC_KEYS * ld);
    uint8_t *SG = IDX + ENC_KEYS * d;

    const long bank = blockIdx.x / n_tiles;
    const int tile = blockIdx.x % n_tiles;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const long n_pad = (long)n_tiles * ENC_KEYS;
    const long key0 = (long)tile * ENC_KEYS;

    if (tid < 32) s_cent[tid >> 4][tid & 15] = a.cent[tid >> 4][tid & 15];
    // 1. keys -> LDS in group order
    const KT *kb = keys + (size_t)bank * n * d;
    for (int e = tid; e < ENC_KEYS * d; e += 256) {
        const int i = e / d, pos = e % d;
        const long key = key0 + i;
        const int c = chan ? chan[pos] : pos;
        X[i * ld + pos] = key < n ? load_key<KT>(kb + (size_t)key * d + c) : 0.0f;
    }
    __syncthreads();

    // 2. per-group norms (fp64 sums of exact float squares)
    for (int kk = 0; kk < 4; ++kk) {
        const int i = 4 * wv + kk;
        for (int g = 0; g < a.ng; ++g) {
            double s = 0.0;
            for (int p = lane; p < a.gdim[g]; p += 64) {
                const double v = X[i * ld + a.goff[g] + p];
                s += v * v;
            }
            s = wave_sum_f64(s);
            if (lane == 0) {
                const double nu = sqrt(s);
                const float nu_s = (float)nu;
                s_inv[i][g] = nu > 0.0 ? (float)(a.sqrt_d[g] / nu) : 0.0f;
                s_coef[i][g] = (float)((double)nu_s / a.sqrt_d[g]);
                norms[((size_t)bank * n_pad + key0 + i) * a.ng + g] = nu_s;
            }
        }
    }
    __syncthreads();

    // 3. stage 1 on MFMA: Y = X_g R_g^T per 16x16 tile, then bucketize and residual
    const int li = lane & 15, lk = lane >> 4;
    const float *Rg = rot;
    for (int g = 0; g < a.ng; ++g) {
        const int dg = a.gdim[g], off = a.goff[g], L = 1 << a.gbits[g];
        const int nt_count = dg / 16;
        for (int nt0 = 2 * wv; nt0 < nt_count; nt0 += 8) {
            const bool two = nt0 + 1 < nt_count;
            f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
            const float *b0p = Rg + (size_t)(16 * nt0 + li) * dg + lk;
            const float *b1p = b0p + (size_t)16 * dg;
            const float *ap = X + li * ld + off + lk;
            for (int s = 0; s < dg / 4; ++s) {
                const float av = ap[4 * s];
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0p[4 * s], acc0, 0, 0, 0);
                if (two) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1p[4 * s], acc1, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t == 1 && !two) break;
                const f32x4 acc = t ? acc1 : acc0;
                const int j = 16 * (nt0 + t) + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * lk + r;
                    const float y = acc[r];
                    const float z = y * s_inv[i][g];
                    int idx = 0;
                    for (int q = 0; q < L - 1; ++q) idx += z >= a.thr[g][q];
                    U[i * ld + off + j] = y - s_coef[i][g] * s_cent[g][idx];
                    IDX[i * d + off + j] = (uint8_t)idx;
                }
            }
        }
        Rg += (size_t)dg * dg;
    }
    __syncthreads();

    // residual norm rho = |u| (fp64 sum)
    for (int kk = 0; kk < 4; ++kk) {
        const int i = 4 * wv + kk;
        double s = 0.0;
        for (int p = lane; p < d; p += 64) {
            const double v = U[i * ld + p];
            s += v * v;
        }
        s = wave_sum_f64(s);
        if (lane == 0) rnorms[(size_t)bank * n_pad + key0 + i] = (float)sqrt(s);
    }

    // 4. stage 2 on MFMA: P = U S'^T, sign = [P >= 0]
    {
        const int nt_count = m / 16;
        for (int nt0 = 2 * wv; nt0 < nt_count; nt0 += 8) {
            const bool two = nt0 + 1 < nt_count;
            f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
            const float *b0p = sp + (size_t)(16 * nt0 + li) * d + lk;
            const float *b1p = b0p + (size_t)16 * d;
            const float *ap = U + li * ld + lk;
            for (int s = 0; s < d / 4; ++s) {
                const float av = ap[4 * s];
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0p[4 * s], acc0, 0, 0, 0);
                if (two) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1p[4 * s], acc1, 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t == 1 && !two) break;
                const f32x4 acc = t ? acc1 : acc0;
                const int row = 16 * (nt0 + t) + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) SG[(4 * lk + r) * m + row] = acc[r] >= 0.0f ? 1 : 0;
            }
        }
    }
    __syncthreads();

    // 5. pack the tile: word w of key i -> bits[bank][tile][w][i]
    uint32_t *tb = bits + ((size_t)bank * n_tiles + tile) * (size_t)a.W * ENC_KEYS;
    for (int item = tid; item < a.W * ENC_KEYS; item += 256) {
        const int w = item / ENC_KEYS, i = item % ENC_KEYS;
        uint32_t word;
        if (w < a.sword) {
            const int g = (a.ng > 1 && w >= a.gword[1]) ? 1 : 0;
            const int wpp = a.gdim[g] / 32, lw = w - a.gword[g];
            const int p = lw / wpp, k = lw % wpp;
            word = pack_plane(IDX + i * d + a.goff[g] + 32 * k, p);
        } else {
            word = pack_plane(SG + i * m + 32 * (w - a.sword), 0);
        }
        tb[item] = word;
    }
}

}  // namespace tq
