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
#include <float.h>

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
    int nh;  // 1: the bank stores binary16 norms
};

// S'[i][pos] for pos = goff[g] + j: sum_k S[i][chan[goff[g]+k]] * R_g[j][k] (fp64 sums in
// ascending k). One work-group per row i of S (its permuted row staged in LDS), one thread
// per output column.
__global__ __launch_bounds__(256) void enc_prep_proj_kernel(const float *__restrict__ S, const float *__restrict__ rot,
                                                            const int *__restrict__ chan, EncArgs a,
                                                            float *__restrict__ sp) {
    __shared__ double s_row[1024];
    const long i = blockIdx.y;
    for (int pos = threadIdx.x; pos < a.d; pos += blockDim.x) {
        const int c = chan ? chan[pos] : pos;
        s_row[pos] = (double)S[i * a.d + ((unsigned)c < (unsigned)a.d ? c : 0)];
    }
    __syncthreads();
    const int pos = blockIdx.x * blockDim.x + threadIdx.x;
    if (pos >= a.d) return;
    const int g = (a.ng > 1 && pos >= a.gdim[0]) ? 1 : 0;
    const int dg = a.gdim[g], off = a.goff[g], j = pos - off;
    const float *R = rot + (g ? (long)a.gdim[0] * a.gdim[0] : 0) + (long)j * dg;
    double s = 0.0;
#pragma unroll 8
    for (int k = 0; k < dg; ++k) s += s_row[off + k] * (double)R[k];
    sp[i * a.d + pos] = (float)s;
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

// Where the keys of a call are stored. Default (pos == nullptr): key k of bank b at slot k
// of banks of n_tiles tiles, the padding slots of the last tile included. Appending: key k
// at slot pos[b] + k of banks of cap_tiles tiles, only keys k < n whose slot is in
// [0, 16 cap_tiles); no other slot is written.
struct EncSlots {
    const int32_t *pos;
    int cap_tiles;
};

template <typename KT>
__global__ __launch_bounds__(256) void encode_kernel(const KT *__restrict__ keys, long n, int n_tiles,
                                                     const float *__restrict__ rot, const float *__restrict__ sp,
                                                     const int *__restrict__ chan, EncArgs a,
                                                     uint32_t *__restrict__ bits, void *__restrict__ norms,
                                                     void *__restrict__ rnorms, EncSlots slots) {
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
    // output slot of key key0 + i within its bank (-1: not stored), and the bank's slot count
    const long out_pad = slots.pos ? (long)slots.cap_tiles * ENC_KEYS : n_pad;
    const long slot_base = slots.pos ? (long)slots.pos[bank] + key0 : key0;
    auto slot_of = [&](int i) -> long {
        const long sl = slot_base + i;
        if (!slots.pos) return sl;
        return (key0 + i < n && sl >= 0 && sl < out_pad) ? sl : -1;
    };

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
                // stored norm (float32 or its binary16 rounding) for the reconstruction
                const float nu_f = (float)nu;
                const uint16_t nu_h = f32_to_binary16(nu_f);
                const float nu_s = a.nh ? norm_f32(nu_h) : nu_f;
                s_inv[i][g] = nu > 0.0 ? (float)(a.sqrt_d[g] / nu) : 0.0f;
                s_coef[i][g] = (float)((double)nu_s / a.sqrt_d[g]);
                const long sl = slot_of(i);
                if (sl >= 0) {
                    const size_t at = ((size_t)bank * out_pad + sl) * a.ng + g;
                    if (a.nh)
                        static_cast<uint16_t *>(norms)[at] = nu_h;
                    else
                        static_cast<float *>(norms)[at] = nu_f;
                }
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
        const long sl = slot_of(i);
        // the MSE-only quantiser (m = 0) stores no residual norm: 0
        if (lane == 0 && sl >= 0) {
            const size_t at = (size_t)bank * out_pad + sl;
            const float rv = m > 0 ? (float)sqrt(s) : 0.0f;
            if (a.nh)
                static_cast<uint16_t *>(rnorms)[at] = f32_to_binary16(rv);
            else
                static_cast<float *>(rnorms)[at] = rv;
        }
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

    // 5. pack the tile: word w of the key in slot sl -> bits[bank][sl / 16][w][sl % 16]
    uint32_t *bb = bits + (size_t)bank * (out_pad / ENC_KEYS) * a.W * ENC_KEYS;
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
        const long sl = slot_of(i);
        if (sl >= 0) bb[((size_t)(sl / ENC_KEYS) * a.W + w) * ENC_KEYS + sl % ENC_KEYS] = word;
    }
}


// ---------------------------------------------------------------------------------------
// Encoder for d <= 128 and m <= 128 (KV-cache key shapes) on the bf16 matrix cores.
//
// The rotation and the projection are dense contractions with small fixed matrices, done
// here in bf16 MFMA (v_mfma_f32_16x16x32_bf16) at fp32-level accuracy: an fp32 value is
// exactly the sum of three bf16 values (x0 = bf16(x), x1 = bf16(x - x0), x2 = bf16(x - x0
// - x1): 8 significant bits each, every difference exact), products of bf16 values are
// exact in fp32 and the MFMA accumulates in fp32. So
//   - the rotation of bf16 keys by R = R0 + R1 + R2 is three MFMAs per 32-deep K block
//     with nothing dropped (six, with pieces of the key, for fp32 keys);
//   - the projection of the fp32 residual U = U0 + U1 + U2 by S' = S'0 + S'1 + S'2 takes
//     the six piece products of order a + b <= 2; each dropped one is below 2^-26 of the
//     leading product.
// The error left is fp32 accumulation rounding, as with fp32 MFMA; unlike fp32 MFMA (which
// issues at the vector fp32 rate), the bf16 matrix instructions run beside vector work.
//
// A persistent work-group of 16 waves walks 16-key tiles in a two-stage pipeline with one
// LDS barrier per tile:
//   - waves 0..7 keep rotation rows (three pieces) of coordinates 16w..16w+15 (group
//     order) as MFMA A operands in registers; for tile t they rotate, bucket, and write
//     the residual pieces to LDS in B-operand order, plus the tile's code bit-planes;
//   - waves 8..15 keep rows 16(w-8).. of S' (three pieces); for tile t-1 they project the
//     residual and add the sign words, stage tile t+1's keys into LDS (B-operand order)
//     with their norms, finish tile t-1's residual norms and store tile t-2's words.
// MFMA operand layout (16x16x32): lane 16k+i holds row i, K elements 8k..8k+7 of its block
// for A; column i, the same K elements for B; the result rows are 4k..4k+3 of column i.
//
// Per-element vector work is kept small, since it bounds the encoder:
//   - bucket = number of thresholds <= z, counted from the sign bits of z - t (no compare
//     and condition-register round trips); the planes come from the same sign words;
//   - norms: fp32 squares (exact for bf16 keys), four per lane summed in turn, then a
//     fixed pairwise tree across the 32 lanes of a key (DPP and row swaps): every term
//     passes through at most 8 roundings, so |x|^2 is within 8 units of fp32 rounding
//     (relative) of the exact sum of non-negative terms, far inside 1e-6 on |x|;
//   - residual norm: per-wave fp32 partial sums over 16 coordinates, combined in fp64;
//   - cross-lane gathers of bit nibbles and partial sums use v_permlane16/32_swap.
constexpr int ENCS_WAVES = 16, ENCS_ROT = 8, ENCS_DMAX = 128, ENCS_WMAX = 16;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive channels of one key, as loaded (one 16- or 8-byte load).
template <typename KT>
struct KeyQuad;
template <>
struct KeyQuad<float> {
    u32x4 v;
    __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
    __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const u32x4 *>(p); }
    __device__ __forceinline__ float get(int u) const { return __uint_as_float(v[u]); }
};
template <>
struct KeyQuad<uint16_t> {
    uint32_t v0, v1;
    __device__ __forceinline__ void zero() { v0 = v1 = 0; }
    __device__ __forceinline__ void load(const uint16_t *p) {
        const uint2 t = *reinterpret_cast<const uint2 *>(p);
        v0 = t.x;
        v1 = t.y;
    }
    __device__ __forceinline__ float get(int u) const {
        const uint32_t w = u < 2 ? v0 : v1;
        return __uint_as_float((u & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};


// v moved across lanes by a DPP pattern (quad permutations, row mirrors): every source lane
// exists, so each lane receives exactly one value
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// x[lane] op x[lane ^ 16] and x[lane] op x[lane ^ 32], as the two outputs of a row swap
__device__ __forceinline__ uint32_t or_rows16(uint32_t x) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return p[0] | p[1];
}
__device__ __forceinline__ uint32_t or_rows32(uint32_t x) {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return p[0] | p[1];
}
__device__ __forceinline__ float add_rows16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_rows32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over the 32 lanes of a half-wave by a fixed pairwise tree (xor 1, xor 2, 8-lane
// mirror, 16-lane mirror, row swap); every lane of the half ends with the same value.
__device__ __forceinline__ float sum_half_wave(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return add_rows16(v);
}

// Buckets and residuals of one lane's four rotated coordinates (MFMA output rows r) of
// one key, for a codebook of NB bits. th: the 2^NB - 1 ascending thresholds. Returns the
// bit-plane nibbles: bit r of pl[p] = bit p of bucket r.
template <int NB>
__device__ __forceinline__ void encr_bucket(const f32x4 &acc, float inv, float coef, const float (&th)[7],
                                            const float *cent, float (&u)[4], uint32_t (&pl)[3]) {
    constexpr int NT = (1 << NB) - 1;
#pragma unroll
    for (int p = 0; p < 3; ++p) pl[p] = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float y = acc[r];
        const float z = y * inv;
        // sign bit of z - t is set iff z < t (z - t is +0 when z == t)
        uint32_t sw[NT];
        uint32_t below = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            sw[t] = __float_as_uint(z - th[t]);
            below += sw[t] >> 31;
        }
        const uint32_t idx = NT - below;
        u[r] = fmaf(-coef, cent[idx], y);  // one rounding, whatever the compiler contracts
        // bit p of the bucket, from the sign words (bucket = number of thresholds <= z)
        uint32_t b0, b1 = 0, b2 = 0;
        if constexpr (NB == 1) {
            b0 = ~sw[0];
        } else if constexpr (NB == 2) {
            b1 = ~sw[1];
            b0 = ~(sw[0] ^ sw[1] ^ sw[2]);
        } else {
            b2 = ~sw[3];
            b1 = ~(sw[1] ^ sw[3] ^ sw[5]);
            b0 = ~(sw[0] ^ sw[1] ^ sw[2] ^ sw[3] ^ sw[4] ^ sw[5] ^ sw[6]);
        }
        pl[0] |= (b0 >> 31) << r;
        if constexpr (NB > 1) pl[1] |= (b1 >> 31) << r;
        if constexpr (NB > 2) pl[2] |= (b2 >> 31) << r;
    }
}


// (a, b) rounded to bf16 (v_cvt_pk_bf16_f32, round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// exact three-piece bf16 split of (a, b): a = lo(p0) + lo(p1) + lo(p2), b likewise (high)
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t &p0, uint32_t &p1, uint32_t &p2) {
    p0 = pk_bf16(a, b);
    a -= bf16_lo(p0);
    b -= bf16_hi(p0);
    p1 = pk_bf16(a, b);
    a -= bf16_lo(p1);
    b -= bf16_hi(p1);
    p2 = pk_bf16(a, b);
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// acc = A * B over NKB 32-deep K blocks. A: three bf16 pieces per block in registers.
// B: from LDS at b[kb * 64] (piece 0) and b[p * ps + kb * 64] (pieces 1, 2 when XP == 3).
// Smaller products first.
template <int NKB, int XP>
__device__ __forceinline__ f32x4 encs_mma(const u32x4 (&am)[4][3], const u32x4 *b, int ps) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 x0 = b[kb * 64];
        if constexpr (XP == 1) {
            acc = mfma_bf16(am[kb][2], x0, acc);
            acc = mfma_bf16(am[kb][1], x0, acc);
            acc = mfma_bf16(am[kb][0], x0, acc);
        } else {
            const u32x4 x1 = b[ps + kb * 64], x2 = b[2 * ps + kb * 64];
            acc = mfma_bf16(am[kb][0], x2, acc);
            acc = mfma_bf16(am[kb][1], x1, acc);
            acc = mfma_bf16(am[kb][2], x0, acc);
            acc = mfma_bf16(am[kb][0], x1, acc);
            acc = mfma_bf16(am[kb][1], x0, acc);
            acc = mfma_bf16(am[kb][0], x0, acc);
        }
    }
    return acc;
}
// the same for a wave-uniform block count nkb in 1..4 (32..128 deep)
template <int XP>
__device__ __forceinline__ f32x4 encs_mma_n(int nkb, const u32x4 (&am)[4][3], const u32x4 *b, int ps) {
    switch (nkb) {
        case 1: return encs_mma<1, XP>(am, b, ps);
        case 2: return encs_mma<2, XP>(am, b, ps);
        case 3: return encs_mma<3, XP>(am, b, ps);
        default: return encs_mma<4, XP>(am, b, ps);
    }
}

// A operand of rows row0.. of a row-major fp32 matrix (row stride ld), K blocks kb < nkb
// starting at column c0: lane (k, i) gets row row0 + i, columns c0 + 32kb + 8k .. + 7,
// split into three bf16 pieces.
__device__ __forceinline__ void encs_load_a(u32x4 (&am)[4][3], const float *mat, int ld, int row0, int c0, int nkb,
                                            int lane) {
    const float *src = mat + (size_t)(row0 + (lane & 15)) * ld + c0 + 8 * (lane >> 4);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t p0 = 0, p1 = 0, p2 = 0;
            if (kb < nkb) split3_pair(src[32 * kb + 2 * d], src[32 * kb + 2 * d + 1], p0, p1, p2);
            am[kb][0][d] = p0;
            am[kb][1][d] = p1;
            am[kb][2][d] = p2;
        }
    }
}

// bf16 element index, inside one piece of the LDS operand layout [kb][64 lanes][8], of
// coordinate pos of key `key`
__device__ __forceinline__ int encs_elem(int pos, int key) {
    return ((((pos >> 5) << 6) + (((pos >> 3) & 3) << 4) + key) << 3) + (pos & 7);
}

// NGT: the channel-group count fixed at compile time (0: read from the arguments); NBT: the
// codebook width of a one-group layout fixed at compile time (0: read from the arguments);
// DT, MT: d and m fixed at compile time (DT = 0: both read from the arguments). Fixed values let the compiler
// drop the unused paths, thresholds and per-lane group masks (which otherwise spill scalar
// registers) and turn the K-block counts and operand offsets into constants. Measured
// (in-process A/Bs, byte-identical banks): two groups about 7 % faster on the long-context
// banks; one group with its width fixed 3.5 % (b = 3) and 7 % (b = 4) faster on the decode
// shapes (one group with the width left variable spilled a vector register and was 10 %
// slower); d = m = 128 fixed on top of that, another 14 % (b = 3) and 16 % (b = 4).
template <typename KT, int NGT, int NBT = 0, int DT = 0, int MT = DT>
__global__ __launch_bounds__(ENCS_WAVES * 64) void encode_split_kernel(
    const KT *__restrict__ keys, long n, int n_tiles, int total_tiles, const float *__restrict__ rot,
    const float *__restrict__ sp, const int *__restrict__ chan, EncArgs a, uint32_t *__restrict__ bits,
    void *__restrict__ norms, void *__restrict__ rnorms, EncSlots slots) {
    constexpr int XP = sizeof(KT) == 2 ? 1 : 3;  // key pieces: bf16 keys are exact in one
    constexpr int PS = 4 * 64;                     // piece stride of the operand buffers (u32x4)
    __shared__ __align__(16) u32x4 XB[2][XP][4][64];
    __shared__ __align__(16) u32x4 UB[2][3][4][64];
    __shared__ __align__(16) uint32_t TW[3][ENCS_WMAX * 16];
    __shared__ float s_inv[2][16][2], s_coef[2][16][2];
    __shared__ float s_cent[2][8];
    __shared__ float s_rho[2][ENCS_ROT][16];
    __shared__ int s_pos[ENCS_DMAX];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int D = DT ? DT : a.d, M = DT ? MT : a.m, ng = NGT ? NGT : a.ng;
    const int grid = gridDim.x;
    const bool rot_role = wv < ENCS_ROT;

    // channel -> coordinate position in group order (entries of a non-permutation are
    // kept in range)
    for (int c = tid; c < ENCS_DMAX; c += ENCS_WAVES * 64) s_pos[c] = c < D ? c : 0;
    if (tid < 16) s_cent[tid >> 3][tid & 7] = a.cent[tid >> 3][tid & 7];
    __syncthreads();
    if (chan)
        for (int p = tid; p < D; p += ENCS_WAVES * 64) {
            const int c = chan[p];
            if ((unsigned)c < (unsigned)D) s_pos[c] = p;
        }
    __syncthreads();

    // ---- rotation role: coordinates pos0..pos0+15 of group g
    const int pos0 = 16 * wv;
    const bool rot_live = rot_role && pos0 < D;
    const int g = (ng > 1 && pos0 >= a.gdim[0]) ? 1 : 0;
    const int dg = (DT && NGT == 1) ? DT : (g ? a.gdim[1] : a.gdim[0]);
    const int off = g ? a.goff[1] : 0;
    const int j0 = pos0 - off, nkb_r = dg / 32;
    const int nb = NBT ? NBT : (g ? a.gbits[1] : a.gbits[0]);
    float th[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) th[t] = t < (1 << nb) - 1 ? (g ? a.thr[1][t] : a.thr[0][t]) : INFINITY;
    const int cw_word = (g ? a.gword[1] : a.gword[0]) + (j0 >> 5), cw_half = (j0 >> 4) & 1, wpp = dg / 32;
    // this lane's residual slot: coordinates pos0 + 4q .. +3 of key i, as 4 bf16 of a piece
    const int u_elem = encs_elem(pos0 + 4 * q, i);

    // ---- projection role: rows r0..r0+15 of S'
    const int r0 = 16 * (wv - ENCS_ROT);
    const bool prj_live = !rot_role && r0 < M;
    const int nkb_p = D / 32;
    const int sw_word = a.sword + (r0 >> 5), sw_half = (r0 >> 4) & 1;

    u32x4 am[4][3];
    if (rot_live)
        encs_load_a(am, rot + (g ? (size_t)a.gdim[0] * a.gdim[0] : 0), dg, j0, 0, nkb_r, lane);
    else if (prj_live)
        encs_load_a(am, sp, D, r0, 0, nkb_p, lane);

    // ---- staging (projection-role threads): key ik, channels 4cq..4cq+3
    const int st = tid - ENCS_ROT * 64;
    const int ik = (st >> 5) & 15, cq = st & 31;
    const bool cq_live = !rot_role && 4 * cq < D;
    const float sqrt_d0 = (float)a.sqrt_d[0], sqrt_d1 = (float)a.sqrt_d[1];
    const float inv_sqrt_d0 = (float)(1.0 / a.sqrt_d[0]), inv_sqrt_d1 = ng > 1 ? (float)(1.0 / a.sqrt_d[1]) : 0.0f;
    int xo[4];
    uint32_t in_g1 = 0;  // bit u: channel 4cq+u belongs to group 1
    bool contig = true;  // the four channels land on four consecutive slots of one lane
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pos = cq_live ? s_pos[4 * cq + u] : 4 * cq + u;
        xo[u] = encs_elem(pos, ik);
        in_g1 |= (ng > 1 && pos >= a.gdim[0]) ? 1u << u : 0u;
        contig = contig && xo[u] == xo[0] + u;
    }
    contig = contig && (xo[0] & 3) == 0;
    const int key_off = ik * D + 4 * cq;
    // flat output slot (bank * slots per bank + slot) of key i of input tile T, or -1 when the
    // key is not stored (appending: past the input keys, or outside the bank)
    const long out_pad = slots.pos ? (long)slots.cap_tiles * 16 : 0;
    auto out_slot = [&](long T, int ki) -> long {
        if (!slots.pos) return T * 16 + ki;
        const long bank = T / n_tiles, k = (T - bank * n_tiles) * 16 + ki;
        const long sl = (long)slots.pos[bank] + k;
        return (k < n && sl >= 0 && sl < out_pad) ? bank * out_pad + sl : -1;
    };

    // (bank, tile) of the next key load; loads go to tiles blockIdx.x + k * grid, k = 0, 1, ...
    int l_bank = (int)blockIdx.x / n_tiles, l_tile = (int)blockIdx.x - l_bank * n_tiles;
    const int step_banks = grid / n_tiles, step_tiles = grid - step_banks * n_tiles;
    auto load_keys = [&](long T, KeyQuad<KT> &kq) {
        kq.zero();
        if (T < total_tiles) {
            const long key0 = (long)l_tile * 16;
            const KT *tile_keys = keys + ((size_t)l_bank * n + key0) * D;  // wave-uniform
            if (cq_live && key0 + ik < n) kq.load(tile_keys + key_off);
        }
        l_bank += step_banks;
        l_tile += step_tiles;
        if (l_tile >= n_tiles) {
            l_tile -= n_tiles;
            ++l_bank;
        }
    };
    // keys -> LDS operand order (pieces for fp32 keys); per-group norms
    auto stage = [&](long T, const KeyQuad<KT> &kq, int buf) {
        float v[4], s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = kq.get(u);
        if (cq_live) {
            uint16_t *xb = reinterpret_cast<uint16_t *>(&XB[buf][0][0][0]);
            if constexpr (XP == 1) {
                if (contig)
                    *reinterpret_cast<u32x2 *>(xb + xo[0]) = u32x2{kq.v0, kq.v1};
                else
#pragma unroll
                    for (int u = 0; u < 4; ++u) xb[xo[u]] = (uint16_t)(__float_as_uint(v[u]) >> 16);
            } else {
                uint32_t pa[3], pb[3];
                split3_pair(v[0], v[1], pa[0], pa[1], pa[2]);
                split3_pair(v[2], v[3], pb[0], pb[1], pb[2]);
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    uint16_t *xp = xb + p * PS * 8;
                    if (contig) {
                        *reinterpret_cast<u32x2 *>(xp + xo[0]) = u32x2{pa[p], pb[p]};
                    } else {
                        xp[xo[0]] = (uint16_t)pa[p];
                        xp[xo[1]] = (uint16_t)(pa[p] >> 16);
                        xp[xo[2]] = (uint16_t)pb[p];
                        xp[xo[3]] = (uint16_t)(pb[p] >> 16);
                    }
                }
            }
        }
        if (ng > 1) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool h = (in_g1 >> u) & 1;
                s0 = fmaf(h ? 0.0f : v[u], v[u], s0);
                s1 = fmaf(h ? v[u] : 0.0f, v[u], s1);
            }
            s1 = sum_half_wave(s1);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) s0 = fmaf(v[u], v[u], s0);
        }
        s0 = sum_half_wave(s0);
        if (cq < ng) {
            const float s = cq ? s1 : s0;
            // |x| = s rsq(s) and sqrt(d)/|x| = sqrt(d) rsq(s) (v_rsq_f32, within 1 ulp) for a
            // normal s; the correctly rounded forms for zero and subnormal sums
            float nu, inv;
            if (s >= FLT_MIN) {
                const float rs = __builtin_amdgcn_rsqf(s);
                nu = s * rs;
                inv = (cq ? sqrt_d1 : sqrt_d0) * rs;
            } else {
                nu = sqrtf(s);
                inv = s > 0.0f ? (cq ? sqrt_d1 : sqrt_d0) / nu : 0.0f;
            }
            s_inv[buf][ik][cq] = inv;
            // the reconstruction (and so the residual) takes the stored norm: with binary16
            // norms its rounding, which the sketch then corrects too
            const uint16_t nu_h = f32_to_binary16(nu);
            const float nu_st = a.nh ? norm_f32(nu_h) : nu;
            s_coef[buf][ik][cq] = nu_st * (cq ? inv_sqrt_d1 : inv_sqrt_d0);
            const long fs = out_slot(T, ik);
            if (fs >= 0) {
                if (a.nh)
                    static_cast<uint16_t *>(norms)[(size_t)fs * ng + cq] = nu_h;
                else
                    static_cast<float *>(norms)[(size_t)fs * ng + cq] = nu;
            }
        }
    };

    const long T0 = blockIdx.x;
    KeyQuad<KT> kq;
    if (!rot_role) {
        load_keys(T0, kq);
        stage(T0, kq, 0);
        load_keys(T0 + grid, kq);
    }
    lds_barrier();
    uint16_t *const tw16 = reinterpret_cast<uint16_t *>(&TW[0][0]);
    int tb = 0;  // it % 3
    for (int it = 0;; ++it, tb = tb == 2 ? 0 : tb + 1) {
        const long tr = T0 + (long)it * grid;  // rotated in this step
        const long tp = tr - grid;             // projected
        const long tw = tr - 2 * (long)grid;   // stored
        if (tw >= total_tiles) break;
        const int buf = it & 1, tb_p = tb == 0 ? 2 : tb - 1, tb_w = tb == 2 ? 0 : tb + 1;
        if (rot_role) {
            if (rot_live && tr < total_tiles) {
                const f32x4 acc = encs_mma_n<XP>(nkb_r, am, &XB[buf][0][off >> 5][lane], PS);
                const float inv = s_inv[buf][i][g], coef = s_coef[buf][i][g];
                float u[4];
                uint32_t pl[3];
                if (nb == 1)
                    encr_bucket<1>(acc, inv, coef, th, s_cent[g], u, pl);
                else if (nb == 2)
                    encr_bucket<2>(acc, inv, coef, th, s_cent[g], u, pl);
                else
                    encr_bucket<3>(acc, inv, coef, th, s_cent[g], u, pl);
                // residual pieces in B-operand order
                uint32_t pa[3], pb[3];
                split3_pair(u[0], u[1], pa[0], pa[1], pa[2]);
                split3_pair(u[2], u[3], pb[0], pb[1], pb[2]);
                uint16_t *ub = reinterpret_cast<uint16_t *>(&UB[buf][0][0][0]) + u_elem;
#pragma unroll
                for (int p = 0; p < 3; ++p) *reinterpret_cast<u32x2 *>(ub + p * PS * 8) = u32x2{pa[p], pb[p]};
                float rr = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) rr = fmaf(u[r], u[r], rr);
                // nibbles of the four lane rows -> the 16 bits of this key's half-word
                uint32_t pl01 = (pl[0] | (pl[1] << 16)) << (4 * q), pl2 = pl[2] << (4 * q);
                pl01 = or_rows32(or_rows16(pl01));
                rr = add_rows32(add_rows16(rr));
                if (q == 0) s_rho[buf][wv][i] = rr;
                if (nb > 2) pl2 = or_rows32(or_rows16(pl2));
                if (q < nb) {
                    const uint32_t vv = q == 0 ? (pl01 & 0xffffu) : (q == 1 ? (pl01 >> 16) : pl2);
                    tw16[((tb * ENCS_WMAX + cw_word + q * wpp) * 16 + i) * 2 + cw_half] = (uint16_t)vv;
                }
            } else if (lane < 16) {
                s_rho[buf][wv][lane] = 0.0f;
            }
        } else {
            // vector work first (it overlaps the rotation waves' MFMA chains), then the
            // projection chain (it overlaps their bucketing)
            // the tile after next: keys (loaded one step ago) into LDS, then the next load
            const long ts = tr + grid;
            if (ts < total_tiles) {
                stage(ts, kq, buf ^ 1);
                load_keys(ts + grid, kq);
            }
            // tile tw is complete: its stored words, one coalesced block
            if (tw >= 0 && !slots.pos && st < a.W * 4)
                reinterpret_cast<u32x4 *>(bits + (size_t)tw * a.W * 16)[st] =
                    reinterpret_cast<const u32x4 *>(&TW[tb_w][0])[st];
            if (tw >= 0 && slots.pos && st < a.W * 16) {  // appending: each key to its slot
                const long fs = out_slot(tw, st & 15);
                if (fs >= 0) bits[((size_t)(fs >> 4) * a.W + (st >> 4)) * 16 + (fs & 15)] = TW[tb_w][st];
            }
            if (tp >= 0 && tp < total_tiles) {
                // residual norm rho = |u| (fp64 sum of the rotation waves' partial sums)
                if (wv == ENCS_WAVES - 1 && lane < 16) {
                    double s = 0.0;
#pragma unroll
                    for (int w = 0; w < ENCS_ROT; ++w) s += (double)s_rho[buf ^ 1][w][lane];
                    const long fs = out_slot(tp, lane);
                    const float rv = M > 0 ? (float)sqrt(s) : 0.0f;  // none stored for m = 0
                    if (fs >= 0) {
                        if (a.nh)
                            static_cast<uint16_t *>(rnorms)[fs] = f32_to_binary16(rv);
                        else
                            static_cast<float *>(rnorms)[fs] = rv;
                    }
                }
                // project tile tp's residual, add its sign words
                if (prj_live) {
                    const f32x4 acc = encs_mma_n<3>(nkb_p, am, &UB[buf ^ 1][0][0][lane], PS);
                    uint32_t sg = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sg |= (acc[r] >= 0.0f ? 1u : 0u) << r;
                    sg = or_rows32(or_rows16(sg << (4 * q)));
                    if (q == 0) tw16[((tb_p * ENCS_WMAX + sw_word) * 16 + i) * 2 + sw_half] = (uint16_t)sg;
                }
            }
        }
        lds_barrier();
    }
}

}  // namespace tq
