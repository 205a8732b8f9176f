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


// ---------------------------------------------------------------------------------------
// Register-resident encoder for d <= 128 and m <= 128 (KV-cache key shapes).
//
// The rotation and the projection are dense contractions with small, fixed right-hand
// matrices, so a persistent work-group of 8 waves keeps them in registers for the whole
// launch as MFMA A operands: wave w holds the rotation rows of its 16 rotated coordinates
// 16w..16w+15 (group order) and rows 16w..16w+15 of S'. It then walks 16-key tiles:
//   - the keys sit in LDS in the B-operand order of v_mfma_f32_16x16x4f32 (lane 16k+i of
//     K-step s holds coordinate 4s+k of key i), so every operand read is one conflict-free
//     ds_read_b128 that serves four K-steps;
//   - each wave rotates its 16 coordinates of the 16 keys (K = d_g), buckets them and
//     writes the residual back to LDS in the same operand order;
//   - each wave projects the residual on its 16 rows of S' (K = d) and keeps the signs;
//   - bit-planes and sign bits are gathered across lanes into the tile's stored words in
//     LDS and leave as one coalesced block.
// The keys of the work-group's next tile are loaded one tile ahead; two LDS-only barriers
// per tile. Arithmetic per element is that of encode_kernel (fp32 products and sums in
// the same K order, fp64 norms, the same bucket and residual formulas).
constexpr int ENCR_WAVES = 8, ENCR_DMAX = 128, ENCR_WMAX = 16;

// LDS float offset of (coordinate pos, key) in the B-operand layout [pos/16][64 lanes][4]
__device__ __forceinline__ int encr_off(int pos, int key) {
    return ((((pos >> 4) << 6) + ((pos & 3) << 4) + key) << 2) + ((pos >> 2) & 3);
}

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

// acc = A * B over NS K-steps: A from registers (a[s], lane (k, i) of K-step s), B from
// the LDS operand layout (b[(s/4)*64] holds K-steps s..s+3 of this lane)
template <int NS>
__device__ __forceinline__ f32x4 encr_mma(const float (&a)[32], const f32x4 *b) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < NS / 4; ++s4) {
        const f32x4 v = b[s4 * 64];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * s4 + 0], v[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * s4 + 1], v[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * s4 + 2], v[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * s4 + 3], v[3], acc, 0, 0, 0);
    }
    return acc;
}
// the same for a wave-uniform K-step count ns in {8, 16, 24, 32} (a group of 32..128
// coordinates)
__device__ __forceinline__ f32x4 encr_mma_n(int ns, const float (&a)[32], const f32x4 *b) {
    switch (ns) {
        case 8: return encr_mma<8>(a, b);
        case 16: return encr_mma<16>(a, b);
        case 24: return encr_mma<24>(a, b);
        default: return encr_mma<32>(a, b);
    }
}

template <typename KT>
__global__ __launch_bounds__(ENCR_WAVES * 64) __attribute__((amdgpu_waves_per_eu(4))) void encode_regs_kernel(
    const KT *__restrict__ keys, long n, int n_tiles, long total_tiles, const float *__restrict__ rot,
    const float *__restrict__ sp, const int *__restrict__ chan, EncArgs a, uint32_t *__restrict__ bits,
    float *__restrict__ norms, float *__restrict__ rnorms) {
    __shared__ __align__(16) float Xf[ENCR_DMAX * 16];
    __shared__ __align__(16) float Uf[ENCR_DMAX * 16];
    __shared__ __align__(16) uint32_t TW[2][ENCR_WMAX * 16];
    __shared__ float s_inv[2][16][2], s_coef[2][16][2];
    __shared__ float s_cent[2][8];
    __shared__ double s_rho[ENCR_WAVES][16];
    __shared__ int s_pos[ENCR_DMAX];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, q = lane >> 4;
    const int D = a.d, M = a.m, ng = a.ng;
    const long n_pad = (long)n_tiles * 16;
    const int grid = gridDim.x;

    // channel -> coordinate position in group order (entries of a non-permutation are
    // kept in range)
    for (int c = tid; c < ENCR_DMAX; c += ENCR_WAVES * 64) s_pos[c] = c < D ? c : 0;
    if (tid < 16) s_cent[tid >> 3][tid & 7] = a.cent[tid >> 3][tid & 7];
    __syncthreads();
    if (chan)
        for (int p = tid; p < D; p += ENCR_WAVES * 64) {
            const int c = chan[p];
            if ((unsigned)c < (unsigned)D) s_pos[c] = p;
        }
    __syncthreads();

    // this thread's share of a tile's keys: key ik, channels 4cq..4cq+3
    const int ik = tid >> 5, cq = tid & 31;
    const bool cq_live = 4 * cq < D;
    // lanes cq = 0, 1 finish the norms of groups 0, 1 (read once here: a lane-dependent
    // choice between kernel arguments inside the loop becomes a memory load)
    const double my_sqrt_d = cq == 1 ? a.sqrt_d[1] : a.sqrt_d[0];
    int xo[4];
    bool in_g1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pos = cq_live ? s_pos[4 * cq + u] : 0;
        xo[u] = encr_off(pos, ik);
        in_g1[u] = ng > 1 && pos >= a.gdim[0];
    }

    // rotation operand: rows j0..j0+15 of R_g, lane (q, i) holds R_g[j0+i][4s+q]
    const int pos0 = 16 * wv;
    const bool rot_live = pos0 < D;
    const int g = (ng > 1 && pos0 >= a.gdim[0]) ? 1 : 0;
    const int dg = g ? a.gdim[1] : a.gdim[0];
    const int off = g ? a.goff[1] : 0;
    const int j0 = pos0 - off, nsr = dg / 4;
    float ra[32];
    {
        const float *Rg = rot + (g ? (size_t)a.gdim[0] * a.gdim[0] : 0) + (size_t)(j0 + i) * dg + q;
#pragma unroll
        for (int s = 0; s < 32; ++s) ra[s] = (rot_live && s < nsr) ? Rg[4 * s] : 0.0f;
    }
    float th[7];
    const int nb = g ? a.gbits[1] : a.gbits[0];
#pragma unroll
    for (int t = 0; t < 7; ++t) th[t] = t < (1 << nb) - 1 ? (g ? a.thr[1][t] : a.thr[0][t]) : INFINITY;
    const int cw_word = (g ? a.gword[1] : a.gword[0]) + (j0 >> 5), cw_half = (j0 >> 4) & 1, wpp = dg / 32;

    // projection operand: rows r0..r0+15 of S', lane (q, i) holds S'[r0+i][4s+q]
    const int r0 = 16 * wv;
    const bool prj_live = r0 < M;
    const int nsp = D / 4;
    float rp[32];
    {
        const float *Sp = sp + (size_t)(r0 + i) * D + q;
#pragma unroll
        for (int s = 0; s < 32; ++s) rp[s] = (prj_live && s < nsp) ? Sp[4 * s] : 0.0f;
    }
    const int sw_word = a.sword + (r0 >> 5), sw_half = (r0 >> 4) & 1;

    auto load_keys = [&](long T, KeyQuad<KT> &kq) {
        kq.zero();
        if (T < total_tiles && cq_live) {
            const long bank = T / n_tiles, key = (T % n_tiles) * 16 + ik;
            if (key < n) kq.load(keys + ((size_t)bank * n + key) * D + 4 * cq);
        }
    };
    // keys -> LDS operand order; per-group norms (fp64 sums of exact float squares)
    auto stage = [&](long T, const KeyQuad<KT> &kq, int buf) {
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float v = kq.get(u);
            if (cq_live) Xf[xo[u]] = v;
            const double dv = v;
            if (in_g1[u])
                s1 += dv * dv;
            else
                s0 += dv * dv;
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            s0 += __shfl_xor(s0, o, 64);
            s1 += __shfl_xor(s1, o, 64);
        }
        if (cq < ng) {
            const double s = cq ? s1 : s0, sd = my_sqrt_d;
            const double nu = sqrt(s);
            const float nu_s = (float)nu;
            s_inv[buf][ik][cq] = nu > 0.0 ? (float)(sd / nu) : 0.0f;
            s_coef[buf][ik][cq] = (float)((double)nu_s / sd);
            const long bank = T / n_tiles, key = (T % n_tiles) * 16 + ik;
            norms[((size_t)bank * n_pad + key) * ng + cq] = nu_s;
        }
    };

    long T = blockIdx.x;
    KeyQuad<KT> kq;
    load_keys(T, kq);
    stage(T, kq, 0);
    load_keys(T + grid, kq);
    lds_barrier();
    uint16_t *const tw16 = reinterpret_cast<uint16_t *>(&TW[0][0]);
    for (int it = 0; T < total_tiles; T += grid, ++it) {
        const int buf = it & 1;
        const long bank = T / n_tiles;
        const int tile = (int)(T % n_tiles);
        // stage 1: rotate, bucket, residual
        if (rot_live) {
            const f32x4 acc = encr_mma_n(nsr, ra, reinterpret_cast<const f32x4 *>(Xf) + (off >> 4) * 64 + lane);
            const float inv = s_inv[buf][i][g], coef = s_coef[buf][i][g];
            double rr = 0.0;
            uint32_t pl01 = 0, pl2 = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float y = acc[r];
                const float z = y * inv;
                int idx = 0;
#pragma unroll
                for (int t = 0; t < 7; ++t) idx += z >= th[t] ? 1 : 0;
                const float u = y - coef * s_cent[g][idx];
                Uf[((wv * 64 + 16 * r + i) << 2) + q] = u;
                rr += (double)u * (double)u;
                pl01 |= ((uint32_t)(idx & 1) << r) | ((uint32_t)((idx >> 1) & 1) << (16 + r));
                pl2 |= (uint32_t)((idx >> 2) & 1) << r;
            }
            pl01 <<= 4 * q;
            pl2 <<= 4 * q;
            pl01 |= __shfl_xor(pl01, 16, 64);
            pl2 |= __shfl_xor(pl2, 16, 64);
            rr += __shfl_xor(rr, 16, 64);
            pl01 |= __shfl_xor(pl01, 32, 64);
            pl2 |= __shfl_xor(pl2, 32, 64);
            rr += __shfl_xor(rr, 32, 64);
            if (q == 0) s_rho[wv][i] = rr;
            // bit-plane p of these 16 coordinates is written by lane group p
            if (q < nb) {
                const uint32_t v = q == 0 ? (pl01 & 0xffffu) : (q == 1 ? (pl01 >> 16) : pl2);
                tw16[((buf * ENCR_WMAX * 16) + (cw_word + q * wpp) * 16 + i) * 2 + cw_half] = (uint16_t)v;
            }
        } else if (lane < 16) {
            s_rho[wv][lane] = 0.0;
        }
        lds_barrier();
        // the next tile's keys (loaded one tile ago) into the now free key buffer
        const long Tn = T + grid;
        if (Tn < total_tiles) {
            stage(Tn, kq, buf ^ 1);
            load_keys(Tn + grid, kq);
        }
        // stage 2: project the residual, keep the signs
        if (prj_live) {
            const f32x4 acc = encr_mma_n(nsp, rp, reinterpret_cast<const f32x4 *>(Uf) + lane);
            uint32_t sg = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) sg |= (acc[r] >= 0.0f ? 1u : 0u) << r;
            sg <<= 4 * q;
            sg |= __shfl_xor(sg, 16, 64);
            sg |= __shfl_xor(sg, 32, 64);
            if (q == 0) tw16[((buf * ENCR_WMAX * 16) + sw_word * 16 + i) * 2 + sw_half] = (uint16_t)sg;
        }
        // residual norm rho = |u| (fp64 sum of the waves' partial sums)
        if (wv == ENCR_WAVES - 1 && lane < 16) {
            double s = 0.0;
#pragma unroll
            for (int w = 0; w < ENCR_WAVES; ++w) s += s_rho[w][lane];
            rnorms[(size_t)bank * n_pad + (size_t)tile * 16 + lane] = (float)sqrt(s);
        }
        lds_barrier();
        // the tile's stored words: bits[bank][tile][W][16], one coalesced block
        if (tid < a.W * 4)
            reinterpret_cast<u32x4 *>(bits + (size_t)T * a.W * 16)[tid] =
                reinterpret_cast<const u32x4 *>(&TW[buf][0])[tid];
    }
}

}  // namespace tq
