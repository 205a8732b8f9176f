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
constexpr int AT_CHUNK = 512;                  // keys per work-group
constexpr int AT_STEPS = AT_CHUNK / AT_STEP;
constexpr int AT_RPL = AT_CHUNK / 256;         // weights per lane and key of a quad: keys 256 r + 4 lane + k
constexpr int AT_DMAX = 128;                   // value dimension: one 32-coordinate word per wave

struct AttnArgs {
    int d, ng, W;                  // value dimension, channel groups, stored words per value
    int gdim[2], goff[2], gbits[2], gword[2];
    double coef[2][4];             // 2 a_P per group, planes: bit 0, bit 1, bit 2, xor of the three
    double bias[2];                // sum_P a_P per group
    double inv_sqrt_d[2];
};

__device__ __forceinline__ float at_wave_max(float v) { return dpp_wave_max_f32(v); }
__device__ __forceinline__ double at_wave_sum(double v) { return dpp_wave_sum_f64(v); }

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

typedef __attribute__((address_space(3))) void at_lds_void;

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int AT_WAIT_VM0 = (7 << 4) | (15 << 8);

// Partial attention of one chunk of AT_CHUNK keys for four queries of one bank.
// grid (banks * chunks, ceil(G / 4)), AT_THREADS threads. Wave q computes the weights of
// query 4 * blockIdx.y + q; wave w accumulates coordinate word w (32 coordinates, group
// order) for the four queries.
// part [bank][G][chunks][2 + d] floats: maximum of z = log2(e) scale logit, sum of
// 2^(z - max), then o_rot (un-normalised, relative to that maximum).
//
// Memory: at entry every wave issues direct-to-LDS loads (global_load_lds_dwordx4) of its
// word's stored planes for all tiles of the chunk, then the logits and norms of its
// query; one wait covers them all, so a work-group costs one memory round trip and the
// products run from LDS.
// NH: the value bank stores binary16 norms. GB: the code width of a one-group value bank
// fixed at compile time (0: read from the arguments).
template <int NG, bool NH, int GB>
__global__ __launch_bounds__(AT_THREADS) void attn_chunk_kernel(
    const float *__restrict__ scores, const uint32_t *__restrict__ vbits, const void *__restrict__ vnorms, long n,
    int n_tiles, int G, int chunks, float scale, const int32_t *__restrict__ lengths, AttnArgs a,
    float *__restrict__ part) {
    constexpr int TILES = AT_CHUNK / 16;
    __shared__ __align__(16) uint32_t s_v[4][TILES * 3][16];    // [wave][tile * planes + p][key]: stored words
    // rows padded by 16 bytes (s_a) and 4 dwords (s_b): the operand reads and the staging
    // writes then spread over all LDS banks
    __shared__ __align__(16) uint8_t s_a[NG][16][AT_CHUNK + 16];     // [group][row 4q + limb][key]: limbs
    __shared__ __align__(16) uint32_t s_b[4][16][AT_STEP / 4 + 4];  // [wave][column 4P + byte][4 keys]
    __shared__ int s_F[NG][4];
    __shared__ double s_vsum[NG][4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long bank = blockIdx.x / chunks;
    const int ch = blockIdx.x % chunks;
    const int q0 = 4 * blockIdx.y;
    const long k0 = (long)ch * AT_CHUNK;
    const long n_pad = (long)n_tiles * 16;
    const int PS = 2 + a.d;
    const int t_first = (int)(k0 >> 4);

    // ---- 0. this wave's coordinate word: group, planes, and the direct loads of its planes
    const int nwords = a.d >> 5;
    const bool wlive = wv < nwords;
    const int g = (NG > 1 && 32 * wv >= a.gdim[0]) ? 1 : 0;
    static_assert(GB == 0 || NG == 1, "a fixed code width needs one channel group");
    const int gb = GB ? GB : a.gbits[g];
    const int pstride = a.gdim[g] >> 5;
    const int wbase = a.gword[g] + wv - (a.goff[g] >> 5);
    const uint32_t *vb = vbits + (size_t)bank * n_tiles * a.W * 16;
    if (wlive) {
        // rows tile * gb + p of 64 bytes (16 keys x one word), sixteen rows per load; tiles
        // past the bank's end re-read its last tile (their keys carry zero weight)
        for (int i = 0; i < AT_RPL * gb; ++i) {
            const int row = 16 * i + (lane >> 2);
            const int rt = gb == 1 ? row : (gb == 2 ? row >> 1 : (row * 43691) >> 17);  // row / gb
            const int tile = min(t_first + rt, n_tiles - 1), p = row - rt * gb;
            __builtin_amdgcn_global_load_lds(vb + ((size_t)tile * a.W + wbase + p * pstride) * 16 + 4 * (lane & 3),
                                             (at_lds_void *)&s_v[wv][16 * i][0], 16, 0,
                                             2);  // nt: each value row is read once
        }
    }

    // ---- 1. weights of query q0 + wv; lane: keys 256 r + 4 lane + (0..3) of the chunk.
    // Exponents in base 2: z = log2(e) scale logit, e = 2^(z - max z) (v_exp_f32); the chunk
    // maximum is stored in the same units.
    {
        const int qg = q0 + wv;
        const bool qlive = qg < G;                       // wave-uniform
        const int nk = (int)min((long)AT_CHUNK, n - k0);  // keys of this chunk in memory, >= 1
        const int nkp = (int)min((long)AT_CHUNK, n_pad - k0);
        // keys that take part: the bank's first lengths[bank] (all n without lengths)
        const long len = lengths ? min((long)max(lengths[bank], 0), n) : n;
        const int nkv = (int)max(min((long)AT_CHUNK, len - k0), 0L);
        const float *sb = scores + ((size_t)bank * G + (qlive ? qg : 0)) * n + k0;
        const size_t nbase = ((size_t)bank * n_pad + k0) * NG;
        // loads at clamped addresses, all issued before the first wait (no branch around a
        // load: each would wait on its own)
        f32x4 nv[AT_RPL][NG];  // norms of keys 4 lane .. 4 lane + 3 (groups interleaved per key)
        u32x4 nraw[AT_RPL];    // the same as binary16 pairs (4 NG halves), widened after the wait
#pragma unroll
        for (int r = 0; r < AT_RPL; ++r) {
            const int kb = min(256 * r + 4 * lane, nkp - 4);
            if constexpr (NH) {
                const uint16_t *nb = static_cast<const uint16_t *>(vnorms) + nbase;
                if constexpr (NG == 1) {
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(nb + kb);
                    nraw[r] = u32x4{v.x, v.y, 0u, 0u};
                } else {
                    nraw[r] = *reinterpret_cast<const u32x4 *>(nb + kb * NG);
                }
            } else {
                const float *nb = static_cast<const float *>(vnorms) + nbase;
#pragma unroll
                for (int h = 0; h < NG; ++h) nv[r][h] = reinterpret_cast<const f32x4 *>(nb + kb * NG)[h];
            }
        }
        float e[AT_RPL][4];
#pragma unroll
        for (int r = 0; r < AT_RPL; ++r)
#pragma unroll
            for (int k = 0; k < 4; ++k) e[r][k] = sb[min(256 * r + 4 * lane + k, nk - 1)];
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NH) {
            // half e of a lane's block is norm (key e / NG, group e % NG), as float e above
#pragma unroll
            for (int r = 0; r < AT_RPL; ++r)
#pragma unroll
                for (int h = 0; h < NG; ++h) {
                    const uint32_t w0 = nraw[r][2 * h], w1 = nraw[r][2 * h + 1];
                    nv[r][h] = f32x4{norm_f32((uint16_t)w0), norm_f32((uint16_t)(w0 >> 16)),
                                     norm_f32((uint16_t)w1), norm_f32((uint16_t)(w1 >> 16))};
                }
        }
        const float c2 = scale * 1.4426950408889634f;
        float mx = -INFINITY;
        if (nkv == AT_CHUNK) {
#pragma unroll
            for (int r = 0; r < AT_RPL; ++r)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    e[r][k] *= c2;
                    mx = fmaxf(mx, e[r][k]);
                }
        } else {
#pragma unroll
            for (int r = 0; r < AT_RPL; ++r)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    e[r][k] = 256 * r + 4 * lane + k < nkv ? e[r][k] * c2 : -INFINITY;
                    mx = fmaxf(mx, e[r][k]);
                }
        }
        mx = at_wave_max(mx);
        const bool live = qlive && mx != -INFINITY;  // a query and at least one key
        double esum = 0.0;
#pragma unroll
        for (int r = 0; r < AT_RPL; ++r) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                e[r][k] = live ? __builtin_amdgcn_exp2f(e[r][k] - mx) : 0.0f;  // 2^-inf = 0
            // pairwise in fp32 (relative error <= 2^-23), then fp64
            esum += (double)((e[r][0] + e[r][1]) + (e[r][2] + e[r][3]));
        }
        esum = at_wave_sum(esum);
        if (qlive && lane == 0) {
            float *pp = part + (((size_t)bank * G + qg) * chunks + ch) * PS;
            pp[0] = mx;
            pp[1] = (float)esum;
        }
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            float w[AT_RPL][4];
            float wm = 0.0f;
#pragma unroll
            for (int r = 0; r < AT_RPL; ++r)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    // norm (key k, group gg) is float NG k + gg of the lane's block; keys that
                    // take no part have e = 0 and whatever their slot holds as norm
                    const float nu = nv[r][(NG * k + gg) >> 2][(NG * k + gg) & 3];
                    w[r][k] = e[r][k] > 0.0f ? e[r][k] * nu : 0.0f;
                    wm = fmaxf(wm, w[r][k]);
                }
            wm = at_wave_max(wm);
            // fixed point: w 2^F < 2^30 for every weight of the chunk
            int E = 0;
            if (wm > 0.0f) frexpf(wm, &E);
            const int F = wm > 0.0f ? 30 - E : 0;
            double vsum = 0.0;  // exact: at most 2^40
#pragma unroll
            for (int r = 0; r < AT_RPL; ++r) {
                u32x4 L;
                uint32_t V[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    V[k] = (uint32_t)__float2int_rn(ldexpf(w[r][k], F));
                    // balanced base-256 digits: bytes of V + 0x80808080, each minus 128
                    L[k] = (V[k] + 0x80808080u) ^ 0x80808080u;
                }
                vsum += (double)(V[0] + V[1]) + (double)(V[2] + V[3]);  // pairs < 2^31: exact
                // limb l of the four keys -> row 4 wv + l
                const u32x4 y = at_transpose_bytes(L);
#pragma unroll
                for (int l = 0; l < 4; ++l)
                    *reinterpret_cast<uint32_t *>(&s_a[gg][4 * wv + l][256 * r + 4 * lane]) = y[l];
            }
            vsum = at_wave_sum(vsum);
            if (lane == 0) {
                s_F[gg][wv] = F;
                s_vsum[gg][wv] = vsum;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(AT_WAIT_VM0);  // this wave's planes are in LDS
    __syncthreads();

    // ---- 2. wave wv: coordinate word wv of the four queries
    if (wlive) {
        // staging role of this lane: tile T of the step, keys 4 s4 .. 4 s4 + 3, plane P; a
        // stored plane P reads its row (and, for the XOR of three planes, the XOR plane reads
        // planes 0, 1, 2); unused columns (coefficient 0) read plane 0
        const int T = lane >> 4, s4 = (lane >> 2) & 3, P = lane & 3;
        const int pa = P < gb ? P : 0;
        const int pb = P < gb ? P : (P == 3 && gb == 3 ? 1 : 0);
        const int pc = P < gb ? P : (P == 3 && gb == 3 ? 2 : 0);

        i32x4 acc[8];
    #pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = i32x4{0, 0, 0, 0};
        const int col = lane & 15, kg = lane >> 4;
        for (int s = 0; s < AT_STEPS; ++s) {
            const int rt = (4 * s + T) * gb;
            u32x4 x = *(const u32x4 *)&s_v[wv][rt + pa][4 * s4];
            if (gb == 3) x ^= *(const u32x4 *)&s_v[wv][rt + pb][4 * s4] ^ *(const u32x4 *)&s_v[wv][rt + pc][4 * s4];
            const u32x4 y = at_transpose_bytes(x);
    #pragma unroll
            for (int b = 0; b < 4; ++b) s_b[wv][4 * P + b][4 * T + s4] = y[b];
            const i8x16 A = *(const i8x16 *)&s_a[g][col][AT_STEP * s + 16 * kg];
            const u32x4 B = *(const u32x4 *)&s_b[wv][col][4 * kg];
    #pragma unroll
            for (int t = 0; t < 8; ++t) {
                const u32x4 bt = B & (0x01010101u << t);
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, __builtin_bit_cast(i8x16, bt), acc[t], 0, 0, 0);
            }
        }

        // ---- 3. recombine: lane (query c, column 4P + b) turns its limb sums into one fp64
        // plane term per shift t; through the wave's (now free) staging LDS, lane (c, b, t0)
        // then adds the four planes of coordinates 8b + t0 and 8b + t0 + 4 and stores them
        {
            const int Pc = col >> 2;
            const double *cf = g ? a.coef[1] : a.coef[0];
            const double coef = Pc == 0 ? cf[0] : (Pc == 1 ? cf[1] : (Pc == 2 ? cf[2] : cf[3]));
            double *so = reinterpret_cast<double *>(&s_v[wv][0][0]);  // [8][64], 4 KB of the wave's 6 KB
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                // exact: |limb sum| <= AT_CHUNK * 128 * 128
                const double v = fma((double)acc[t][3], 16777216.0,
                                     fma((double)acc[t][2], 65536.0, fma((double)acc[t][1], 256.0, (double)acc[t][0])));
                so[64 * t + lane] = v * (coef * (t == 7 ? -1.0 / 128.0 : 1.0 / (double)(1 << t)));
            }
            const int c = lane >> 4, bc = (lane >> 2) & 3, t0 = lane & 3;
            const int qg = q0 + c;
            const double fscale = ldexp(a.inv_sqrt_d[g], -s_F[g][c]);
            const double bterm = a.bias[g] * s_vsum[g][c];
            float *prow = part + (((size_t)bank * G + (qg < G ? qg : 0)) * chunks + ch) * PS + 2 + 32 * wv + 8 * bc;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = t0 + 4 * h;
                const double *r = so + 64 * t + 16 * c + bc;
                const double xv = (r[0] + r[4]) + (r[8] + r[12]);  // planes 0..3 of (c, b)
                if (qg < G) prow[t] = (float)((xv - bterm) * fscale);
            }
        }
    }
}

// Merge of the chunks and the rotation back: one work-group of AT_MERGE_WAVES waves per
// (bank, query). Every wave reads all chunk maxima and weight sums (so each holds the same
// global maximum and total) and the partial rows of its own chunks c = AT_MERGE_WAVES i + wave
// (two coordinates per lane), each pass's reads issued before its first wait, beside its share
// of the rotation R_g (direct-to-LDS). The chunk maxima (base-2 units) give factors
// 2^(max_c - max); the waves' sums of factor_c o_rot_c add in LDS in wave order (fp64);
// o_rot = that / sum_c factor_c sum_c; then thread k forms
// out[chan[off_g + k]] = sum_j R_g[j][k] o_rot[off_g + j]. out [bank][G][d] float32.
constexpr int AT_MERGE_WAVES = 4;

__global__ __launch_bounds__(AT_MERGE_WAVES * 64) void attn_combine_kernel(const float *__restrict__ part, int chunks,
                                                                          const float *__restrict__ rot,
                                                                          const int *__restrict__ chan, AttnArgs a,
                                                                          float *__restrict__ out) {
    constexpr int MW = AT_MERGE_WAVES, PER = 64 / MW;  // a wave's chunks in a pass of 64
    __shared__ __align__(16) float s_R[AT_DMAX * AT_DMAX];
    __shared__ double s_v[MW][AT_DMAX];
    __shared__ double s_o[AT_DMAX];
    const int tid = threadIdx.x, lane = tid & 63, d = a.d, PS = 2 + d;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const float *pq = part + (size_t)blockIdx.x * chunks * PS;
    // the rotation blocks, back to back: d_0^2 (+ d_1^2) floats, a multiple of 256
    const int nR = a.gdim[0] * a.gdim[0] + (a.ng > 1 ? a.gdim[1] * a.gdim[1] : 0);
    for (int i = wv; i < nR / 256; i += MW)
        __builtin_amdgcn_global_load_lds(rot + 256 * i + 4 * lane, (at_lds_void *)&s_R[256 * i], 16, 0, 0);
    const int k0 = min(lane, d - 1), k1 = min(lane + 64, d - 1);  // clamped reads; results unused
    float pv0[PER], pv1[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float *pr = pq + (size_t)min(MW * i + wv, chunks - 1) * PS + 2;
        pv0[i] = pr[k0];
        pv1[i] = pr[k1];
    }
    const int c0 = min(lane, chunks - 1);
    const float m0 = pq[(size_t)c0 * PS], e0 = pq[(size_t)c0 * PS + 1];
    __builtin_amdgcn_sched_barrier(0);
    float mx = lane < chunks ? m0 : -INFINITY;
    for (int c = lane + 64; c < chunks; c += 64) mx = fmaxf(mx, pq[(size_t)c * PS]);
    mx = at_wave_max(mx);
    double tot = 0.0, v0 = 0.0, v1 = 0.0;
    for (int cb = 0; cb < chunks; cb += 64) {
        float f, e;
        if (cb == 0) {
            f = lane < chunks ? m0 : -INFINITY;
            e = e0;
        } else {
            const int c = min(cb + lane, chunks - 1);
            f = cb + lane < chunks ? pq[(size_t)c * PS] : -INFINITY;
            e = pq[(size_t)c * PS + 1];
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const float *pr = pq + (size_t)min(cb + MW * i + wv, chunks - 1) * PS + 2;
                pv0[i] = pr[k0];
                pv1[i] = pr[k1];
            }
        }
        f = __builtin_amdgcn_exp2f(f - mx);  // 0 past the last chunk
        tot += (double)f * (double)e;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const double fi = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), MW * i + wv));
            v0 += fi * (double)pv0[i];
            v1 += fi * (double)pv1[i];
        }
    }
    tot = at_wave_sum(tot);  // the same in every wave
    if (mx == -INFINITY) tot = 0.0, v0 = v1 = 0.0;  // no key took part: the output is 0
    s_v[wv][lane] = v0;
    s_v[wv][lane + 64] = v1;
    __builtin_amdgcn_s_waitcnt(AT_WAIT_VM0);  // this wave's share of the rotation is in LDS
    __syncthreads();
    if (tid < AT_DMAX) {
        double v = 0.0;
#pragma unroll
        for (int w = 0; w < MW; ++w) v += s_v[w][tid];
        s_o[tid] = tot > 0.0 ? v / tot : 0.0;
    }
    __syncthreads();
    const int k = tid;
    if (k < d) {
        const bool g1 = a.ng > 1 && k >= a.gdim[0];
        const int dg = g1 ? a.gdim[1] : a.gdim[0], off = g1 ? a.goff[1] : 0, kk = k - off;
        const float *R = s_R + (g1 ? a.gdim[0] * a.gdim[0] : 0) + kk;
        double r = 0.0;
#pragma unroll 16
        for (int j = 0; j < dg; ++j) r += (double)R[j * dg] * s_o[off + j];
        out[(size_t)blockIdx.x * d + (chan ? chan[k] : k)] = (float)r;
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
    int nh;  // 1: binary16 norms
};

__global__ __launch_bounds__(256) void decode_kernel(const uint32_t *__restrict__ bits, const void *__restrict__ norms,
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
        const size_t ni = ((size_t)bank * n_pad + 16 * t + i) * a.ng + g;
        const float nu = a.nh ? norm_f32(static_cast<const uint16_t *>(norms)[ni]) : static_cast<const float *>(norms)[ni];
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
