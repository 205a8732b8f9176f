// Encoder for larger keys (d > 128 or m > 128, e.g. 768-dimensional search vectors), as two
// tiled GEMMs on the bf16 matrix cores with exact three-piece splits.
//
// turboquant-pytorch write-up (discuss.pytorch.kr), two-stage algorithm section: stage 1
// rotates each key and quantises every rotated coordinate against the Lloyd-Max codebook;
// stage 2 projects the stage-1 residual with a Gaussian matrix and keeps the signs.
//
// At these sizes the rotation and S' do not fit in registers or LDS, so both stages are
// plain tiled GEMMs over 128-key blocks (keys processed in chunks of EG_CHUNK rows):
//   stage 1: Y[coord][key] = R_g[coord][:] . x_g[key][:] per 128-coordinate tile; the
//            epilogue buckets y, writes the code words of its coordinates, the residual u
//            (fp32, into a workspace chunk) and per-tile partial sums of u^2;
//   stage 2: P[row][key] = S'[row][:] . u[key][:] per 128-row tile; the epilogue writes the
//            sign words, and the first row tile finishes |u| from the partial sums.
// Operands are split exactly into three bf16 pieces (see the register-resident encoder):
// R and S' once per call (enc_split3_kernel), keys and residuals as they are staged. The
// products kept are those of piece orders a + b <= 2; bf16 keys are exact in one piece.
//
// Work-group: 8 waves, a 128 x 128 output tile, K in steps of 32 through double-buffered
// LDS (A and B pieces in MFMA operand order, one ds_read_b128 per fragment). Wave w owns
// rows 64(w&1).. and keys 32(w>>1).. (4 x 2 MFMA blocks of 16 x 16). One LDS barrier per
// K step: the next step's operands are loaded to registers before the MFMAs and written
// to the other buffer after them.
#pragma once
#include "tq_encode.h"

namespace tq {

constexpr int EG_THREADS = 512, EG_TILE = 128, EG_KC = 32;
constexpr int EG_CHUNK = 32768;  // key rows per residual chunk (a multiple of EG_TILE)

// Three bf16 pieces of every element of src (count elements): dst[p * count + e].
__global__ __launch_bounds__(256) void enc_split3_kernel(const float *__restrict__ src, long count,
                                                         uint16_t *__restrict__ dst) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= count) return;
    uint32_t p0, p1, p2;
    split3_pair(src[e], 0.0f, p0, p1, p2);
    dst[e] = (uint16_t)p0;
    dst[count + e] = (uint16_t)p1;
    dst[2 * count + e] = (uint16_t)p2;
}

// Key row kl of a chunk starting at 16-key tile t0 -> (global tile, source key or -1).
struct EgRow {
    long tile;
    long src;  // bank * n + key, or -1 for a padding slot / past the end
};
__device__ __forceinline__ EgRow eg_row(long t0, int kl, int rows, int n_tiles, long n) {
    EgRow r{t0 + (kl >> 4), -1};
    if (kl < rows) {
        const long bank = r.tile / n_tiles, key = (r.tile - bank * n_tiles) * 16 + (kl & 15);
        if (key < n) r.src = bank * n + key;
    }
    return r;
}

// Block -> (key block, output tile), with the tiles of one key block on one XCD (blocks are
// dealt to the 8 XCDs round-robin), so they share the key block's reads in L2.
__device__ __forceinline__ void eg_block(int ntile, int &kblock, int &tile) {
    const int nb = gridDim.x, id = blockIdx.x;
    const int logical = (nb % 8 == 0) ? (id % 8) * (nb / 8) + id / 8 : id;
    tile = logical % ntile;
    kblock = logical / ntile;
}

// One K step of a wave's MFMA blocks from the LDS operand buffers. A: three bf16 pieces of
// the tile's 128 rows; B: XP pieces of its 128 key rows. acc[rb][kb]: rows 64 wr + 16 rb +
// 4q + r, keys 32 wk + 16 kb + i of the tile (lane 16q + i).
template <int XP>
struct EgOperands {
    u32x4 (*As)[3][8][64];
    u32x4 (*Bs)[XP][8][64];
};

template <int XP>
__device__ __forceinline__ void eg_mma(const EgOperands<XP> &op, int buf, int wr, int wk, int lane,
                                       f32x4 (&acc)[4][2]) {
    u32x4 bf[2][XP];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int p = 0; p < XP; ++p) bf[kb][p] = op.Bs[buf][p][2 * wk + kb][lane];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        u32x4 af[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) af[p] = op.As[buf][p][4 * wr + rb][lane];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x4 c = acc[rb][kb];
            if constexpr (XP == 1) {
                c = mfma_bf16(af[2], bf[kb][0], c);
                c = mfma_bf16(af[1], bf[kb][0], c);
                c = mfma_bf16(af[0], bf[kb][0], c);
            } else {
                c = mfma_bf16(af[0], bf[kb][2], c);
                c = mfma_bf16(af[1], bf[kb][1], c);
                c = mfma_bf16(af[2], bf[kb][0], c);
                c = mfma_bf16(af[0], bf[kb][1], c);
                c = mfma_bf16(af[1], bf[kb][0], c);
                c = mfma_bf16(af[0], bf[kb][0], c);
            }
            acc[rb][kb] = c;
        }
    }
}

// Stores this thread's 8 values of a B row (split into XP pieces) at its operand slot.
template <int XP>
__device__ __forceinline__ void eg_store_b(const float (&v)[8], u32x4 (*Bs)[8][64], int srow, int sk) {
    u32x4 pc[3];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (XP == 1) {
            pc[0][d] = (__float_as_uint(v[2 * d]) >> 16) | (__float_as_uint(v[2 * d + 1]) & 0xffff0000u);
        } else {
            uint32_t p0, p1, p2;
            split3_pair(v[2 * d], v[2 * d + 1], p0, p1, p2);
            pc[0][d] = p0;
            pc[1][d] = p1;
            pc[2][d] = p2;
        }
    }
#pragma unroll
    for (int p = 0; p < XP; ++p) Bs[p][srow >> 4][16 * sk + (srow & 15)] = pc[p];
}

__device__ __forceinline__ void eg_load_a(const uint16_t *__restrict__ ap, long a_rows, int K, int arow, int k0,
                                          int sk, bool live, u32x4 (&a)[3]) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
        a[p] = live ? *reinterpret_cast<const u32x4 *>(ap + ((size_t)p * a_rows + arow) * K + k0 + 8 * sk)
                    : u32x4{0, 0, 0, 0};
}

// ---- stage 1: rotation of group g, buckets, code words, residual chunk, |u|^2 partials
template <typename KT>
__global__ __launch_bounds__(EG_THREADS) void enc_gemm_rot_kernel(
    const KT *__restrict__ keys, const int *__restrict__ chan, const uint16_t *__restrict__ rp3, EncArgs a, int g,
    long t0, int rows, int n_tiles, long n, int jbase, float *__restrict__ U, float *__restrict__ rho_part,
    uint32_t *__restrict__ bits, void *__restrict__ norms) {
    constexpr int XP = sizeof(KT) == 2 ? 1 : 3;
    __shared__ __align__(16) u32x4 As[2][3][8][64];
    __shared__ __align__(16) u32x4 Bs[2][XP][8][64];
    __shared__ float s_inv[EG_TILE], s_coef[EG_TILE];
    __shared__ float s_cent[8];
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, i = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wv & 1, wk = wv >> 1;
    const int dg = a.gdim[g], off = a.goff[g], D = a.d, ng = a.ng, nb = a.gbits[g];
    const int ntile = (dg + EG_TILE - 1) / EG_TILE;
    int kblock, tile;
    eg_block(ntile, kblock, tile);
    const int kbase = kblock * EG_TILE, c0 = tile * EG_TILE;
    if (tid < 8) s_cent[tid] = a.cent[g][tid];

    // staging role: row srow of the A tile and of the B tile, K elements 8 sk ..
    const int srow = tid >> 2, sk = tid & 3;
    const bool a_live = c0 + srow < dg;
    const EgRow br = eg_row(t0, kbase + srow, rows, n_tiles, n);
    const KT *xrow = br.src >= 0 ? keys + (size_t)br.src * D : nullptr;
    double nsq = 0.0;  // |x_g|^2 of key row srow, this thread's share
    auto load_b = [&](int k0, float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        if (!xrow) return;
        const int kk = off + k0 + 8 * sk;
        if (!chan) {
            if constexpr (XP == 1) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(xrow + kk);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    v[2 * d] = __uint_as_float(w[d] << 16);
                    v[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
                }
            } else {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(xrow + kk);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(xrow + kk + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = w0[e];
                    v[4 + e] = w1[e];
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = chan[kk + e];
                v[e] = load_key<KT>(xrow + ((unsigned)c < (unsigned)D ? c : 0));
            }
        }
    };

    EgOperands<XP> op{As, Bs};
    f32x4 acc[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[rb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nk = dg / EG_KC;
    {
        u32x4 av[3];
        float bv[8];
        eg_load_a(rp3, dg, dg, c0 + srow, 0, sk, a_live, av);
        load_b(0, bv);
#pragma unroll
        for (int p = 0; p < 3; ++p) As[0][p][srow >> 4][16 * sk + (srow & 15)] = av[p];
#pragma unroll
        for (int e = 0; e < 8; ++e) nsq += (double)bv[e] * (double)bv[e];
        eg_store_b<XP>(bv, Bs[0], srow, sk);
    }
    lds_barrier();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        u32x4 av[3];
        float bv[8];
        const bool more = kc + 1 < nk;
        if (more) {
            eg_load_a(rp3, dg, dg, c0 + srow, (kc + 1) * EG_KC, sk, a_live, av);
            load_b((kc + 1) * EG_KC, bv);
        }
        eg_mma<XP>(op, buf, wr, wk, lane, acc);
        if (more) {
#pragma unroll
            for (int p = 0; p < 3; ++p) As[buf ^ 1][p][srow >> 4][16 * sk + (srow & 15)] = av[p];
#pragma unroll
            for (int e = 0; e < 8; ++e) nsq += (double)bv[e] * (double)bv[e];
            eg_store_b<XP>(bv, Bs[buf ^ 1], srow, sk);
        }
        lds_barrier();
    }

    // norms of the tile's key rows (fp64 sums of exact float squares)
    nsq += __shfl_xor(nsq, 1, 64);
    nsq += __shfl_xor(nsq, 2, 64);
    if (sk == 0) {
        const double nu = sqrt(nsq);
        // the stored norm (float32, or its binary16 rounding): the reconstruction, and so
        // the residual, use it; the rotated coordinates use the unrounded norm
        const float nu_f = (float)nu;
        const uint16_t nu_h = f32_to_binary16(nu_f);
        const float nu_s = a.nh ? norm_f32(nu_h) : nu_f;
        s_inv[srow] = nu > 0.0 ? (float)(a.sqrt_d[g] / nu) : 0.0f;
        s_coef[srow] = (float)((double)nu_s / a.sqrt_d[g]);
        if (tile == 0 && kbase + srow < rows) {
            const size_t at = ((size_t)br.tile * 16 + (srow & 15)) * ng + g;
            if (a.nh)
                static_cast<uint16_t *>(norms)[at] = nu_h;
            else
                static_cast<float *>(norms)[at] = nu_f;
        }
    }
    float th[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) th[t] = t < (1 << nb) - 1 ? a.thr[g][t] : INFINITY;
    lds_barrier();

    // epilogue: lane (q, i) of block (rb, kb) holds coordinates 64 wr + 16 rb + 4q + r of
    // key 32 wk + 16 kb + i
    const int W = a.W, wpp = dg / 32;
    float rr[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int kl = kbase + 32 * wk + 16 * kb + i;
        const bool row_live = kl < rows;
        const long T = t0 + (kl >> 4);
        const float inv = s_inv[32 * wk + 16 * kb + i], coef = s_coef[32 * wk + 16 * kb + i];
        uint32_t half[4][3];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int crow = c0 + 64 * wr + 16 * rb;  // first coordinate (in the group) of the block
            float u[4];
            uint32_t pl[3];
            if (nb == 1)
                encr_bucket<1>(acc[rb][kb], inv, coef, th, s_cent, u, pl);
            else if (nb == 2)
                encr_bucket<2>(acc[rb][kb], inv, coef, th, s_cent, u, pl);
            else
                encr_bucket<3>(acc[rb][kb], inv, coef, th, s_cent, u, pl);
            if (crow < dg) {
                if (row_live)
                    *reinterpret_cast<f32x4 *>(U + (size_t)kl * D + off + crow + 4 * q) = f32x4{u[0], u[1], u[2], u[3]};
#pragma unroll
                for (int r = 0; r < 4; ++r) rr[kb] = fmaf(u[r], u[r], rr[kb]);
            }
#pragma unroll
            for (int p = 0; p < 3; ++p) half[rb][p] = or_rows32(or_rows16(pl[p] << (4 * q)));
        }
        // code words: blocks (0, 1) and (2, 3) are the two halves of a 32-coordinate word
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int crow = c0 + 64 * wr + 32 * h;
            if (crow < dg && row_live && q < nb) {
                const uint32_t wd = q == 0 ? (half[2 * h][0] | (half[2 * h + 1][0] << 16))
                                           : (q == 1 ? (half[2 * h][1] | (half[2 * h + 1][1] << 16))
                                                     : (half[2 * h][2] | (half[2 * h + 1][2] << 16)));
                const int w = a.gword[g] + q * wpp + (crow >> 5);
                bits[((size_t)T * W + w) * 16 + (kl & 15)] = wd;
            }
        }
    }
    // |u|^2 partial of this wave's 64 coordinates, per key
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const float s = add_rows32(add_rows16(rr[kb]));
        const int kl = kbase + 32 * wk + 16 * kb + i;
        if (q == 0 && kl < rows) rho_part[(size_t)(jbase + 2 * tile + wr) * EG_CHUNK + kl] = s;
    }
}

// ---- stage 2: projection of the residual chunk, sign words, residual norms
__global__ __launch_bounds__(EG_THREADS) void enc_gemm_prj_kernel(const float *__restrict__ U,
                                                                  const uint16_t *__restrict__ sp3, EncArgs a,
                                                                  long t0, int rows, int J,
                                                                  const float *__restrict__ rho_part,
                                                                  uint32_t *__restrict__ bits,
                                                                  void *__restrict__ rnorms) {
    __shared__ __align__(16) u32x4 As[2][3][8][64];
    __shared__ __align__(16) u32x4 Bs[2][3][8][64];
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, i = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wv & 1, wk = wv >> 1;
    const int D = a.d, M = a.m;
    const int ntile = (M + EG_TILE - 1) / EG_TILE;
    int kblock, tile;
    eg_block(ntile, kblock, tile);
    const int kbase = kblock * EG_TILE, r0 = tile * EG_TILE;

    const int srow = tid >> 2, sk = tid & 3;
    const bool a_live = r0 + srow < M;
    const bool b_live = kbase + srow < rows;
    const float *urow = U + (size_t)(kbase + srow) * D;
    auto load_b = [&](int k0, float (&v)[8]) {
        if (b_live) {
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(urow + k0 + 8 * sk);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(urow + k0 + 8 * sk + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = w0[e];
                v[4 + e] = w1[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
    };

    EgOperands<3> op{As, Bs};
    f32x4 acc[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[rb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nk = D / EG_KC;
    {
        u32x4 av[3];
        float bv[8];
        eg_load_a(sp3, M, D, r0 + srow, 0, sk, a_live, av);
        load_b(0, bv);
#pragma unroll
        for (int p = 0; p < 3; ++p) As[0][p][srow >> 4][16 * sk + (srow & 15)] = av[p];
        eg_store_b<3>(bv, Bs[0], srow, sk);
    }
    lds_barrier();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        u32x4 av[3];
        float bv[8];
        const bool more = kc + 1 < nk;
        if (more) {
            eg_load_a(sp3, M, D, r0 + srow, (kc + 1) * EG_KC, sk, a_live, av);
            load_b((kc + 1) * EG_KC, bv);
        }
        eg_mma<3>(op, buf, wr, wk, lane, acc);
        if (more) {
#pragma unroll
            for (int p = 0; p < 3; ++p) As[buf ^ 1][p][srow >> 4][16 * sk + (srow & 15)] = av[p];
            eg_store_b<3>(bv, Bs[buf ^ 1], srow, sk);
        }
        lds_barrier();
    }

    // sign words: lane (q, i) of block (rb, kb) holds rows 64 wr + 16 rb + 4q + r of key
    // 32 wk + 16 kb + i
    const int W = a.W;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int kl = kbase + 32 * wk + 16 * kb + i;
        const long T = t0 + (kl >> 4);
        uint32_t half[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            uint32_t sg = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) sg |= (acc[rb][kb][r] >= 0.0f ? 1u : 0u) << r;
            half[rb] = or_rows32(or_rows16(sg << (4 * q)));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = r0 + 64 * wr + 32 * h;
            if (row < M && kl < rows && q == 0)
                bits[((size_t)T * W + a.sword + (row >> 5)) * 16 + (kl & 15)] = half[2 * h] | (half[2 * h + 1] << 16);
        }
    }
    // residual norms, from the stage-1 partial sums in a fixed order
    if (tile == 0 && tid < EG_TILE) {
        const int kl = kbase + tid;
        if (kl < rows) {
            double s = 0.0;
            for (int j = 0; j < J; ++j) s += (double)rho_part[(size_t)j * EG_CHUNK + kl];
            const size_t at = (size_t)(t0 + (kl >> 4)) * 16 + (kl & 15);
            const float rv = (float)sqrt(s);
            if (a.nh)
                static_cast<uint16_t *>(rnorms)[at] = f32_to_binary16(rv);
            else
                static_cast<float *>(rnorms)[at] = rv;
        }
    }
}

}  // namespace tq
