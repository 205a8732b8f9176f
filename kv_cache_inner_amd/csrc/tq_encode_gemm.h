// Encoder for larger keys (d > 128 or m > 128, e.g. 768-dimensional search vectors), as two
// tiled GEMMs on the bf16 matrix cores with exact three-piece splits.
//
// turboquant-pytorch write-up (discuss.pytorch.kr), two-stage algorithm section: stage 1
// rotates each key and quantises every rotated coordinate against the Lloyd-Max codebook;
// stage 2 projects the stage-1 residual with a Gaussian matrix and keeps the signs.
//
// At these sizes the rotation and S' do not fit in registers or LDS, so both stages are
// plain tiled GEMMs over 256-key blocks (keys processed in chunks of EG_CHUNK rows):
//   stage 1: Y[coord][key] = R_g[coord][:] . x_g[key][:] per 128-coordinate tile; the
//            epilogue buckets y, writes the code words of its coordinates, the residual u
//            (fp32, into a workspace chunk) and per-tile partial sums of u^2;
//   stage 2: P[row][key] = S'[row][:] . u[key][:] per 128-row tile; the epilogue writes the
//            sign words, and the first row tile finishes |u| from the partial sums.
// Operands are split exactly into three bf16 pieces (see the register-resident encoder):
// R and S' once per call (enc_split3_kernel), keys and residuals as they are staged. The
// products kept are those of piece orders a + b <= 2; bf16 keys are exact in one piece.
//
// Work-group: 8 waves, a 128-row x 256-key output tile, K in steps of 32 through
// double-buffered LDS (A and B pieces in MFMA operand order, one ds_read_b128 per fragment).
// Wave w owns rows 64(w&1).. and keys 64(w>>1).. (4 x 4 MFMA blocks of 16 x 16), so each
// fragment read from LDS feeds four MFMAs (with 64 x 32 per wave, two: 16 % slower over the
// two stages at d = m = 768, the LDS reads and the MFMAs then alternating more than they
// overlap). One LDS barrier per K step: the next step's operands are loaded to registers
// before the MFMAs and written to the other buffer after them.
#pragma once
#include "tq_encode.h"

namespace tq {

constexpr int EG_THREADS = 512, EG_TILE = 128, EG_KC = 32;
constexpr int EG_KT = 256;  // key rows per work-group tile
constexpr int EG_CHUNK = 32768;  // key rows per residual chunk (a multiple of EG_KT)

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

// Slot of (row r of a 16-row block, K slot sk) in the block's 64 16-byte operand slots: the
// MFMA lane 16 sk + r, with bits 2-3 of r flipped by sk. Lane l reads slot l ^ (4 (l >> 4)),
// a permutation inside each 16-lane group; the staging threads (four K slots of one row
// in consecutive lanes) then write 16 distinct slots per 16 lanes instead of 4 each 256 B
// apart.
__device__ __forceinline__ int eg_slot(int r, int sk) { return 16 * sk + ((r & 15) ^ (4 * sk)); }

// Stores this thread's 8 values of a B row (split into XP pieces) at its operand slot.
template <int XP, int NBLK = 8>
__device__ __forceinline__ void eg_store_b(const float (&v)[8], u32x4 (*Bs)[NBLK][64], int srow, int sk) {
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
    for (int p = 0; p < XP; ++p) Bs[p][srow >> 4][eg_slot(srow, sk)] = pc[p];
}

// One K step of a wave's 4 x 4 MFMA blocks (64 rows x 64 keys) from the LDS operand buffers
// of a 128-row x 256-key tile: acc[rb][kb] holds rows 64 wr + 16 rb + 4q + r, keys
// 64 wk + 16 kb + i (lane 16q + i). Every fragment read from LDS feeds four MFMAs.
template <int XP>
__device__ __forceinline__ void eg_mma4(const u32x4 (*As)[8][64], const u32x4 (*Bs)[16][64], int wr, int wk, int lane,
                                        f32x4 (&acc)[4][4]) {
    const int sl = lane ^ (4 * (lane >> 4));  // eg_slot of this lane's fragment
    u32x4 bf[4][XP];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int p = 0; p < XP; ++p) bf[kb][p] = Bs[p][4 * wk + kb][sl];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        u32x4 af[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) af[p] = As[p][4 * wr + rb][sl];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
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

__device__ __forceinline__ void eg_load_a(const uint16_t *__restrict__ ap, long a_rows, int K, int arow, int k0,
                                          int sk, bool live, u32x4 (&a)[3]) {
#pragma unroll
    for (int p = 0; p < 3; ++p)
        a[p] = live ? *reinterpret_cast<const u32x4 *>(ap + ((size_t)p * a_rows + arow) * K + k0 + 8 * sk)
                    : u32x4{0, 0, 0, 0};
}

// ---- stage 1: rotation of group g, buckets, code words, residual chunk, |u|^2 partials
// Work-group tile: 128 coordinates x EG_KT = 256 keys; wave w owns coordinates 64 (w & 1)..
// and keys 64 (w >> 1).. (4 x 4 MFMA blocks of 16 x 16): each fragment read from LDS feeds
// four MFMAs. DT: the dimension of a one-group layout with d = m fixed at compile time (0: read
// from the arguments); the d = m = 768 instance encodes search keys about 5 % faster, bytes unchanged.
template <typename KT, int DT = 0>
__global__ __launch_bounds__(EG_THREADS) void enc_gemm_rot_kernel(
    const KT *__restrict__ keys, const int *__restrict__ chan, const uint16_t *__restrict__ rp3, EncArgs a, int g,
    long t0, int rows, int n_tiles, long n, int jbase, float *__restrict__ U, float *__restrict__ rho_part,
    uint32_t *__restrict__ bits, void *__restrict__ norms) {
    constexpr int XP = sizeof(KT) == 2 ? 1 : 3;
    __shared__ __align__(16) u32x4 As[2][3][8][64];
    __shared__ __align__(16) u32x4 Bs[2][XP][16][64];
    __shared__ float s_inv[EG_KT], s_coef[EG_KT];
    __shared__ float s_cent[8];
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, i = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wv & 1, wk = wv >> 1;
    const int dg = DT ? DT : a.gdim[g], off = DT ? 0 : a.goff[g], D = DT ? DT : a.d, ng = DT ? 1 : a.ng;
    const int nb = a.gbits[g];
    const int ntile = (dg + EG_TILE - 1) / EG_TILE;
    int kblock, tile;
    eg_block(ntile, kblock, tile);
    const int kbase = kblock * EG_KT, c0 = tile * EG_TILE;
    if (tid < 8) s_cent[tid] = a.cent[g][tid];

    // staging role: row srow of the A tile, rows srow and srow + 128 of the B tile, K
    // elements 8 sk ..
    const int srow = tid >> 2, sk = tid & 3;
    const bool a_live = c0 + srow < dg;
    EgRow br[2];
    const KT *xrow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        br[h] = eg_row(t0, kbase + srow + 128 * h, rows, n_tiles, n);
        xrow[h] = br[h].src >= 0 ? keys + (size_t)br[h].src * D : nullptr;
    }
    double nsq[2] = {0.0, 0.0};  // |x_g|^2 of key rows srow, srow + 128: this thread's share
    auto load_b = [&](const KT *xr, int k0, float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        if (!xr) return;
        const int kk = off + k0 + 8 * sk;
        if (!chan) {
            if constexpr (XP == 1) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(xr + kk);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    v[2 * d] = __uint_as_float(w[d] << 16);
                    v[2 * d + 1] = __uint_as_float(w[d] & 0xffff0000u);
                }
            } else {
                const f32x4 w0 = *reinterpret_cast<const f32x4 *>(xr + kk);
                const f32x4 w1 = *reinterpret_cast<const f32x4 *>(xr + kk + 4);
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
                v[e] = load_key<KT>(xr + ((unsigned)c < (unsigned)D ? c : 0));
            }
        }
    };
    auto stage = [&](int buf, const u32x4 (&av)[3], const float (&bv)[2][8]) {
#pragma unroll
        for (int p = 0; p < 3; ++p) As[buf][p][srow >> 4][eg_slot(srow, sk)] = av[p];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) nsq[h] += (double)bv[h][e] * (double)bv[h][e];
            eg_store_b<XP, 16>(bv[h], Bs[buf], srow + 128 * h, sk);
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[rb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nk = dg / EG_KC;
    {
        u32x4 av[3];
        float bv[2][8];
        eg_load_a(rp3, dg, dg, c0 + srow, 0, sk, a_live, av);
        load_b(xrow[0], 0, bv[0]);
        load_b(xrow[1], 0, bv[1]);
        stage(0, av, bv);
    }
    lds_barrier();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        u32x4 av[3];
        float bv[2][8];
        const bool more = kc + 1 < nk;
        if (more) {
            eg_load_a(rp3, dg, dg, c0 + srow, (kc + 1) * EG_KC, sk, a_live, av);
            load_b(xrow[0], (kc + 1) * EG_KC, bv[0]);
            load_b(xrow[1], (kc + 1) * EG_KC, bv[1]);
        }
        eg_mma4<XP>(As[buf], Bs[buf], wr, wk, lane, acc);
        if (more) stage(buf ^ 1, av, bv);
        lds_barrier();
    }

    // norms of the tile's key rows (fp64 sums of exact float squares)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        double ns = nsq[h];
        ns += __shfl_xor(ns, 1, 64);
        ns += __shfl_xor(ns, 2, 64);
        if (sk == 0) {
            const int kr = srow + 128 * h;
            const double nu = sqrt(ns);
            // the stored norm (float32, or its binary16 rounding): the reconstruction, and so
            // the residual, use it; the rotated coordinates use the unrounded norm
            const float nu_f = (float)nu;
            const uint16_t nu_h = f32_to_binary16(nu_f);
            const float nu_s = a.nh ? norm_f32(nu_h) : nu_f;
            s_inv[kr] = nu > 0.0 ? (float)(a.sqrt_d[g] / nu) : 0.0f;
            s_coef[kr] = (float)((double)nu_s / a.sqrt_d[g]);
            if (tile == 0 && kbase + kr < rows) {
                const size_t at = ((size_t)br[h].tile * 16 + (kr & 15)) * ng + g;
                if (a.nh)
                    static_cast<uint16_t *>(norms)[at] = nu_h;
                else
                    static_cast<float *>(norms)[at] = nu_f;
            }
        }
    }
    float th[7];
#pragma unroll
    for (int t = 0; t < 7; ++t) th[t] = t < (1 << nb) - 1 ? a.thr[g][t] : INFINITY;
    lds_barrier();

    // epilogue: lane (q, i) of block (rb, kb) holds coordinates 64 wr + 16 rb + 4q + r of
    // key 64 wk + 16 kb + i
    const int W = a.W, wpp = dg / 32;
    float rr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int kt = 64 * wk + 16 * kb + i;
        const int kl = kbase + kt;
        const bool row_live = kl < rows;
        const long T = t0 + (kl >> 4);
        const float inv = s_inv[kt], coef = s_coef[kt];
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
    for (int kb = 0; kb < 4; ++kb) {
        const float s = add_rows32(add_rows16(rr[kb]));
        const int kl = kbase + 64 * wk + 16 * kb + i;
        if (q == 0 && kl < rows) rho_part[(size_t)(jbase + 2 * tile + wr) * EG_CHUNK + kl] = s;
    }
}

// ---- stage 2: projection of the residual chunk, sign words, residual norms (DT as in stage 1)
template <int DT = 0>
__global__ __launch_bounds__(EG_THREADS) void enc_gemm_prj_kernel(const float *__restrict__ U,
                                                                  const uint16_t *__restrict__ sp3, EncArgs a,
                                                                  long t0, int rows, int J,
                                                                  const float *__restrict__ rho_part,
                                                                  uint32_t *__restrict__ bits,
                                                                  void *__restrict__ rnorms) {
    __shared__ __align__(16) u32x4 As[2][3][8][64];
    __shared__ __align__(16) u32x4 Bs[2][3][16][64];
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, i = lane & 15;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), wr = wv & 1, wk = wv >> 1;
    const int D = DT ? DT : a.d, M = DT ? DT : a.m;
    const int ntile = (M + EG_TILE - 1) / EG_TILE;
    int kblock, tile;
    eg_block(ntile, kblock, tile);
    const int kbase = kblock * EG_KT, r0 = tile * EG_TILE;

    // staging role: row srow of the A tile, rows srow and srow + 128 of the B tile
    const int srow = tid >> 2, sk = tid & 3;
    const bool a_live = r0 + srow < M;
    auto load_b = [&](int h, int k0, float (&v)[8]) {
        const int kr = kbase + srow + 128 * h;
        const float *urow = U + (size_t)kr * D;
        if (kr < rows) {
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

    auto stage = [&](int buf, const u32x4 (&av)[3], const float (&bv)[2][8]) {
#pragma unroll
        for (int p = 0; p < 3; ++p) As[buf][p][srow >> 4][eg_slot(srow, sk)] = av[p];
#pragma unroll
        for (int h = 0; h < 2; ++h) eg_store_b<3, 16>(bv[h], Bs[buf], srow + 128 * h, sk);
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[rb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nk = D / EG_KC;
    {
        u32x4 av[3];
        float bv[2][8];
        eg_load_a(sp3, M, D, r0 + srow, 0, sk, a_live, av);
        load_b(0, 0, bv[0]);
        load_b(1, 0, bv[1]);
        stage(0, av, bv);
    }
    lds_barrier();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        u32x4 av[3];
        float bv[2][8];
        const bool more = kc + 1 < nk;
        if (more) {
            eg_load_a(sp3, M, D, r0 + srow, (kc + 1) * EG_KC, sk, a_live, av);
            load_b(0, (kc + 1) * EG_KC, bv[0]);
            load_b(1, (kc + 1) * EG_KC, bv[1]);
        }
        eg_mma4<3>(As[buf], Bs[buf], wr, wk, lane, acc);
        if (more) stage(buf ^ 1, av, bv);
        lds_barrier();
    }

    // sign words: lane (q, i) of block (rb, kb) holds rows 64 wr + 16 rb + 4q + r of key
    // 64 wk + 16 kb + i
    const int W = a.W;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int kl = kbase + 64 * wk + 16 * kb + i;
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
    if (tile == 0 && tid < EG_KT) {
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
