// Scorer with the query operands in LDS, and the fused per-query top-k.
//
// Vector search (tambur.pub article on TurboQuant, vector-search paragraph: the packed
// database is searched directly by estimated inner products; turboquant-pytorch write-up,
// usage example: inner_product(query, compressed)) needs many queries per bank and large
// key dimensions, whose MFMA operands do not fit in registers. Here a work-group stages
// the prepared operands (tq_prepare_queries) of RQ row tiles of one bank in LDS, and each
// of its waves streams a contiguous run of that bank's 16-key tiles, reading every operand
// fragment from LDS as it is used. The estimates are then either stored (scores) or kept
// as a running per-query top-k that never leaves the chip until the end.
//
// Top-k: the k best (value, index) pairs of a query live across the lanes of a wave, entry
// i in lane i, best first (larger value; equal values by lower index). A tile's estimates
// that beat the k-th entry are inserted one at a time by a lane-parallel shift. Each wave
// writes its k entries per query as a partial list; a merge kernel reduces the partial
// lists of a query to the final top-k.
#pragma once
#include "tq_score.h"

namespace tq {

// Each operand fragment read from LDS (1 KiB per wave) feeds the MFMAs of lds_tb() key tiles,
// and each expanded key operand the MFMAs of lds_rows() row tiles. Per MFMA the CU's LDS
// (128 B/clk) and vector ALU (4 ops per 16-cycle MFMA per SIMD) are then loaded with 1 KiB /
// TB and 4 / RQ. A work-group has 8 waves (two per SIMD, 256 VGPRs each): with two tiles per
// read the key words are double-buffered in registers; with four they are loaded once per
// batch and the SIMD's other wave computes while they arrive.
constexpr int LDS_WAVES = 8;

template <class L>
constexpr int lds_tb() {
    return L::NF * 1024 > 50 * 1024 ? 4 : 2;
}
// double-buffered key loads (two batches in registers) for two tiles per read
template <class L>
constexpr bool lds_db() {
    return lds_tb<L>() <= 2;
}

// row tiles of operands a work-group holds in LDS (fragments and constants in ~150 KiB); at
// most two beside four key tiles per read (their accumulators share the register budget)
template <class L>
constexpr int lds_rows() {
    constexpr int per = L::NF * 1024 + 4 * L::NCLS * 16;
    constexpr int r = (150 * 1024) / per;
    constexpr int cap = lds_tb<L>() > 2 ? 2 : 4;
    return r > cap ? cap : (r < 1 ? 1 : r);
}

template <class L>
constexpr bool lds_fits() {
    return L::NF * 1024 + 4 * L::NCLS * 16 <= 150 * 1024;
}

// Entry i of a per-query list sits in lane i. `better` orders candidates: larger value
// first, equal values by lower index.
__device__ __forceinline__ bool topk_better(float v, int i, float lv, int li) { return v > lv || (v == lv && i < li); }

// Inserts (v, id) into the wave-distributed sorted list (lv, li) (entries past k-1 are
// dropped off the end by the shift; lanes >= k hold entries that are never read back).
__device__ __forceinline__ void topk_insert(float &lv, int &li, float v, int id, int lane) {
    const bool b = topk_better(v, id, lv, li);
    const float pv = __shfl_up(lv, 1, 64);
    const int pi = __shfl_up(li, 1, 64);
    const bool pb = __shfl_up(b ? 1 : 0, 1, 64) != 0 && lane > 0;
    if (b) {
        lv = pb ? pv : v;
        li = pb ? pi : id;
    }
}

// Offers a tile's estimates to the four lists of a row tile: lane group g holds the 16
// estimates (est, key index key, valid flag ok) of query g, whose list is (lv[g], li[g]) and
// whose current k-th entry every lane of group g keeps in (tv, ti). One compare and one ballot
// find the candidates of all four queries; those (rare once the lists fill) are inserted in
// lane order, and the thresholds are then refreshed. A stale threshold only admits more
// candidates, and inserting one that no longer qualifies leaves the list unchanged.
__device__ __forceinline__ void topk_offer4(float (&lv)[4], int (&li)[4], float &tv, int &ti, float est, int key,
                                            bool ok, int gl, int k, int lane) {
    uint64_t m = __ballot(ok && topk_better(est, key, tv, ti));
    if (!m) return;
    while (m) {
        const int src = __builtin_ctzll(m);
        m &= m - 1;
        const float v = __shfl(est, src, 64);
        const int id = __shfl(key, src, 64);
        const int g = src >> 4;  // wave-uniform
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q == g) topk_insert(lv[q], li[q], v, id, lane);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float t = __shfl(lv[q], k - 1, 64);
        const int i = __shfl(li[q], k - 1, 64);
        if (gl == q) {
            tv = t;
            ti = i;
        }
    }
}

template <class L, int RQ, bool TOPK>
__global__ __launch_bounds__(LDS_WAVES * 64) void score_lds_kernel(
    const uint32_t *__restrict__ bits, const typename L::NormT *__restrict__ norms,
    const typename L::NormT *__restrict__ rnorms, const int8_t *__restrict__ frags, const double *__restrict__ consts, long n, int n_tiles, int G, int Gpad,
    int qblocks, int kchunks, int chunk_tiles, ScoreScale sc, float *__restrict__ scores, int k,
    float *__restrict__ part_v, int *__restrict__ part_i) {
    __shared__ __attribute__((aligned(16))) int8_t fa[RQ][L::NF][64][16];
    __shared__ double cst[4 * RQ][L::NCLS][2];
    const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, gl = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // block -> (bank, key chunk, query block), query block fastest: the work-groups that
    // read the same key chunk run side by side
    int blk = blockIdx.x;
    const int qb = blk % qblocks;
    blk /= qblocks;
    const int kc = blk % kchunks;
    const long bank = blk / kchunks;
    const int NRT = Gpad / 4, rt0 = qb * RQ;

    // stage this block's operands (row tiles past the bank's last are zero)
    const int8_t *fsrc = frags + ((size_t)bank * NRT + rt0) * L::NF * 1024;
    for (int e = tid; e < RQ * L::NF * 64; e += LDS_WAVES * 64) {
        const int rt = e / (L::NF * 64);
        const u32x4 v = rt0 + rt < NRT ? *reinterpret_cast<const u32x4 *>(fsrc + (size_t)e * 16) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4 *>(&fa[0][0][0][0] + (size_t)e * 16) = v;
    }
    for (int e = tid; e < 4 * RQ * L::NCLS * 2; e += LDS_WAVES * 64) {
        const int qq = e / (L::NCLS * 2), r = e % (L::NCLS * 2);
        const int gq = 4 * rt0 + qq;
        (&cst[0][0][0])[e] = gq < Gpad ? consts[((size_t)bank * Gpad + gq) * L::NCLS * 2 + r] : 0.0;
    }
    __syncthreads();
    // per (row tile, term): constants of this lane's query with the term's scale folded in
    double cs[RQ][L::NCLS], ck[RQ][L::NCLS];
#pragma unroll
    for (int rt = 0; rt < RQ; ++rt)
        static_for<L::NCLS>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int g = c < L::NG ? c : 0;
            const double f = c < L::NG ? sc.inv_sqrt_d[g] : sc.qjl;
            cs[rt][c] = cst[4 * rt + gl][c][0] * f;
            ck[rt][c] = cst[4 * rt + gl][c][1] * f;
        });

    // this wave's contiguous run of the chunk's tiles
    const int c0 = kc * chunk_tiles, c1 = min(c0 + chunk_tiles, n_tiles);
    const int per = (c1 - c0 + LDS_WAVES - 1) / LDS_WAVES;
    const int t0 = min(c0 + wv * per, c1), t1 = min(t0 + per, c1);
    const long n_pad = (long)n_tiles * 16;
    constexpr int TB = lds_tb<L>();
    constexpr bool DB = lds_db<L>();
    TileStream<L, 1, TB> ts{bits + (size_t)bank * n_tiles * L::W * 16, norms + (size_t)bank * n_pad * L::NG,
                           rnorms + (size_t)bank * n_pad, nullptr, n, G, t0, t1};
    ts.init_lane();
    float *ob = TOPK ? nullptr : scores + (size_t)bank * G * n;

    // per-query top-k lists (4 queries per row tile), entry i in lane i, and the k-th entry of
    // the lane's own query in each row tile
    float lv[RQ][4];
    int li[RQ][4];
    float tv[RQ];
    int ti[RQ];
#pragma unroll
    for (int rt = 0; rt < RQ; ++rt) {
        tv[rt] = -INFINITY;
        ti[rt] = INT32_MAX;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            lv[rt][g] = -INFINITY;
            li[rt][g] = INT32_MAX;
        }
    }

    TileBatch<L, TB> A, B;
    if (DB && t0 < t1) ts.load(A, t0);
    for (int t = t0; t < t1; t += TB) {
        if constexpr (DB) {
            if (t + TB < t1) ts.load(B, t + TB);
        } else {
            ts.load(A, t);
        }
        i32x4 acc[TB][RQ][L::NCLS];
#pragma unroll
        for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int rt = 0; rt < RQ; ++rt)
#pragma unroll
                for (int c = 0; c < L::NCLS; ++c) acc[u][rt][c] = i32x4{0, 0, 0, 0};
        static_for<L::NQ>([&](auto qc) {
            constexpr int qd = decltype(qc)::value;
            constexpr int nx = L::quad_nx(qd);
            uint32_t der[TB];
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                der[u] = A.sw[u][L::quad_sq(qd, 0)];
                if constexpr (nx > 1) der[u] ^= A.sw[u][L::quad_sq(qd, 1)];
                if constexpr (nx > 2) der[u] ^= A.sw[u][L::quad_sq(qd, 2)];
            }
            static_for<2>([&](auto hc) {
                constexpr int h = decltype(hc)::value;
                i8x16 b[TB];
#pragma unroll
                for (int u = 0; u < TB; ++u) b[u] = expand_half<h>(der[u]);
                static_for<L::NCLS>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
                    if constexpr (L::quad_has(qd, c)) {
                        constexpr int f = L::frag_index(qd, h, c);
#pragma unroll
                        for (int rt = 0; rt < RQ; ++rt) {
                            const i8x16 a = *reinterpret_cast<const i8x16 *>(&fa[rt][f][lane][0]);
#pragma unroll
                            for (int u = 0; u < TB; ++u)
                                acc[u][rt][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[u], acc[u][rt][c], 0, 0, 0);
                        }
                    }
                });
            });
            // the fragment reads of later quads stay below this point (all of them live at
            // once would exceed the register budget)
            asm volatile("" ::: "memory");
        });
#pragma unroll
        for (int u = 0; u < TB; ++u) {
        if (t + u >= t1) break;
        const long key = (long)(t + u) * 16 + j;
        const bool key_live = key < n;
#pragma unroll
        for (int rt = 0; rt < RQ; ++rt) {
            double est = 0.0;
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                constexpr int g = c < L::NG ? c : 0;
                const double s = c < L::NG ? (double)A.nu[u][g] : (double)A.rho[u];
                est = fma(s, fma(limbs_to_f64<L::class_positions(c)>(acc[u][rt][c]), cs[rt][c], ck[rt][c]), est);
            });
            const float e = (float)est;
            const int gq = 4 * (rt0 + rt) + gl;
            if constexpr (TOPK) {
                // queries past G never enter a list (their lists are not written back)
                topk_offer4(lv[rt], li[rt], tv[rt], ti[rt], e, (int)key, key_live && gq < G, gl, k, lane);
            } else {
                if (key_live && gq < G) ob[(size_t)gq * n + key] = e;
            }
        }
        }
        if constexpr (DB) A = B;
    }
    if constexpr (TOPK) {
        // partial lists: [bank][query][chunk * LDS_WAVES + wave][k]
        const int slots = kchunks * LDS_WAVES, slot = kc * LDS_WAVES + wv;
#pragma unroll
        for (int rt = 0; rt < RQ; ++rt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int gq = 4 * (rt0 + rt) + g;
                if (gq < G && lane < k) {
                    const size_t o = (((size_t)bank * G + gq) * slots + slot) * k + lane;
                    part_v[o] = lv[rt][g];
                    part_i[o] = li[rt][g];
                }
            }
    }
}

// Reduces the partial lists of each (bank, query) to its top-k: one wave per query.
__global__ __launch_bounds__(256) void topk_merge_kernel(const float *__restrict__ part_v,
                                                         const int *__restrict__ part_i, long queries, int slots, int k,
                                                         float *__restrict__ vals, int *__restrict__ idx) {
    const int lane = threadIdx.x & 63;
    const long qy = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (qy >= queries) return;
    float lv = -INFINITY;
    int li = INT32_MAX;
    const float *pv = part_v + (size_t)qy * slots * k;
    const int *pi = part_i + (size_t)qy * slots * k;
    const long total = (long)slots * k;
    for (long base = 0; base < total; base += 64) {
        const long e = base + lane;
        const bool ok = e < total;
        const float v = ok ? pv[e] : -INFINITY;
        const int id = ok ? pi[e] : INT32_MAX;
        const float tv = __shfl(lv, k - 1, 64);
        const int ti = __shfl(li, k - 1, 64);
        uint64_t m = __ballot(ok && id != INT32_MAX && topk_better(v, id, tv, ti));
        while (m) {
            const int src = __builtin_ctzll(m);
            m &= m - 1;
            topk_insert(lv, li, __shfl(v, src, 64), __shfl(id, src, 64), lane);
        }
    }
    if (lane < k) {
        vals[(size_t)qy * k + lane] = lv;
        idx[(size_t)qy * k + lane] = li;
    }
}

}  // namespace tq
