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

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));  // a 32 x 32 MFMA accumulator

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

// Streamed batches (four key tiles per operand read). A batch's 2 NQ MFMA steps (derived
// quad, half) run in a fixed order that takes the derived words word-group by word-group
// (every Walsh subset of stored words 4k..4k+3 of a class, then the next four words, the
// sketch words last), so each stored quad is read by steps close together. Its loads are
// issued LDS_LA quads before its first step (those of the next batch's first quads during
// this batch's last ones): the key words in registers are then those of a few quads, not
// of the whole batch, and no batch waits for a round trip to memory at its start. The freed
// registers hold the next step's expanded key operand and operand fragments, formed while
// the current step's MFMAs run (one MFMA, then two of the next step's vector instructions).
constexpr int LDS_LA = 8;

// Streamed batches with two row tiles run on v_mfma_i32_32x32x32_i8 (LDS_WIDE), with
// LDS_WIDE_VALU vector instructions scheduled after each MFMA. Measured at d = 768, b = 4
// (1024 queries, 2M keys): 20.6-20.8 ms against 21.3-21.6 for the 16 x 16 x 64 form, the
// same lists; 4 or 9 instructions per MFMA, a lookahead of 5 or 12 quads, or separate
// accumulators per K half (four chains instead of two) measured no faster.
constexpr bool LDS_WIDE = true;
constexpr int LDS_WIDE_VALU = 6;

template <class L>
struct StreamOrder {
    struct Table {
        int v[64];
    };
    static_assert(L::NQ <= 64 && L::NSQ <= 64, "stream tables");
    // sort key of derived quad q: class, then word index inside its plane, then subset
    static constexpr int key(int q) {
        for (int g = 0; g < 4; ++g) {
            const DWord w = L::dword(4 * q + g);
            if (w.cls >= 0) return ((w.cls * 4096) + (w.k - g)) * 8 + w.sub;
        }
        return 1 << 30;  // padding only: last
    }
    static constexpr Table make_order() {
        Table keys{}, ord{};
        for (int q = 0; q < L::NQ; ++q) keys.v[q] = key(q);
        for (int q = 0; q < L::NQ; ++q) {
            int rank = 0;
            for (int p = 0; p < L::NQ; ++p)
                if (keys.v[p] < keys.v[q] || (keys.v[p] == keys.v[q] && p < q)) ++rank;
            ord.v[rank] = q;
        }
        return ord;
    }
    static constexpr Table order = make_order();
    static constexpr Table make_first() {
        Table f{};
        for (int sq = 0; sq < L::NSQ; ++sq) f.v[sq] = L::NQ;
        for (int i = L::NQ - 1; i >= 0; --i) {
            const int q = order.v[i];
            for (int c = 0; c < L::quad_nx(q); ++c) f.v[L::quad_sq(q, c)] = i;
        }
        return f;
    }
    static constexpr Table first = make_first();
    // the i-th derived quad of a batch
    static constexpr int at(int i) { return order.v[i]; }
    // position of the first quad that reads stored quad sq (NQ: none)
    static constexpr int first_use(int sq) { return first.v[sq]; }
};

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

// Offers the estimates of a 32-key pair to two queries of a row tile: lanes 0..31 hold
// query Q0's (lists lv[Q0]), lanes 32..63 query Q0 + 1's; every lane keeps its own query's
// k-th entry in (tv, ti). Otherwise as topk_offer4.
template <int Q0>
__device__ __forceinline__ void topk_offer_pair(float (&lv)[4], int (&li)[4], float &tv, int &ti, float est, int key,
                                                bool ok, int kh, int k, int lane) {
    uint64_t m = __ballot(ok && topk_better(est, key, tv, ti));
    if (!m) return;
    while (m) {
        const int src = __builtin_ctzll(m);
        m &= m - 1;
        const float v = __shfl(est, src, 64);
        const int id = __shfl(key, src, 64);
        if (src < 32)
            topk_insert(lv[Q0], li[Q0], v, id, lane);
        else
            topk_insert(lv[Q0 + 1], li[Q0 + 1], v, id, lane);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float t = __shfl(lv[Q0 + h], k - 1, 64);
        const int i = __shfl(li[Q0 + h], k - 1, 64);
        if (kh == h) {
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
    constexpr bool WIDE = !DB && TB == 4 && RQ == 2 && LDS_WIDE;
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

    // estimates of the batch at tile t from its accumulators: stored, or offered to the lists
    auto finish = [&](int t, const float (&nu)[TB][L::NG], const float (&rho)[TB], i32x4 (&acc)[TB][RQ][L::NCLS]) {
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
                    const double s = c < L::NG ? (double)nu[u][g] : (double)rho[u];
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
    };

    if constexpr (DB) {
    TileBatch<L, TB> A, B;
    if (t0 < t1) ts.load(A, t0);
    for (int t = t0; t < t1; t += TB) {
        if (t + TB < t1) ts.load(B, t + TB);
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
        finish(t, A.nu, A.rho, acc);
        A = B;
    }
    } else if constexpr (!WIDE) {
    // streamed batches: stored quad sq of tile u in kw[sq][u] (the next batch's first quads
    // in kn until the batch ends)
    using SO = StreamOrder<L>;
    // every stored quad is loaded in a batch's positions 0 .. NQ - 1 for this batch or the next
    static_assert(L::NQ >= LDS_LA, "the lookahead spans at most one batch");
    constexpr int NSTEP = 2 * L::NQ;
    const uint32_t *bbank = bits + (size_t)bank * n_tiles * L::W * 16;
    const typename L::NormT *nbank = norms + (size_t)bank * n_pad * L::NG;
    const typename L::NormT *rbank = rnorms + (size_t)bank * n_pad;
    // The chunk's bit words through one buffer resource (the host keeps a chunk below 2 GiB):
    // a load is then a scalar offset (tile, stored quad) plus this lane's 32-bit offset, with
    // no per-load address arithmetic on the vector ALU. Word 4 sq + gl of key j of a tile
    // sits 4 (16 (4 sq + gl) + j) bytes into it.
    const __amdgpu_buffer_rsrc_t chunk_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(bbank) + (size_t)c0 * (L::W * 16), 0, (c1 - c0) * (L::W * 64), BUF_DWORD3);
    const int lane_off = 4 * (16 * gl + j);
    auto load_sq = [&](uint32_t (&dst)[TB], int sq, int tile0) {
        const bool live = 4 * sq + gl < L::W;
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int tile = min(tile0 + u, t1 - 1);  // clamped: the last batch may be partial
            const int soff = (tile - c0) * (L::W * 64) + 256 * sq;
            const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(chunk_rs, live ? lane_off : 4 * j, soff, 0);
            dst[u] = live ? v : 0u;
        }
    };
    uint32_t kw[L::NSQ][TB];
    static_for<L::NSQ>([&](auto sc) {
        constexpr int sq = decltype(sc)::value;
        if constexpr (SO::first_use(sq) < LDS_LA)
            if (t0 < t1) load_sq(kw[sq], sq, t0);
    });
    for (int t = t0; t < t1; t += TB) {
        float nu[TB][L::NG], rho[TB];
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int tile = min(t + u, t1 - 1);
#pragma unroll
            for (int g = 0; g < L::NG; ++g) nu[u][g] = norm_f32(nbank[(size_t)tile * (16 * L::NG) + j * L::NG + g]);
            rho[u] = norm_f32(rbank[(size_t)tile * 16 + j]);
        }
        uint32_t kn[L::NSQ][TB];
        i32x4 acc[TB][RQ][L::NCLS];
#pragma unroll
        for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int rt = 0; rt < RQ; ++rt)
#pragma unroll
                for (int c = 0; c < L::NCLS; ++c) acc[u][rt][c] = i32x4{0, 0, 0, 0};
        // operands of step s = (position i, half h): expanded key words and fragments
        auto der_of = [&](auto ic, uint32_t (&der)[TB]) {
            constexpr int q = SO::at(decltype(ic)::value);
            constexpr int nx = L::quad_nx(q);
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                der[u] = kw[L::quad_sq(q, 0)][u];
                if constexpr (nx > 1) der[u] ^= kw[L::quad_sq(q, 1)][u];
                if constexpr (nx > 2) der[u] ^= kw[L::quad_sq(q, 2)][u];
            }
        };
        auto frags_of = [&](auto sc, i8x16 (&a)[L::NCLS][RQ]) {
            constexpr int s = decltype(sc)::value;
            constexpr int q = SO::at(s / 2), h = s % 2;
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (L::quad_has(q, c)) {
#pragma unroll
                    for (int rt = 0; rt < RQ; ++rt)
                        a[c][rt] = *reinterpret_cast<const i8x16 *>(&fa[rt][L::frag_index(q, h, c)][lane][0]);
                }
            });
        };
        uint32_t der[TB];
        i8x16 bk[TB], ak[L::NCLS][RQ];
        der_of(std::integral_constant<int, 0>{}, der);
#pragma unroll
        for (int u = 0; u < TB; ++u) bk[u] = expand_half<0>(der[u]);
        frags_of(std::integral_constant<int, 0>{}, ak);
        static_for<NSTEP>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int i = s / 2, h = s % 2;
            constexpr int q = SO::at(i);
            __builtin_amdgcn_sched_barrier(0);
            // loads of the stored quads first read LDS_LA quads ahead (this batch or the next)
            if constexpr (h == 0) {
                static_for<L::NSQ>([&](auto qc) {
                    constexpr int sq = decltype(qc)::value;
                    constexpr int fu = SO::first_use(sq);
                    if constexpr (fu < L::NQ && fu == i + LDS_LA) load_sq(kw[sq], sq, t);
                    if constexpr (fu < LDS_LA && fu == i + LDS_LA - L::NQ) load_sq(kn[sq], sq, t + TB);
                });
            }
            // the next step's operands, formed while this step's MFMAs run
            i8x16 bn[TB], an[L::NCLS][RQ];
            if constexpr (s + 1 < NSTEP) {
                if constexpr (h == 1) der_of(std::integral_constant<int, i + 1>{}, der);
#pragma unroll
                for (int u = 0; u < TB; ++u) bn[u] = expand_half<(s + 1) % 2>(der[u]);
                frags_of(std::integral_constant<int, s + 1>{}, an);
            }
            constexpr int nmf = [] {
                int m = 0;
                for (int c = 0; c < L::NCLS; ++c) m += L::quad_has(q, c) ? RQ * TB : 0;
                return m;
            }();
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (L::quad_has(q, c)) {
#pragma unroll
                    for (int rt = 0; rt < RQ; ++rt)
#pragma unroll
                        for (int u = 0; u < TB; ++u)
                            acc[u][rt][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ak[c][rt], bk[u], acc[u][rt][c], 0, 0, 0);
                }
            });
            // schedule: the fragment reads, then each MFMA followed by two vector instructions
            __builtin_amdgcn_sched_group_barrier(0x100, RQ, 0);
            static_for<nmf>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            });
            if constexpr (s + 1 < NSTEP) {
#pragma unroll
                for (int u = 0; u < TB; ++u) bk[u] = bn[u];
                static_for<L::NCLS>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
#pragma unroll
                    for (int rt = 0; rt < RQ; ++rt) ak[c][rt] = an[c][rt];
                });
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        finish(t, nu, rho, acc);
        static_for<L::NSQ>([&](auto sc) {
            constexpr int sq = decltype(sc)::value;
            if constexpr (SO::first_use(sq) < LDS_LA) {
#pragma unroll
                for (int u = 0; u < TB; ++u) kw[sq][u] = kn[sq][u];
            }
        });
    }
    } else {
    // 32 x 32 x 32 form of the streamed batches (four key tiles, two row tiles): the two row
    // tiles are the 32 rows of one v_mfma_i32_32x32x32_i8 and a pair of key tiles its 32
    // columns, so a step issues half as many MFMAs for the same multiply-adds, and each one
    // leaves the issue port free for more of the vector work (about six instructions per
    // MFMA instead of two). Lane (n, kh) = (lane & 31, lane >> 5) holds key j of tile
    // 2 p + hi of the batch (hi = n >> 4; pairs p = 0, 1) and, of each quad, stored words
    // 4 sq + 2 w + kh for w = 0, 1 (the two 32-deep halves of the quad's K step); the
    // operand fragments are the same LDS bytes read at other lane offsets (row tile hi,
    // row j, word 2 w + kh). Its accumulator registers 4 a .. 4 a + 3 hold the four limbs of
    // query 2 a + kh of the eight (row tile a / 2, query 2 (a % 2) + kh in it).
    using SO = StreamOrder<L>;
    static_assert(L::NQ >= LDS_LA, "the lookahead spans at most one batch");
    constexpr int NSTEP = 2 * L::NQ;
    const int kh = lane >> 5, hi = (lane >> 4) & 1;
    const uint32_t *bbank = bits + (size_t)bank * n_tiles * L::W * 16;
    const typename L::NormT *nbank = norms + (size_t)bank * n_pad * L::NG;
    const typename L::NormT *rbank = rnorms + (size_t)bank * n_pad;
    const __amdgpu_buffer_rsrc_t chunk_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t *>(bbank) + (size_t)c0 * (L::W * 16), 0, (c1 - c0) * (L::W * 64), BUF_DWORD3);
    // byte offset of word kh of this lane's key in pair p of the batch at tile tb (tiles past
    // the run clamped to its last: their keys are never offered or stored)
    auto pair_off = [&](int tb, int p) { return (min(tb + 2 * p + hi, t1 - 1) - c0) * (L::W * 64) + 4 * (16 * kh + j); };
    // stored quad sq: word 4 sq + 2 w + kh of pair p in dst[2 p + w]
    auto load_sq = [&](uint32_t (&dst)[4], auto sqc, const int (&vo)[2]) {
        constexpr int sq = decltype(sqc)::value;
        static_for<2>([&](auto wc) {
            constexpr int w = decltype(wc)::value;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                if constexpr (4 * sq + 2 * w + 1 < L::W) {
                    dst[2 * p + w] = __builtin_amdgcn_raw_buffer_load_b32(chunk_rs, vo[p] + 128 * w, 256 * sq, 0);
                } else if constexpr (4 * sq + 2 * w < L::W) {
                    // word 2 w + 1 is past the key's words: lanes kh = 1 read word 4 sq instead
                    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(chunk_rs, kh ? vo[p] - 64 : vo[p] + 128 * w,
                                                                            256 * sq, 0);
                    dst[2 * p + w] = kh ? 0u : v;
                } else {
                    dst[2 * p + w] = 0u;
                }
            }
        });
    };
    // the thresholds (k-th entries) of this lane's four queries
    float tw[4];
    int tiw[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        tw[a] = -INFINITY;
        tiw[a] = INT32_MAX;
    }
    // the per-query constants with the terms' scales folded in, as the other paths form them
    __shared__ double csf[4 * RQ][L::NCLS][2];
    for (int e = tid; e < 4 * RQ * L::NCLS * 2; e += LDS_WAVES * 64) {
        const int c = (e / 2) % L::NCLS;
        const double f = c < L::NG ? (c == 0 ? sc.inv_sqrt_d[0] : sc.inv_sqrt_d[1]) : sc.qjl;
        (&csf[0][0][0])[e] = (&cst[0][0][0])[e] * f;
    }
    __syncthreads();
    auto finish_w = [&](int t, const float (&nu)[2][L::NG], const float (&rho)[2], i32x16 (&acc)[2][L::NCLS]) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int tile = t + 2 * p + hi;
            const long key = (long)tile * 16 + j;
            const bool key_live = tile < t1 && key < n;
            static_for<4>([&](auto ac) {
                constexpr int a = decltype(ac)::value;
                const int qi = 2 * a + kh;  // query of the eight
                double est = 0.0;
                static_for<L::NCLS>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
                    constexpr int g = c < L::NG ? c : 0;
                    const double s = c < L::NG ? (double)nu[p][g] : (double)rho[p];
                    const i32x4 lm{acc[p][c][4 * a], acc[p][c][4 * a + 1], acc[p][c][4 * a + 2], acc[p][c][4 * a + 3]};
                    est = fma(s, fma(limbs_to_f64<L::class_positions(c)>(lm), csf[qi][c][0], csf[qi][c][1]), est);
                });
                const float e = (float)est;
                const int gq = 4 * rt0 + qi;
                if constexpr (TOPK) {
                    topk_offer_pair<2 * (a % 2)>(lv[a / 2], li[a / 2], tw[a], tiw[a], e, (int)key, key_live && gq < G,
                                                 kh, k, lane);
                } else {
                    if (key_live && gq < G) ob[(size_t)gq * n + key] = e;
                }
            });
        }
    };
    int vo[2], vn[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) vo[p] = pair_off(t0, p);
    uint32_t kw[L::NSQ][4];
    static_for<L::NSQ>([&](auto sc) {
        constexpr int sq = decltype(sc)::value;
        if constexpr (SO::first_use(sq) < LDS_LA)
            if (t0 < t1) load_sq(kw[sq], sc, vo);
    });
    for (int t = t0; t < t1; t += TB) {
#pragma unroll
        for (int p = 0; p < 2; ++p) vn[p] = pair_off(t + TB, p);
        float nu[2][L::NG], rho[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int tile = min(t + 2 * p + hi, t1 - 1);
#pragma unroll
            for (int g = 0; g < L::NG; ++g) nu[p][g] = norm_f32(nbank[(size_t)tile * (16 * L::NG) + j * L::NG + g]);
            rho[p] = norm_f32(rbank[(size_t)tile * 16 + j]);
        }
        uint32_t kn[L::NSQ][4];
        i32x16 acc[2][L::NCLS];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int c = 0; c < L::NCLS; ++c) acc[p][c] = i32x16{};
        auto der_of = [&](auto ic, uint32_t (&der)[4]) {
            constexpr int q = SO::at(decltype(ic)::value);
            constexpr int nx = L::quad_nx(q);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                der[x] = kw[L::quad_sq(q, 0)][x];
                if constexpr (nx > 1) der[x] ^= kw[L::quad_sq(q, 1)][x];
                if constexpr (nx > 2) der[x] ^= kw[L::quad_sq(q, 2)][x];
            }
        };
        auto frags_of = [&](auto sc, i8x16 (&a)[L::NCLS][2]) {
            constexpr int s = decltype(sc)::value;
            constexpr int q = SO::at(s / 2), h = s % 2;
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (L::quad_has(q, c)) {
#pragma unroll
                    for (int w = 0; w < 2; ++w)
                        a[c][w] = *reinterpret_cast<const i8x16 *>(&fa[hi][L::frag_index(q, h, c)][16 * (2 * w + kh) + j][0]);
                }
            });
        };
        uint32_t der[4];
        i8x16 bk[4], ak[L::NCLS][2];
        der_of(std::integral_constant<int, 0>{}, der);
#pragma unroll
        for (int x = 0; x < 4; ++x) bk[x] = expand_half<0>(der[x]);
        frags_of(std::integral_constant<int, 0>{}, ak);
        static_for<NSTEP>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int i = s / 2, h = s % 2;
            constexpr int q = SO::at(i);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (h == 0) {
                static_for<L::NSQ>([&](auto qc) {
                    constexpr int sq = decltype(qc)::value;
                    constexpr int fu = SO::first_use(sq);
                    if constexpr (fu < L::NQ && fu == i + LDS_LA) load_sq(kw[sq], qc, vo);
                    if constexpr (fu < LDS_LA && fu == i + LDS_LA - L::NQ) load_sq(kn[sq], qc, vn);
                });
            }
            i8x16 bn[4], an[L::NCLS][2];
            if constexpr (s + 1 < NSTEP) {
                if constexpr (h == 1) der_of(std::integral_constant<int, i + 1>{}, der);
#pragma unroll
                for (int x = 0; x < 4; ++x) bn[x] = expand_half<(s + 1) % 2>(der[x]);
                frags_of(std::integral_constant<int, s + 1>{}, an);
            }
            constexpr int nmf = [] {
                int m = 0;
                for (int c = 0; c < L::NCLS; ++c) m += L::quad_has(q, c) ? 4 : 0;
                return m;
            }();
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (L::quad_has(q, c)) {
#pragma unroll
                    for (int w = 0; w < 2; ++w)
#pragma unroll
                        for (int p = 0; p < 2; ++p)
                            acc[p][c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ak[c][w], bk[2 * p + w], acc[p][c], 0, 0, 0);
                }
            });
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            static_for<nmf>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, LDS_WIDE_VALU, 0);
            });
            if constexpr (s + 1 < NSTEP) {
#pragma unroll
                for (int x = 0; x < 4; ++x) bk[x] = bn[x];
                static_for<L::NCLS>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
#pragma unroll
                    for (int w = 0; w < 2; ++w) ak[c][w] = an[c][w];
                });
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        finish_w(t, nu, rho, acc);
        static_for<L::NSQ>([&](auto sc) {
            constexpr int sq = decltype(sc)::value;
            if constexpr (SO::first_use(sq) < LDS_LA) {
#pragma unroll
                for (int x = 0; x < 4; ++x) kw[sq][x] = kn[sq][x];
            }
        });
#pragma unroll
        for (int p = 0; p < 2; ++p) vo[p] = vn[p];
    }
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
