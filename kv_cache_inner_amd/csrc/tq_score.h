// Query preparation and the packed-key scorer for gfx950.
//
// The estimator (turboquant-pytorch write-up, two-stage algorithm section and usage
// example; tambur.pub article on why the 1-bit residual correction removes the
// inner-product bias) for a full-precision query q and a packed key:
//   est = sum_g (nu_g/sqrt(d_g)) <R_g q_g, c_g[idx_g]> + sqrt(pi/2)/m rho <S q, 2 s - 1>.
//
// Query preparation turns every query into integer MFMA operands once: the
// Walsh-expanded codebook weights 2*chat_S*(R_g q_g)_j and the sketch weights 2*(S q)_i are
// rounded to fixed point with a per-(query, term) exponent F (|w| 2^F < 2^30) and split
// into four signed 8-bit limbs. A 16-row MFMA operand then holds 4 queries x 4 limbs.
// Key bits enter the MFMA as bytes {0, 2^t} (t = bit position inside the byte, 2^7
// read as -128), so the weight at a position with shift t is pre-divided by 2^t; the
// int32 accumulation is exact and the limbs are recombined exactly in fp64.
#pragma once
#include <math.h>

#include "tq_device.h"
#include "tq_layout.h"

namespace tq {

struct PrepArgs {
    double walsh[2][4];  // 2 * chat_S per group and Walsh subset
    double cmax[2];      // c[L-1] per group (sum of the chat_S)
};

// smallest power-of-two split of a row of d columns into chunks of at most 48 columns
constexpr int prep_chunks(int d) {
    int c = 1;
    while (d / c > 48 || d % c) c *= 2;
    return c;
}

// Query operands of 4*RT queries (one bank), computed cooperatively by NT threads.
// Outputs (generic pointers: LDS or global):
//   frag_out  [RT][NF][64 lanes][16 bytes]: MFMA A operands, lane = 16*gl + 4*query + limb,
//             the 16 bytes being the K positions of lane group gl;
//   const_out [4*RT][NCLS][2] (fp64): {2^-F, additive constant} per query and term.
// R_g q_g and S q are formed in fp32 (relative error ~ sqrt(d) 2^-24, far inside the score
// tolerance). Each weight w is rounded to V = rint(w * 2^(F-t)) (|V| <= 2^30), t the bit's
// shift inside its byte; V splits into balanced signed base-256 digits via U = V + 0x80808080,
// whose plain base-256 digits minus 128 are the limbs. The additive constant is formed from
// the same fp32 weights, so the integer part and the constant stay consistent.
template <class L, int RT>
struct PrepScratch {
    static constexpr int NR = L::D + L::M;
    static constexpr int CPR = prep_chunks(L::D);  // column chunks per matrix row (power of two)
    static constexpr int RB = 64 / CPR;            // matrix rows per wave in the product
    float qv[L::D][4 * RT];                        // queries, column-major
    float qg[L::D][4 * RT];                        // columns in group order (qg[pos] = column chan[pos])
    float w[4 * RT][NR];                           // R_g q_g (group order) then S q
    float pmax[NR / RB][4 * RT];                   // per row-block max |w|
    double psum[NR / RB][4 * RT];                  // per row-block sum of w
    int F[4 * RT][L::NCLS];
};

template <class L, int RT, int NT>
__device__ __forceinline__ void prep_operands(int tid, const float *__restrict__ q, long bank, int G, int q0,
                                              const float *__restrict__ rot, const float *__restrict__ proj,
                                              const int *__restrict__ chan, const PrepArgs &pa,
                                              PrepScratch<L, RT> &ps, int8_t *frag_out, double *const_out) {
    using PS = PrepScratch<L, RT>;
    constexpr int NQ4 = 4 * RT;
    constexpr int NR = PS::NR, CPR = PS::CPR, RB = PS::RB;
    constexpr int CH = L::D / CPR;  // columns per chunk
    static_assert(CH % 4 == 0 && 64 % CPR == 0, "bad chunking");
    static_assert(L::D0 % RB == 0 && L::D % RB == 0, "row blocks must not straddle estimator terms");
    const int lane = tid & 63, wv = tid / 64;
    for (int e = tid; e < NQ4 * L::D; e += NT) {
        const int qq = e / L::D, c = e % L::D, gq = q0 + qq;
        const float *qrow = q + ((size_t)bank * G + gq) * L::D;
        ps.qv[c][qq] = gq < G ? qrow[c] : 0.0f;
        ps.qg[c][qq] = gq < G ? qrow[chan ? chan[c] : c] : 0.0f;
    }
    __syncthreads();
    // Items (query quad, row, part). Part p of a row takes the float4 columns p, p+CPR, ...
    // so that the CPR lanes of a row read contiguous 16*CPR-byte runs; all loads of an item
    // are issued before its arithmetic. Parts of a row sit in adjacent lanes, rows of a
    // wave form one row block; both are reduced with shuffles in a fixed order.
    for (int it = tid; it < NR * RT * CPR; it += NT) {
        const int part = it % CPR, item = it / CPR;
        const int r = item % NR, qb = 4 * (item / NR);
        const float *row;
        int K, off = 0;
        const bool rotated = r < L::D;
        if (rotated) {
            const int g = r < L::D0 ? 0 : 1;
            off = g ? L::D0 : 0;
            K = g ? L::D1 : L::D0;
            row = rot + (g ? (size_t)L::D0 * L::D0 : 0) + (size_t)(r - off) * K;
        } else {
            K = L::D;
            row = proj + (size_t)(r - L::D) * L::D;
        }
        const float(*src)[NQ4] = rotated ? ps.qg + off : ps.qv;  // operand columns of this row
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4 m[CH / 4];
#pragma unroll
            for (int i = 0; i < CH / 4; ++i) {
                const int k = 4 * (i * CPR + part);
                m[i] = k < K ? *reinterpret_cast<const f32x4 *>(row + k) : f32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < CH / 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = min(4 * (i * CPR + part) + e, K - 1);  // past K the loaded value is 0
                    const f32x4 qc = *reinterpret_cast<const f32x4 *>(&src[k][qb]);
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) acc[qq] = fmaf(m[i][e], qc[qq], acc[qq]);
                }
                // keep the LDS operand reads of later column groups from being hoisted here
                // (all of them live at once would exceed the register budget)
                asm volatile("" ::: "memory");
            }
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) acc[qq] += __shfl_xor(acc[qq], o, 64);
        // row-block partials: max |w| and the fp64 sum of the fp32 values
        float mx[4];
        double sm[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            if (part == 0) ps.w[qb + qq][r] = acc[qq];
            mx[qq] = fabsf(acc[qq]);
            sm[qq] = part == 0 ? (double)acc[qq] : 0.0;
        }
#pragma unroll
        for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                mx[qq] = fmaxf(mx[qq], __shfl_xor(mx[qq], o, 64));
                sm[qq] += __shfl_xor(sm[qq], o, 64);
            }
        if (lane == 0)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                ps.pmax[r / RB][qb + qq] = mx[qq];
                ps.psum[r / RB][qb + qq] = sm[qq];
            }
    }
    __syncthreads();
    // per (query, term): exponent F from the max |weight|, additive constant from the sum
    for (int it = tid; it < NQ4 * L::NCLS; it += NT) {
        const int qq = it / L::NCLS, c = it % L::NCLS, gq = q0 + qq;
        const int r0 = c < L::NG ? (c ? L::D0 : 0) : L::D;
        const int r1 = c < L::NG ? (c ? L::D : L::D0) : NR;
        double mx = 0.0, sm = 0.0;
        for (int bk = r0 / RB; bk < r1 / RB; ++bk) {
            mx = fmax(mx, (double)ps.pmax[bk][qq]);
            sm += ps.psum[bk][qq];
        }
        double wmax;
        if (c < L::NG) {
            double cm = 0.0;
            const int nsub = walsh_planes(c ? L::B1 : L::B0);
            for (int s2 = 0; s2 < nsub; ++s2) cm = fmax(cm, fabs(pa.walsh[c][s2]));
            wmax = mx * cm;
        } else {
            wmax = 2.0 * mx;
        }
        int e = 0;
        if (wmax > 0.0) frexp(wmax, &e);  // wmax < 2^e
        const int F = wmax > 0.0 ? 30 - e : 0;
        ps.F[qq][c] = F;
        double *o = const_out + ((size_t)qq * L::NCLS + c) * 2;
        o[0] = ldexp(1.0, -F);
        o[1] = gq < G ? (c < L::NG ? -pa.cmax[c] * sm : -sm) : 0.0;
    }
    __syncthreads();
    // fragments: RT waves per fragment (wave-uniform fragment id); item (gl, query, dword v)
    // -> 4 K positions x 4 limbs (one dword in each of four lanes)
    for (int fw = wv; fw < L::NF * RT; fw += NT / 64) {
        const int fr = fw / RT, it = (fw % RT) * 64 + lane;
        const int v = it & 3, qq = (it >> 2) % NQ4, gl = (it >> 2) / NQ4;
        static_for<L::NF>([&](auto fcst) {
            constexpr int f = decltype(fcst)::value;
            if (fr != f) return;
            constexpr int fq = L::frag_q(f), fh = L::frag_h(f), fc = L::frag_c(f);
            // per lane group: the derived word's term, word index and Walsh subset (scalars
            // selected one by one: a runtime pick of a whole struct would go through memory)
            constexpr DWord d0 = L::dword(4 * fq + 0), d1 = L::dword(4 * fq + 1);
            constexpr DWord d2 = L::dword(4 * fq + 2), d3 = L::dword(4 * fq + 3);
            const int cls = gl == 0 ? d0.cls : gl == 1 ? d1.cls : gl == 2 ? d2.cls : d3.cls;
            const int wk = gl == 0 ? d0.k : gl == 1 ? d1.k : gl == 2 ? d2.k : d3.k;
            const int sub = gl == 0 ? d0.sub : gl == 1 ? d1.sub : gl == 2 ? d2.sub : d3.sub;
            const bool live = (q0 + qq < G) && cls == fc;
            const int t = 4 * fh + v;
            const double scale = ldexp(1.0, ps.F[qq][fc] - t);  // 2^(F - t)
            const float *src = fc < L::NG ? &ps.w[qq][(fc ? L::D0 : 0) + 32 * wk] : &ps.w[qq][L::D + 32 * wk];
            const double mul = fc < L::NG ? pa.walsh[fc][sub] : 2.0;
            uint32_t U[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double wt = live ? mul * (double)src[8 * e + t] : 0.0;
                int V = __double2int_rn(wt * scale);
                if (t == 7) V = -V;  // the byte 0x80 reads as -128
                U[e] = (uint32_t)V + 0x80808080u;
            }
            const int rt = qq / 4;
            int8_t *base = frag_out + (((size_t)rt * L::NF + f) * 64 + 16 * gl + 4 * (qq % 4)) * 16 + 4 * v;
#pragma unroll
            for (int limb = 0; limb < 4; ++limb) {
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) packed |= (((U[e] >> (8 * limb)) & 0xFFu) ^ 0x80u) << (8 * e);
                *reinterpret_cast<uint32_t *>(base + limb * 16) = packed;
            }
        });
    }
}

// Standalone query preparation: one 1024-thread work-group per (bank, row tile of 4 queries).
//   frags [bank][Gpad/4][NF][64][16 B], consts [bank][Gpad][NCLS][2]
template <class L>
__global__ __launch_bounds__(1024) void qprep_kernel(const float *__restrict__ q, const float *__restrict__ rot,
                                                    const float *__restrict__ proj, const int *__restrict__ chan,
                                                    PrepArgs pa, int G, int Gpad, int8_t *__restrict__ frags,
                                                    double *__restrict__ consts) {
    __shared__ PrepScratch<L, 1> ps;
    const int nrt = Gpad / 4;
    const long bank = blockIdx.x / nrt;
    const int rt = blockIdx.x % nrt;
    prep_operands<L, 1, 1024>(threadIdx.x, q, bank, G, 4 * rt, rot, proj, chan, pa, ps,
                             frags + ((size_t)bank * nrt + rt) * L::NF * 1024,
                             consts + ((size_t)bank * Gpad + 4 * rt) * L::NCLS * 2);
}

// Exact recombination of the four int32 limb sums of a term with P bit positions.
// |limb sum| <= P/8 * 128 * (1 + 2 + ... + 128) = 4080 P for limbs 0..2 (|limb| <= 128, one
// eighth of the positions at each shift t) and 2072 P for limb 3 (|limb| <= 65), so for
// P < 2048 the pairs (a3 << 8) + a2 and (a1 << 8) + a0 fit in int32 and two conversions
// suffice; larger terms take four.
template <int P>
__device__ __forceinline__ double limbs_to_f64(i32x4 a) {
    if constexpr (P < 2048) {
        const int hi = (a[3] << 8) + a[2], lo = (a[1] << 8) + a[0];
        return fma((double)hi, 65536.0, (double)lo);
    } else {
        return fma((double)a[3], 16777216.0, fma((double)a[2], 65536.0, fma((double)a[1], 256.0, (double)a[0])));
    }
}

// Expands derived word `w` into the B operand of half h (16 bytes: byte e of dword v is
// bit 8e+4h+v of w, scaled by 2^(4h+v)).
template <int H>
__device__ __forceinline__ i8x16 expand_half(uint32_t w) {
    u32x4 r;
    r[0] = w & (0x01010101u << (4 * H + 0));
    r[1] = w & (0x01010101u << (4 * H + 1));
    r[2] = w & (0x01010101u << (4 * H + 2));
    r[3] = w & (0x01010101u << (4 * H + 3));
    return __builtin_bit_cast(i8x16, r);
}

// Scores one 16-key tile against the RT row tiles (4 queries each) held in `wf`.
// Returns the fp64 estimates in est[rt] for query 4*rt + lane/16, key lane%16.
template <class L, int RT>
__device__ __forceinline__ void score_tile(const uint32_t (&sw)[L::NSQ], const i8x16 (&wf)[RT][L::NF],
                                           i32x4 (&acc)[RT][L::NCLS]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < L::NCLS; ++c) acc[rt][c] = i32x4{0, 0, 0, 0};
    static_for<L::NQ>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        constexpr int nx = L::quad_nx(q);
        uint32_t der = sw[L::quad_sq(q, 0)];
        if constexpr (nx > 1) der ^= sw[L::quad_sq(q, 1)];
        if constexpr (nx > 2) der ^= sw[L::quad_sq(q, 2)];
        static_for<2>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const i8x16 b = expand_half<h>(der);
            static_for<L::NCLS>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if constexpr (L::quad_has(q, c)) {
                    constexpr int f = L::frag_index(q, h, c);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[rt][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[rt][f], b, acc[rt][c], 0, 0, 0);
                }
            });
        });
    });
}

// Decode-shaped scorer. A wave holds the operands of RT row tiles (G <= 4*RT queries of
// one bank) in VGPRs and streams a contiguous run [t0, t1) of 16-key tiles of that bank,
// TB tiles per batch, issuing the next batch's loads before computing the current one.
template <class L, int TB>
struct TileBatch {
    uint32_t sw[TB][L::NSQ];
    float nu[TB][L::NG];
    float rho[TB];
};

template <class L, int RT, int TB>
struct TileStream {
    const uint32_t *__restrict__ bb;  // this bank's tiles (wave-uniform)
    const float *__restrict__ nb;     // its norms
    const float *__restrict__ rb;     // its residual norms
    float *__restrict__ ob;           // its score rows
    long n;
    int G, t0, t1;  // wave-uniform
    // per-lane constants: word offsets inside a tile, score-row offsets
    int woff[L::NSQ];
    bool wlive[L::NSQ];
    long soff[RT];
    bool slive[RT];

    __device__ __forceinline__ void init_lane() {
        const int lane = threadIdx.x & 63, j = lane & 15, gl = lane >> 4;
#pragma unroll
        for (int s = 0; s < L::NSQ; ++s) {
            wlive[s] = 4 * s + gl < L::W;
            woff[s] = wlive[s] ? (4 * s + gl) * 16 + j : j;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            slive[rt] = 4 * rt + gl < G;
            soff[rt] = (long)(4 * rt + gl) * n + j;
        }
    }

    __device__ __forceinline__ void load(TileBatch<L, TB> &b, int tile0) const {
        const int j = threadIdx.x & 15;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int tile = min(tile0 + t, t1 - 1);  // clamped: the last batch may be partial
            const uint32_t *tb = bb + (size_t)tile * (L::W * 16);
#pragma unroll
            for (int s = 0; s < L::NSQ; ++s) {
                const uint32_t v = tb[woff[s]];
                b.sw[t][s] = wlive[s] ? v : 0u;
            }
            const float *tn = nb + (size_t)tile * (16 * L::NG);
#pragma unroll
            for (int g = 0; g < L::NG; ++g) b.nu[t][g] = tn[j * L::NG + g];
            b.rho[t] = rb[(size_t)tile * 16 + j];
        }
    }

    __device__ __forceinline__ void compute(const TileBatch<L, TB> &b, int tile0, const i8x16 (&wf)[RT][L::NF],
                                            const double (&cs)[RT][L::NCLS], const double (&ck)[RT][L::NCLS],
                                            const ScoreScale &sc) const {
        const int j = threadIdx.x & 15;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int tile = tile0 + t;
            if (tile >= t1) break;
            i32x4 acc[RT][L::NCLS];
            score_tile<L, RT>(b.sw[t], wf, acc);
            const bool key_live = (long)tile * 16 + j < n;
            float *tout = ob + (size_t)tile * 16;
            double scale[L::NCLS];
#pragma unroll
            for (int c = 0; c < L::NCLS; ++c)
                scale[c] = c < L::NG ? (double)b.nu[t][c] * sc.inv_sqrt_d[c] : (double)b.rho[t] * sc.qjl;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                double est = 0.0;
                static_for<L::NCLS>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
                    const double dot = fma(limbs_to_f64<L::class_positions(c)>(acc[rt][c]), cs[rt][c], ck[rt][c]);
                    est = fma(scale[c], dot, est);
                });
                if (slive[rt] && key_live) tout[soff[rt]] = (float)est;
            }
        }
    }

    // Issues the loads of the first two batches (tiles t0.. and t0+TB..).
    __device__ __forceinline__ void prefetch(TileBatch<L, TB> &A, TileBatch<L, TB> &B) const {
        if (t0 >= t1) return;
        load(A, t0);
        if (t0 + TB < t1) load(B, t0 + TB);
    }

    // Streams [t0, t1) given the two prefetched batches: while one batch is computed the
    // other one's loads are in flight.
    __device__ __forceinline__ void run(TileBatch<L, TB> &A, TileBatch<L, TB> &B, const i8x16 (&wf)[RT][L::NF],
                                        const double (&cs)[RT][L::NCLS], const double (&ck)[RT][L::NCLS],
                                        const ScoreScale &sc) const {
        int tile = t0;
        while (tile < t1) {
            compute(A, tile, wf, cs, ck, sc);
            tile += TB;
            if (tile >= t1) break;
            if (tile + TB < t1) load(A, tile + TB);
            compute(B, tile, wf, cs, ck, sc);
            tile += TB;
            if (tile + TB < t1) load(B, tile + TB);
        }
    }
};

// Scorer on prepared operands (tq_score_prepared): operands read from the workspace.
template <class L, int RT, int TB>
__global__ __launch_bounds__(256) void score_kernel(const uint32_t *__restrict__ bits, const float *__restrict__ norms,
                                                    const float *__restrict__ rnorms, const int8_t *__restrict__ frags,
                                                    const double *__restrict__ consts, float *__restrict__ scores,
                                                    int banks, long n, int n_tiles, int G, int Gpad, int tiles_per_wave,
                                                    int waves_per_bank, ScoreScale sc) {
    const int lane = threadIdx.x & 63;
    // wave-uniform indices (readfirstlane lets the compiler keep tile addressing scalar)
    const long wid = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long bank = wid / waves_per_bank;
    const int chunk = (int)(wid % waves_per_bank);
    if (bank >= banks) return;
    const int t0 = chunk * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, n_tiles);
    if (t0 >= t1) return;
    const int gl = lane >> 4;
    const long n_pad = (long)n_tiles * 16;

    i8x16 wf[RT][L::NF];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int f = 0; f < L::NF; ++f)
            wf[rt][f] = *reinterpret_cast<const i8x16 *>(frags + (((size_t)(bank * (Gpad / 4) + rt) * L::NF + f) * 64 + lane) * 16);
    double cs[RT][L::NCLS], ck[RT][L::NCLS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < L::NCLS; ++c) {
            const double *o = consts + (((size_t)bank * Gpad + 4 * rt + gl) * L::NCLS + c) * 2;
            cs[rt][c] = o[0];
            ck[rt][c] = o[1];
        }
    TileStream<L, RT, TB> ts{bits + (size_t)bank * n_tiles * L::W * 16, norms + (size_t)bank * n_pad * L::NG,
                             rnorms + (size_t)bank * n_pad, scores + (size_t)bank * G * n, n, G, t0, t1};
    ts.init_lane();
    TileBatch<L, TB> A, B;
    ts.prefetch(A, B);
    ts.run(A, B, wf, cs, ck, sc);
}

// Fused scorer (tq_score): each 16-wave work-group first builds its bank's query operands
// in LDS (query preparation as a prologue, so one launch per call), then its waves stream
// their share of the bank's key tiles.
template <int RT>
constexpr int fused_waves() {
    return RT == 1 ? 16 : 8;
}

template <class L, int RT>
struct FusedLds {
    PrepScratch<L, RT> ps;
    alignas(16) int8_t frags[RT][L::NF][64][16];
    double consts[4 * RT][L::NCLS][2];
};

template <class L, int RT, int TB>
__global__ __launch_bounds__(fused_waves<RT>() * 64) void score_fused_kernel(
    const uint32_t *__restrict__ bits, const float *__restrict__ norms, const float *__restrict__ rnorms,
    const float *__restrict__ q, const float *__restrict__ rot, const float *__restrict__ proj,
    const int *__restrict__ chan, PrepArgs pa, float *__restrict__ scores, int banks, long n, int n_tiles, int G,
    int wgs_per_bank, int tiles_per_wg, ScoreScale sc) {
    __shared__ FusedLds<L, RT> lds;
    const long bank = blockIdx.x / wgs_per_bank;
    const int part = blockIdx.x % wgs_per_bank;
    const int tid = threadIdx.x, lane = tid & 63, gl = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    constexpr int WAVES = fused_waves<RT>();
    // this work-group's tiles, split into contiguous per-wave runs
    const int w0 = part * tiles_per_wg, w1 = min(w0 + tiles_per_wg, n_tiles);
    const int per = (w1 - w0 + WAVES - 1) / WAVES;
    const int t0 = min(w0 + wv * per, w1), t1 = min(t0 + per, w1);
    const long n_pad = (long)n_tiles * 16;
    TileStream<L, RT, TB> ts{bits + (size_t)bank * n_tiles * L::W * 16, norms + (size_t)bank * n_pad * L::NG,
                             rnorms + (size_t)bank * n_pad, scores + (size_t)bank * G * n, n, G, t0, t1};
    ts.init_lane();
    // the first two batches are requested before the prologue, which then overlaps their latency
    TileBatch<L, TB> A, B;
    ts.prefetch(A, B);
    prep_operands<L, RT, WAVES * 64>(tid, q, bank, G, 0, rot, proj, chan, pa, lds.ps, &lds.frags[0][0][0][0],
                                     &lds.consts[0][0][0]);
    __syncthreads();
    if (t0 >= t1) return;
    i8x16 wf[RT][L::NF];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int f = 0; f < L::NF; ++f) wf[rt][f] = *reinterpret_cast<const i8x16 *>(&lds.frags[rt][f][lane][0]);
    double cs[RT][L::NCLS], ck[RT][L::NCLS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < L::NCLS; ++c) {
            cs[rt][c] = lds.consts[4 * rt + gl][c][0];
            ck[rt][c] = lds.consts[4 * rt + gl][c][1];
        }
    ts.run(A, B, wf, cs, ck, sc);
}

}  // namespace tq
