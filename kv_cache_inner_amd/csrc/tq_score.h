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

#include <type_traits>

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
struct PrepDims {
    static constexpr int NR = L::D + L::M;
    static constexpr int CPR = prep_chunks(L::D);  // column chunks per matrix row (power of two)
    static constexpr int RB = 64 / CPR;            // matrix rows per wave in the product
};

// LDS scratch of the query preparation, as one block.
template <class L, int RT>
struct PrepScratch {
    using PD = PrepDims<L, RT>;
    float qsrc[2][L::D][4 * RT];         // [0]: queries column-major; [1]: columns in group order
    float w[4 * RT][PD::NR];             // R_g q_g (group order) then S q
    int F[4 * RT][L::NCLS];
};

// The scratch arrays by reference: members of one PrepScratch, or separate LDS arrays
// (which the compiler can tell apart from LDS written by direct-to-LDS loads).
template <class L, int RT>
struct PrepView {
    using PD = PrepDims<L, RT>;
    float (&qsrc)[2][L::D][4 * RT];
    float (&w)[4 * RT][PD::NR];
    int (&F)[4 * RT][L::NCLS];
};

template <class L, int RT>
__device__ __forceinline__ PrepView<L, RT> view_of(PrepScratch<L, RT> &s) {
    return PrepView<L, RT>{s.qsrc, s.w, s.F};
}

// One GEMV item of the query preparation: (row tile, matrix row, part). Part p of a row
// takes the float4 columns p, p+CPR, ... so that the CPR lanes of a row read contiguous
// 16*CPR-byte runs.
template <class L, int RT>
struct PrepItem {
    static constexpr int NR = PrepDims<L, RT>::NR, CPR = PrepDims<L, RT>::CPR;
    static constexpr int CH = L::D / CPR;  // columns per chunk
    const float *row;
    int K, off, part, r, qb;
    bool rotated;

    __device__ __forceinline__ PrepItem(int it, const float *__restrict__ rot, const float *__restrict__ proj) {
        part = it % CPR;
        const int item = it / CPR;
        r = item % NR;
        qb = 4 * (item / NR);
        rotated = r < L::D;
        off = 0;
        if (rotated) {
            const int g = r < L::D0 ? 0 : 1;
            off = g ? L::D0 : 0;
            K = g ? L::D1 : L::D0;
            row = rot + (g ? (size_t)L::D0 * L::D0 : 0) + (size_t)(r - off) * K;
        } else {
            K = L::D;
            row = proj + (size_t)(r - L::D) * L::D;
        }
    }

    __device__ __forceinline__ void load(f32x4 (&m)[CH / 4]) const {
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) {
            const int k = 4 * (i * CPR + part);
            m[i] = k < K ? *reinterpret_cast<const f32x4 *>(row + k) : f32x4{0, 0, 0, 0};
        }
    }
};

// The prologue's global reads that a thread can request up front: its first query
// element and the matrix chunks of its first PRE GEMV items (items tid, tid + NT, ...).
// Issuing them before any other vector-memory traffic lets the later waits on them ignore
// that traffic (loads complete in issue order).
template <class L, int RT, int NT>
struct PrepRegs {
    static constexpr int ITEMS = PrepItem<L, RT>::NR * RT * PrepItem<L, RT>::CPR;
    static constexpr int PER = (ITEMS + NT - 1) / NT;  // items per thread
    // of which preloaded: two where a thread has 256 VGPRs, one in 1024-thread work-groups
    // (128 VGPRs; two 32-column chunks there spilled to scratch at d = 256)
    static constexpr int PRE = PER < 2 ? PER : (NT >= 1024 ? 1 : 2);
    float qv, qg;
    f32x4 m[PRE][PrepItem<L, RT>::CH / 4];
};

template <class L, int RT, int NT>
__device__ __forceinline__ void prep_load(PrepRegs<L, RT, NT> &pr, int tid, const float *__restrict__ q, long bank,
                                          int G, int q0, const float *__restrict__ rot,
                                          const float *__restrict__ proj, const int *__restrict__ chan) {
    using PR = PrepRegs<L, RT, NT>;
    constexpr int NQ4 = 4 * RT;
    {
        // an unconditional load at a clamped address (a load inside a branch would be waited
        // for where the branch joins, before the matrix loads below are even issued); the
        // channel-permuted copy needs the channel list first and is read in prep_finish
        const int e = min(tid, NQ4 * L::D - 1);
        const int qq = e / L::D, c = e % L::D;
        const float v = q[((size_t)bank * G + min(q0 + qq, G - 1)) * L::D + c];
        const bool use = (NT <= NQ4 * L::D || tid < NQ4 * L::D) && q0 + qq < G;
        pr.qv = __uint_as_float(__float_as_uint(v) & (use ? ~0u : 0u));  // a mask, not a branch
        pr.qg = pr.qv;
    }
#pragma unroll
    for (int k = 0; k < PR::PRE; ++k)
        if (tid + k * NT < PR::ITEMS) PrepItem<L, RT>(tid + k * NT, rot, proj).load(pr.m[k]);
}

template <bool LDS_ONLY>
__device__ __forceinline__ void prep_barrier() {
    if constexpr (LDS_ONLY)
        lds_barrier();
    else
        __syncthreads();
}

// Where the preparation writes its outputs: a flat byte array (the global workspace, or a
// block of LDS), or LDS arrays of one row tile reached by typed indexing.
template <class L>
struct OperandPtr {
    int8_t *frags;   // [RT][NF][64][16 B]
    double *consts;  // [4 RT][NCLS][2]
    __device__ __forceinline__ uint32_t &frag(int rt, int f, int ln, int v) const {
        return *reinterpret_cast<uint32_t *>(frags + ((((size_t)rt * L::NF + f) * 64 + ln) * 16 + 4 * v));
    }
    __device__ __forceinline__ double &cst(int qq, int c, int k) const {
        return consts[((size_t)qq * L::NCLS + c) * 2 + k];
    }
};

template <class L>
struct OperandLds {
    uint32_t (&frags)[L::NF][64][4];
    double (&consts)[4][L::NCLS][2];
    __device__ __forceinline__ uint32_t &frag(int, int f, int ln, int v) const { return frags[f][ln][v]; }
    __device__ __forceinline__ double &cst(int qq, int c, int k) const { return consts[qq][c][k]; }
};

struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

// `hook(k)` runs in every thread right after the k-th of the three work-group barriers
// (k = 1, 2, 3), for work that can interleave with the preparation.
template <class L, int RT, int NT, bool LDS_ONLY = false, class Out = OperandPtr<L>, class Hook = NoHook>
__device__ __forceinline__ void prep_finish(const PrepRegs<L, RT, NT> &pr, int tid, const float *__restrict__ q, long bank,
                                            int G, int q0, const float *__restrict__ rot,
                                            const float *__restrict__ proj, const int *__restrict__ chan,
                                            const PrepArgs &pa, const PrepView<L, RT> &ps, const Out &out,
                                            Hook hook = Hook{}) {
    using PS = PrepDims<L, RT>;
    using PI = PrepItem<L, RT>;
    constexpr int NQ4 = 4 * RT;
    constexpr int NR = PS::NR, CPR = PS::CPR;
    constexpr int CH = PI::CH;
    static_assert(CH % 4 == 0 && 64 % CPR == 0, "bad chunking");
    const int lane = tid & 63, wv = tid / 64;
    for (int e = tid; e < NQ4 * L::D; e += NT) {
        const int qq = e / L::D, c = e % L::D, gq = q0 + qq;
        const float *qrow = q + ((size_t)bank * G + gq) * L::D;
        float a = pr.qv, b = pr.qg;
        if (e != tid) {
            a = gq < G ? qrow[c] : 0.0f;
            b = gq < G ? qrow[chan ? chan[c] : c] : 0.0f;
        } else if (chan) {
            b = gq < G ? qrow[chan[c]] : 0.0f;
        }
        ps.qsrc[0][c][qq] = a;
        ps.qsrc[1][c][qq] = b;
    }
    prep_barrier<LDS_ONLY>();
    hook(1);
    // GEMV items; parts of a row sit in adjacent lanes, rows of a wave form one row block;
    // both are reduced with shuffles in a fixed order.
    for (int it = tid; it < NR * RT * CPR; it += NT) {
        const PI pi(it, rot, proj);
        const int part = pi.part, r = pi.r, qb = pi.qb;
        // operand columns of this row (one array, indexed: no choice between two objects)
        const float(*src)[NQ4] = ps.qsrc[pi.rotated ? 1 : 0] + (pi.rotated ? pi.off : 0);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4 m[CH / 4];
            const int k = (it - tid) / NT;
            if (k < PrepRegs<L, RT, NT>::PRE) {
#pragma unroll
                for (int kk = 0; kk < PrepRegs<L, RT, NT>::PRE; ++kk)
                    if (kk == k)
#pragma unroll
                        for (int i = 0; i < CH / 4; ++i) m[i] = pr.m[kk][i];
            } else {
                pi.load(m);
            }
#pragma unroll
            for (int i = 0; i < CH / 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = min(4 * (i * CPR + part) + e, pi.K - 1);  // past K the loaded value is 0
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
        for (int qq = 0; qq < 4; ++qq) acc[qq] = group_sum_f32<CPR>(acc[qq]);  // the CPR parts of a row
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            if (part == 0) ps.w[qb + qq][r] = acc[qq];
    }
    prep_barrier<LDS_ONLY>();
    hook(2);
    // per (query, term): exponent F from the max |weight|, additive constant from the fp64 sum
    // of the fp32 weights; one wave per (query, term), its lanes over the term's rows, reduced
    // on the vector ALU
    for (int it = wv; it < NQ4 * L::NCLS; it += NT / 64) {
        const int qq = it / L::NCLS, c = it % L::NCLS, gq = q0 + qq;
        const int r0 = c < L::NG ? (c ? L::D0 : 0) : L::D;
        const int r1 = c < L::NG ? (c ? L::D : L::D0) : NR;
        float mxf = 0.0f;
        double sm = 0.0;
        for (int rr = r0 + lane; rr < r1; rr += 64) {
            const float w = ps.w[qq][rr];
            mxf = fmaxf(mxf, fabsf(w));
            sm += (double)w;
        }
        const double mx = (double)dpp_wave_max_f32(mxf);
        sm = dpp_wave_sum_f64(sm);
        if (lane == 0) {
        // (kernel-argument arrays are indexed with constants only: a runtime index would
        // read them through vector memory)
        double wmax;
        if (c < L::NG) {
            double cm = 0.0;
            const int nsub = walsh_planes(c ? L::B1 : L::B0);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                if (s2 < nsub) cm = fmax(cm, fabs(c ? pa.walsh[1][s2] : pa.walsh[0][s2]));
            wmax = mx * cm;
        } else {
            wmax = 2.0 * mx;
        }
        int e = 0;
        if (wmax > 0.0) frexp(wmax, &e);  // wmax < 2^e
        const int F = wmax > 0.0 ? 30 - e : 0;
        ps.F[qq][c] = F;
        out.cst(qq, c, 0) = ldexp(1.0, -F);
        out.cst(qq, c, 1) = gq < G ? (c < L::NG ? -(c ? pa.cmax[1] : pa.cmax[0]) * sm : -sm) : 0.0;
        }
    }
    prep_barrier<LDS_ONLY>();
    hook(3);
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
            constexpr int fg = fc < L::NG ? fc : 0;
            const double mul = fc < L::NG ? (sub == 0   ? pa.walsh[fg][0]
                                             : sub == 1 ? pa.walsh[fg][1]
                                             : sub == 2 ? pa.walsh[fg][2]
                                                        : pa.walsh[fg][3])
                                          : 2.0;
            uint32_t U[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double wt = live ? mul * (double)src[8 * e + t] : 0.0;
                int V = __double2int_rn(wt * scale);
                if (t == 7) V = -V;  // the byte 0x80 reads as -128
                U[e] = (uint32_t)V + 0x80808080u;
            }
            const int rt = qq / 4, ln0 = 16 * gl + 4 * (qq % 4);
#pragma unroll
            for (int limb = 0; limb < 4; ++limb) {
                uint32_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) packed |= (((U[e] >> (8 * limb)) & 0xFFu) ^ 0x80u) << (8 * e);
                out.frag(rt, f, ln0 + limb, v) = packed;
            }
        });
    }
}

template <class L, int RT, int NT>
__device__ __forceinline__ void prep_operands(int tid, const float *__restrict__ q, long bank, int G, int q0,
                                              const float *__restrict__ rot, const float *__restrict__ proj,
                                              const int *__restrict__ chan, const PrepArgs &pa,
                                              PrepScratch<L, RT> &ps, int8_t *frag_out, double *const_out) {
    PrepRegs<L, RT, NT> pr;
    prep_load<L, RT, NT>(pr, tid, q, bank, G, q0, rot, proj, chan);
    prep_finish<L, RT, NT>(pr, tid, q, bank, G, q0, rot, proj, chan, pa, view_of(ps),
                           OperandPtr<L>{frag_out, const_out});
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
    const typename L::NormT *__restrict__ nb;  // its norms
    const typename L::NormT *__restrict__ rb;  // its residual norms
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
            const typename L::NormT *tn = nb + (size_t)tile * (16 * L::NG);
#pragma unroll
            for (int g = 0; g < L::NG; ++g) b.nu[t][g] = norm_f32(tn[j * L::NG + g]);
            b.rho[t] = norm_f32(rb[(size_t)tile * 16 + j]);
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
__global__ __launch_bounds__(256) void score_kernel(const uint32_t *__restrict__ bits,
                                                    const typename L::NormT *__restrict__ norms,
                                                    const typename L::NormT *__restrict__ rnorms,
                                                    const int8_t *__restrict__ frags,
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
    const uint32_t *__restrict__ bits, const typename L::NormT *__restrict__ norms,
    const typename L::NormT *__restrict__ rnorms, const float *__restrict__ q, const float *__restrict__ rot,
    const float *__restrict__ proj, const int *__restrict__ chan, PrepArgs pa, float *__restrict__ scores, int banks,
    long n, int n_tiles, int G, int wgs_per_bank, int tiles_per_wg, ScoreScale sc) {
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
    // the prologue's own reads go first, then the first two batches of tiles, whose latency
    // the rest of the prologue overlaps (loads complete in issue order)
    PrepRegs<L, RT, WAVES * 64> pr;
    prep_load<L, RT, WAVES * 64>(pr, tid, q, bank, G, 0, rot, proj, chan);
    asm volatile("" ::: "memory");
    TileBatch<L, TB> A, B;
    ts.prefetch(A, B);
    prep_finish<L, RT, WAVES * 64>(pr, tid, q, bank, G, 0, rot, proj, chan, pa, view_of(lds.ps),
                                   OperandPtr<L>{&lds.frags[0][0][0][0], &lds.consts[0][0][0]});
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

// ------------------------------------------------------------------------------------------
// Ring-staged fused scorer for up to 4 queries per bank. Key tiles move from HBM straight
// into LDS (global_load_lds_dwordx4), S tiles ahead of the compute in every wave, so the
// loads in flight hold no VGPRs and the first S tiles of every wave stream in while the
// work-group builds its query operands.
//
// A tile slot holds the tile's W bit rows (64 B each: one word of 16 keys), its NG norm rows
// and its residual-norm row, in that order. The waits count only the direct loads issued
// after the awaited tile; loads complete in issue order, so such a wait is exact for the
// tile whatever the score stores pending beside them (it may also wait on those stores,
// which is why each score is stored two tiles late).

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in [15:14])
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int waitcnt_lgkm0() { return 15 | (7 << 4) | (3 << 14); }

template <class L>
struct RingTile {
    static constexpr int ROWS = L::W + L::NG + 1;
    static constexpr int WORDS = ROWS * 16;
    static constexpr int BIT_LOADS = (L::W + 15) / 16;  // 1 KiB direct loads for the bit rows
    static constexpr int LOADS = BIT_LOADS + 1;         // and one for the norm rows
    static_assert(L::NG + 1 <= 16, "norm rows exceed one load");
};

constexpr int RING_WAVES = 16;

template <class L>
constexpr int ring_slots() {
    // the ring and the prologue's scratch within 160 KiB of LDS; at most 8 tiles ahead, 6 for
    // two channel groups (whose three estimator terms leave no registers for a deeper
    // unrolled ring: with 8 slots one VGPR spilled to scratch, and the launch was about 2 %
    // slower on the long-context banks)
    constexpr int budget = 160 * 1024 - (int)sizeof(FusedLds<L, 1>);
    constexpr int s = budget / (RING_WAVES * RingTile<L>::WORDS * 4);
    constexpr int cap = L::NG > 1 ? 6 : 8;
    return (s > cap ? cap : s) & ~1;  // even: the steady state fills the ring by halves
}

// Norms per 16-byte lane load (4 float32 or 8 binary16), and the lanes that load a tile's
// norm rows (the group norms, then the residual norms).
template <class L>
struct NormRows {
    static constexpr int PER = 16 / (int)sizeof(typename L::NormT);
    static constexpr int NU_LANES = 16 * L::NG / PER;
    static constexpr int LANES = NU_LANES + 16 / PER;
};

// Issues the direct loads of one tile into a slot (every lane of the wave calls it):
// `tile_bits` is the tile's bit block, `nr_src` this lane's 16 bytes of the tile's norm
// rows (see NormLane). Every tile is read once, so the loads carry the non-temporal cache
// hint (aux = 2, the nt bit; measured about 0.7 % faster than the default policy).
template <class L>
__device__ __forceinline__ void ring_fetch(const char *tile_bits, const void *nr_src, lds_u32 *slot, int lane) {
    static_for<RingTile<L>::BIT_LOADS>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int rows = L::W - 16 * i < 16 ? L::W - 16 * i : 16;
        if (rows == 16 || lane < 4 * rows)
            __builtin_amdgcn_global_load_lds(tile_bits + 1024 * i + 16 * lane, (lds_void *)(slot + 256 * i), 16, 0,
                                             2);
    });
    if (lane < NormRows<L>::LANES)
        __builtin_amdgcn_global_load_lds(nr_src, (lds_void *)(slot + 16 * L::W), 16, 0, 2);
}

// A lane's share of the norm rows: its source for tile 0 and its stride per tile.
template <class L>
struct NormLane {
    using T = typename L::NormT;
    const T *base;
    int stride;  // norms per tile
    __device__ __forceinline__ NormLane(const T *nb, const T *rb, int lane) {
        using NR = NormRows<L>;
        const bool is_nu = lane < NR::NU_LANES;
        base = is_nu ? nb + NR::PER * lane : rb + NR::PER * (lane - NR::NU_LANES);
        stride = is_nu ? 16 * L::NG : 16;
    }
    __device__ __forceinline__ const T *at(int tile) const { return base + (size_t)tile * stride; }
};

template <class L>
__device__ __forceinline__ const char *tile_bits(const uint32_t *bb, int tile) {
    return reinterpret_cast<const char *>(bb + (size_t)tile * (L::W * 16));
}

// Waits until at most `ahead` tiles' direct loads (and nothing older) are outstanding.
template <class L, int S>
__device__ __forceinline__ void ring_wait(int ahead) {
    static_for<S>([&](auto ac) {
        constexpr int a = decltype(ac)::value;
        if (ahead == a) __builtin_amdgcn_s_waitcnt(waitcnt_vm(a * RingTile<L>::LOADS));
    });
}

template <class L, int S>
__global__ __launch_bounds__(RING_WAVES * 64) void score_ring_kernel(
    const uint32_t *__restrict__ bits, const typename L::NormT *__restrict__ norms,
    const typename L::NormT *__restrict__ rnorms, const float *__restrict__ q, const float *__restrict__ rot,
    const float *__restrict__ proj, const int *__restrict__ chan, PrepArgs pa, float *__restrict__ scores, int banks,
    long n, int n_tiles, int G, int wgs_per_bank, int tiles_per_wg, ScoreScale sc) {
    using RTL = RingTile<L>;
    using PD = PrepDims<L, 1>;
    // the preparation's scratch, operands and ring as separate LDS arrays: LDS accesses to
    // the first ones then never wait for direct-to-LDS loads into the ring
    __shared__ float s_qsrc[2][L::D][4];
    __shared__ float s_w[4][PD::NR];
    __shared__ int s_F[4][L::NCLS];
    __shared__ __attribute__((aligned(16))) uint32_t s_frags[L::NF][64][4];
    __shared__ double s_consts[4][L::NCLS][2];
    __shared__ __attribute__((aligned(16))) uint32_t ring_mem[RING_WAVES][S][RTL::WORDS];
    const long bank = blockIdx.x / wgs_per_bank;
    const int part = blockIdx.x % wgs_per_bank;
    const int tid = threadIdx.x, lane = tid & 63, j = lane & 15, gl = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int w0 = part * tiles_per_wg, w1 = min(w0 + tiles_per_wg, n_tiles);
    const int per = (w1 - w0 + RING_WAVES - 1) / RING_WAVES;
    const int t0 = min(w0 + wv * per, w1), t1 = min(t0 + per, w1);
    const int nt = t1 - t0;
    const long n_pad = (long)n_tiles * 16;
    const uint32_t *bb = bits + (size_t)bank * n_tiles * L::W * 16;
    const typename L::NormT *nb = norms + (size_t)bank * n_pad * L::NG;
    const typename L::NormT *rb = rnorms + (size_t)bank * n_pad;
    float *ob = scores + (size_t)bank * G * n;
    lds_u32 *ring = (lds_u32 *)&ring_mem[wv][0][0];
    const NormLane<L> nl(nb, rb, lane);

    // Prologue. Every wave first requests and consumes its share of the preparation's
    // global reads (loads complete in issue order, and a load consumed while a direct-to-LDS
    // load is pending would wait for that too). It then fills its own ring in four pieces,
    // one before the preparation and one after each of its barriers, so that the fill
    // streams from HBM while the operands are built and no phase stalls on issuing it.
    PrepRegs<L, 1, RING_WAVES * 64> pr;
    prep_load<L, 1, RING_WAVES * 64>(pr, tid, q, bank, G, 0, rot, proj, chan);
    asm volatile("" : "+v"(pr.qv), "+v"(pr.qg));
#pragma unroll
    for (int k = 0; k < PrepRegs<L, 1, RING_WAVES * 64>::PRE; ++k)
#pragma unroll
        for (int i = 0; i < PrepItem<L, 1>::CH / 4; ++i) asm volatile("" : "+v"(pr.m[k][i]));
    asm volatile("" ::: "memory");
    const int tlast = max(t1 - 1, 0);
    // slots past a short run reload its last tile, so the fill has no branches
    auto fill_piece = [&](int piece) {
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (i * 4 / S == piece) {
                const int t = min(t0 + i, tlast);
                ring_fetch<L>(tile_bits<L>(bb, t), nl.at(t), ring + i * RTL::WORDS, lane);
            }
    };
    fill_piece(0);
    PrepView<L, 1> view{s_qsrc, s_w, s_F};
    prep_finish<L, 1, RING_WAVES * 64, true>(pr, tid, q, bank, G, 0, rot, proj, chan, pa, view,
                                             OperandLds<L>{s_frags, s_consts}, fill_piece);
    lds_barrier();
    if (nt <= 0) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        return;
    }
    i8x16 wf[1][L::NF];
#pragma unroll
    for (int f = 0; f < L::NF; ++f) wf[0][f] = *reinterpret_cast<const i8x16 *>(&s_frags[f][lane][0]);
    // per-term constants with the term's scale folded in: est = sum_c s_c (S_c cs_c + ck_c),
    // s_c = nu_g for the code terms of group g and rho for the sketch term
    double cs[L::NCLS], ck[L::NCLS];
    static_for<L::NCLS>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int g = c < L::NG ? c : 0;
        const double f = c < L::NG ? sc.inv_sqrt_d[g] : sc.qjl;
        cs[c] = s_consts[gl][c][0] * f;
        ck[c] = s_consts[gl][c][1] * f;
    });
    // per-lane word offsets inside a slot (lane group gl takes word 4s+gl of key j)
    int woff[L::NSQ];
    bool wlive[L::NSQ];
#pragma unroll
    for (int s = 0; s < L::NSQ; ++s) {
        wlive[s] = 4 * s + gl < L::W;
        woff[s] = (wlive[s] ? 4 * s + gl : 0) * 16 + j;
    }

    // A slot's words for this lane, read in one asm block that ends with its own wait: the
    // compiler sees no LDS access there that it could order against the ring's direct-to-LDS
    // loads, so the only waits on those are the explicit ones above. Lane group gl takes
    // word 4s+gl of key j (words past the tile's W are read from the slot's later rows and
    // dropped); norms of key j; residual norm of key j.
    // With binary16 norms the norm rows are half as long: key j's norms at 2 (NG j + g)
    // bytes into them, its residual norm at 2 j bytes past the NG group rows' 32 NG bytes.
    static_assert(4 * L::NSQ <= RingTile<L>::ROWS && L::NSQ <= 4 && L::NG <= 2, "slot read layout");
    constexpr uint32_t NB = sizeof(typename L::NormT);
    const uint32_t lane_w = 4u * lane, lane_n = NB * j * L::NG, lane_r = NB * j;
    auto read_slot = [&](const lds_u32 *slot, uint32_t(&sw)[L::NSQ], float(&nu)[L::NG], float &rho) {
        const uint32_t base = (uint32_t)(uintptr_t)slot;
        uint32_t w[4], nn[2], r;
        constexpr int O1 = (L::NSQ > 1 ? 1 : 0) * 256, O2 = (L::NSQ > 2 ? 2 : 0) * 256,
                      O3 = (L::NSQ > 3 ? 3 : 0) * 256, ON = 64 * L::W, ON1 = 64 * L::W + (L::NG > 1 ? (int)NB : 0),
                      OR = 64 * L::W + 16 * (int)NB * L::NG;
        if constexpr (L::NH)
            asm volatile(
                "ds_read_b32 %0, %7\n"
                "ds_read_b32 %1, %7 offset:%10\n"
                "ds_read_b32 %2, %7 offset:%11\n"
                "ds_read_b32 %3, %7 offset:%12\n"
                "ds_read_u16 %4, %8 offset:%13\n"
                "ds_read_u16 %5, %8 offset:%14\n"
                "ds_read_u16 %6, %9 offset:%15\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(nn[0]), "=&v"(nn[1]), "=&v"(r)
                : "v"(base + lane_w), "v"(base + lane_n), "v"(base + lane_r), "i"(O1), "i"(O2), "i"(O3), "i"(ON),
                  "i"(ON1), "i"(OR)
                : "memory");
        else
            asm volatile(
                "ds_read_b32 %0, %7\n"
                "ds_read_b32 %1, %7 offset:%10\n"
                "ds_read_b32 %2, %7 offset:%11\n"
                "ds_read_b32 %3, %7 offset:%12\n"
                "ds_read_b32 %4, %8 offset:%13\n"
                "ds_read_b32 %5, %8 offset:%14\n"
                "ds_read_b32 %6, %9 offset:%15\n"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(nn[0]), "=&v"(nn[1]), "=&v"(r)
                : "v"(base + lane_w), "v"(base + lane_n), "v"(base + lane_r), "i"(O1), "i"(O2), "i"(O3), "i"(ON),
                  "i"(ON1), "i"(OR)
                : "memory");
#pragma unroll
        for (int s = 0; s < L::NSQ; ++s) sw[s] = wlive[s] ? w[s] : 0u;
        if constexpr (L::NH) {
#pragma unroll
            for (int g = 0; g < L::NG; ++g) nu[g] = norm_f32((uint16_t)nn[g]);
            rho = norm_f32((uint16_t)r);
        } else {
#pragma unroll
            for (int g = 0; g < L::NG; ++g) nu[g] = __uint_as_float(nn[g]);
            rho = __uint_as_float(r);
        }
    };
    auto tile_est = [&](const uint32_t(&sw)[L::NSQ], const float(&nu)[L::NG], float rho) -> float {
        i32x4 acc[1][L::NCLS];
        score_tile<L, 1>(sw, wf, acc);
        double est = 0.0;
        static_for<L::NCLS>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            constexpr int g = c < L::NG ? c : 0;
            const double s = c < L::NG ? (double)nu[g] : (double)rho;
            est = fma(s, fma(limbs_to_f64<L::class_positions(c)>(acc[0][c]), cs[c], ck[c]), est);
        });
        return (float)est;
    };

    // Steady state, for four live queries: groups of U = S/2 tiles that fill one half of the
    // ring, so tile i sits in slot (i / U odd ? U : 0) + k for its position k in the group;
    // every refill stays inside the run and every key is below n. Waits, store offsets and
    // slot offsets inside a half are then constants; the scores of a group are stored
    // during the next one.
    constexpr int U = S / 2;
    static_assert(S % 2 == 0, "the ring is filled by halves");
    int i = 0;
    const int full = (int)(n >> 4);  // tiles whose 16 keys are all below n
    const int loff = gl * (int)n + j;  // lane offset into the bank's score rows
    // Scores stored one float per lane (16 lanes: 64 contiguous bytes of a query row) carry the
    // non-temporal hint in the per-tile loop at the end of a run, and in the steady state only
    // for two channel groups. Measured against plain stores in one process on one box: hint
    // everywhere made the long-context banks (two groups, 3-tile ring halves) about 8 % faster
    // but the decode shapes at b = 4 (one group, 3-tile halves) about 8 % slower; the hint in
    // the end loop alone left b = 4 unchanged, made b = 3 (whose last 8 tiles per wave take
    // that loop) about 2 % faster and gave the long-context banks under half of their gain.
    constexpr bool NT_GROUP = L::NG > 1;
    auto store1 = [](float *p, float v) {
        if constexpr (NT_GROUP)
            __builtin_nontemporal_store(v, p);
        else
            *p = v;
    };
    // Scores of a group of four tiles leave as one 16-byte store per lane: a 4 x 4 transpose
    // inside each lane quad (tile index <-> key bits 0-1) gives lane 4c + x the keys
    // 4c .. 4c + 3 of tile x, so a query row's 16 lanes cover 256 contiguous bytes with one
    // instruction. Rows must start 16-byte aligned (n a multiple of 4). These stores go
    // through a buffer resource over the bank's score rows (a 32-bit byte range: n < 2^27 at
    // G = 4) with system scope (sc0 sc1: written through the L2): in three same-process A/Bs
    // the decode shapes were 0.9-1.5 % faster than with plain stores (and about 3 % slower
    // with the non-temporal hint instead).
    const bool wide = U == 4 && (n & 3) == 0 && ((uintptr_t)scores & 15) == 0 && n < (1L << 27);
    const int wide_off = gl * (int)n + 16 * (lane & 3) + 4 * ((lane >> 2) & 3);
    const __amdgpu_buffer_rsrc_t srows = __builtin_amdgcn_make_buffer_rsrc(ob, 0, wide ? (int)(16 * n) : 0, BUF_DWORD3);
    auto store_group = [&](float *base, const float(&pv)[U]) {
        if constexpr (U == 4) {
            float v0 = pv[0], v1 = pv[1], v2 = pv[2], v3 = pv[3];
            const bool o = lane & 1, h = lane & 2;
            float r = dpp_mov_f32<DPP_XOR1>(o ? v0 : v1);
            v0 = o ? r : v0;
            v1 = o ? v1 : r;
            r = dpp_mov_f32<DPP_XOR1>(o ? v2 : v3);
            v2 = o ? r : v2;
            v3 = o ? v3 : r;
            r = dpp_mov_f32<DPP_XOR2>(h ? v0 : v2);
            v0 = h ? r : v0;
            v2 = h ? v2 : r;
            r = dpp_mov_f32<DPP_XOR2>(h ? v1 : v3);
            v1 = h ? r : v1;
            v3 = h ? v3 : r;
            const uint32_t off = 4u * (uint32_t)((base - ob) + wide_off);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2),
                                                         __float_as_uint(v3)},
                                                   srows, off, 0, CPOL_SC0 | CPOL_SC1);
        }
    };
    if (G == 4 && 2 * S <= nt && t0 + U <= full) {
        float pend[U];
        auto group = [&](auto store_prev) {
            constexpr bool SP = decltype(store_prev)::value;
            float *prev_out = ob + (size_t)(t0 + i - U) * 16;
            lds_u32 *half = ring + ((i / U) & 1) * (U * RTL::WORDS);
            static_for<U>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                __builtin_amdgcn_s_waitcnt(waitcnt_vm((S - 1) * RTL::LOADS));
                uint32_t sw[L::NSQ];
                float nu[L::NG], rho;
                read_slot(half + k * RTL::WORDS, sw, nu, rho);
                if constexpr (SP) {
                    if (wide) {
                        if (k == 0) store_group(prev_out, pend);
                    } else {
                        store1(prev_out + loff + 16 * k, pend[k]);
                    }
                }
                const int tn = t0 + i + S + k;
                ring_fetch<L>(tile_bits<L>(bb, tn), nl.at(tn), half + k * RTL::WORDS, lane);
                pend[k] = tile_est(sw, nu, rho);
            });
            i += U;
        };
        group(std::false_type{});
        while (i + S + U <= nt && t0 + i + U <= full) group(std::true_type{});
        float *last_out = ob + (size_t)(t0 + i - U) * 16;
        if (wide) {
            store_group(last_out, pend);
        } else {
            static_for<U>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                store1(last_out + loff + 16 * k, pend[k]);
            });
        }
    }
    // the rest one tile at a time: waits by the loads actually issued after the tile,
    // refills while inside the run, stores checked against G and n
    const bool qlive = gl < G;
    for (; i < nt; ++i) {
        ring_wait<L, S>(min(S - 1, nt - 1 - i));
        uint32_t sw[L::NSQ];
        float nu[L::NG], rho;
        read_slot(ring + (i % S) * RTL::WORDS, sw, nu, rho);
        if (i + S < nt) {
            const int tn = t0 + i + S;
            ring_fetch<L>(tile_bits<L>(bb, tn), nl.at(tn), ring + (i % S) * RTL::WORDS, lane);
        }
        const float est = tile_est(sw, nu, rho);
        if (qlive && (long)(t0 + i) * 16 + j < n) __builtin_nontemporal_store(est, ob + (size_t)(t0 + i) * 16 + loff);
    }
}

}  // namespace tq
