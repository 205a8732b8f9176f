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

// Fixed-point split of V (|V| <= 2^30 + 1) into balanced signed bytes, V = sum l_k 256^k.
__device__ __forceinline__ int8_t limb_of(long long V, int limb) {
    long long r = V;
    int8_t l = 0;
    for (int k = 0; k <= limb; ++k) {
        l = (int8_t)(((r + 128) & 255) - 128);
        r = (r - l) / 256;
    }
    return l;
}

// One work-group per (bank, query slot). Writes
//   frags [bank][Gpad/4][NF][64 lanes][16 bytes]  (the A operands, lane order of the MFMA)
//   consts[bank][Gpad][NCLS][2] = {2^-F, additive constant} (fp64)
template <class L>
__global__ __launch_bounds__(256) void qprep_kernel(const float *__restrict__ q, const float *__restrict__ rot,
                                                    const float *__restrict__ proj, const int *__restrict__ chan,
                                                    PrepArgs pa, int G, int Gpad, int8_t *__restrict__ frags,
                                                    double *__restrict__ consts) {
    __shared__ double qv[L::D], qr[L::D], qs[L::M];
    __shared__ double red_max[256][L::NCLS], red_sum[256][L::NCLS];
    __shared__ int sF[L::NCLS];
    const int bank = blockIdx.x / Gpad, qq = blockIdx.x % Gpad, tid = threadIdx.x;
    const bool valid = qq < G;
    for (int c = tid; c < L::D; c += 256) qv[c] = valid ? (double)q[((size_t)bank * G + qq) * L::D + c] : 0.0;
    __syncthreads();
    // R_g q_g (group order) and S q, fp64 sums
    for (int pos = tid; pos < L::D; pos += 256) {
        const int g = pos < L::D0 ? 0 : 1;
        const int dg = g ? L::D1 : L::D0, off = g ? L::D0 : 0, j = pos - off;
        const float *Rg = rot + (g ? (size_t)L::D0 * L::D0 : 0) + (size_t)j * dg;
        double s = 0.0;
        for (int k = 0; k < dg; ++k) s += (double)Rg[k] * qv[chan ? chan[off + k] : off + k];
        qr[pos] = s;
    }
    for (int i = tid; i < L::M; i += 256) {
        const float *Si = proj + (size_t)i * L::D;
        double s = 0.0;
        for (int k = 0; k < L::D; ++k) s += (double)Si[k] * qv[k];
        qs[i] = s;
    }
    __syncthreads();
    // per-class max |weight| and sum of the raw operand (for the additive constant)
    double mx[L::NCLS], sm[L::NCLS];
    for (int c = 0; c < L::NCLS; ++c) mx[c] = sm[c] = 0.0;
    for (int pos = tid; pos < L::D; pos += 256) {
        const int g = pos < L::D0 ? 0 : 1;
        mx[g] = fmax(mx[g], fabs(qr[pos]));
        sm[g] += qr[pos];
    }
    for (int i = tid; i < L::M; i += 256) {
        mx[L::NG] = fmax(mx[L::NG], fabs(qs[i]));
        sm[L::NG] += qs[i];
    }
    for (int c = 0; c < L::NCLS; ++c) {
        red_max[tid][c] = mx[c];
        red_sum[tid][c] = sm[c];
    }
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s)
            for (int c = 0; c < L::NCLS; ++c) {
                red_max[tid][c] = fmax(red_max[tid][c], red_max[tid + s][c]);
                red_sum[tid][c] += red_sum[tid + s][c];
            }
        __syncthreads();
    }
    if (tid < L::NCLS) {
        const int c = tid;
        double wmax;
        if (c < L::NG) {
            double cmax = 0.0;
            const int nsub = walsh_planes(c ? L::B1 : L::B0);
            for (int s = 0; s < nsub; ++s) cmax = fmax(cmax, fabs(pa.walsh[c][s]));
            wmax = red_max[0][c] * cmax;
        } else {
            wmax = 2.0 * red_max[0][c];
        }
        int e = 0;
        if (wmax > 0.0) frexp(wmax, &e);  // wmax < 2^e
        const int F = wmax > 0.0 ? 30 - e : 0;
        sF[c] = F;
        const double konst = c < L::NG ? -pa.cmax[c] * red_sum[0][c] : -red_sum[0][c];
        double *o = consts + (((size_t)bank * Gpad + qq) * L::NCLS + c) * 2;
        o[0] = ldexp(1.0, -F);
        o[1] = valid ? konst : 0.0;
    }
    __syncthreads();
    // fragments: item = (frag f, lane group gl, limb)
    const int rt = qq / 4, row0 = 4 * (qq % 4);
    for (int item = tid; item < L::NF * 16; item += 256) {
        const int f = item / 16, gl = (item / 4) % 4, limb = item % 4;
        int fq = 0, fh = 0, fc = 0;
        {
            int k = 0;
            for (int q2 = 0; q2 < L::NQ; ++q2)
                for (int h2 = 0; h2 < 2; ++h2)
                    for (int c2 = 0; c2 < L::NCLS; ++c2)
                        if (L::quad_has(q2, c2)) {
                            if (k == f) {
                                fq = q2;
                                fh = h2;
                                fc = c2;
                            }
                            ++k;
                        }
        }
        const DWord dw = L::dword(4 * fq + gl);
        const int F = sF[fc];
        uint32_t out[4];
        for (int v = 0; v < 4; ++v) {
            uint32_t packed = 0;
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * fh + v, pos = 8 * e + t;
                double w = 0.0;
                if (valid && dw.cls == fc) {
                    if (fc < L::NG) {
                        const int off = fc ? L::D0 : 0;
                        w = pa.walsh[fc][dw.sub] * qr[off + 32 * dw.k + pos];
                    } else {
                        w = 2.0 * qs[32 * dw.k + pos];
                    }
                }
                long long V = (long long)llrint(ldexp(w, F - t));
                if (t == 7) V = -V;  // the byte 0x80 reads as -128
                packed |= (uint32_t)(uint8_t)limb_of(V, limb) << (8 * e);
            }
            out[v] = packed;
        }
        const int lane = gl * 16 + row0 + limb;
        uint32_t *dst = reinterpret_cast<uint32_t *>(frags + ((((size_t)bank * (Gpad / 4) + rt) * L::NF + f) * 64 + lane) * 16);
        dst[0] = out[0];
        dst[1] = out[1];
        dst[2] = out[2];
        dst[3] = out[3];
    }
}

// Exact recombination of the four int32 limb sums.
__device__ __forceinline__ double limbs_to_f64(i32x4 a) {
    return fma((double)a[3], 16777216.0, fma((double)a[2], 65536.0, fma((double)a[1], 256.0, (double)a[0])));
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

// Decode-shaped scorer: a wave holds the operands of RT row tiles (G <= 4*RT queries of
// one bank) in VGPRs and streams a contiguous run of 16-key tiles of that bank.
template <class L, int RT>
__global__ __launch_bounds__(256) void score_kernel(const uint32_t *__restrict__ bits, const float *__restrict__ norms,
                                                    const float *__restrict__ rnorms, const int8_t *__restrict__ frags,
                                                    const double *__restrict__ consts, float *__restrict__ scores,
                                                    int banks, long n, int n_tiles, int G, int Gpad, int tiles_per_wave,
                                                    int waves_per_bank, ScoreScale sc) {
    const int lane = threadIdx.x & 63;
    const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long bank = wid / waves_per_bank;
    const int chunk = (int)(wid % waves_per_bank);
    if (bank >= banks) return;
    const int t0 = chunk * tiles_per_wave;
    const int t1 = min(t0 + tiles_per_wave, n_tiles);
    if (t0 >= t1) return;
    const int j = lane & 15, gl = lane >> 4;
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

    const uint32_t *bb = bits + (size_t)bank * n_tiles * L::W * 16;
    const float *nb = norms + (size_t)bank * n_pad * L::NG;
    const float *rb = rnorms + (size_t)bank * n_pad;
    float *ob = scores + (size_t)bank * G * n;

    for (int tile = t0; tile < t1; ++tile) {
        const uint32_t *tb = bb + (size_t)tile * L::W * 16;
        uint32_t sw[L::NSQ];
#pragma unroll
        for (int s = 0; s < L::NSQ; ++s) sw[s] = (4 * s + gl < L::W) ? tb[(4 * s + gl) * 16 + j] : 0u;
        const long key = (long)tile * 16 + j;
        float nu[2];
#pragma unroll
        for (int g = 0; g < L::NG; ++g) nu[g] = nb[key * L::NG + g];
        const float rho = rb[key];

        i32x4 acc[RT][L::NCLS];
        score_tile<L, RT>(sw, wf, acc);

#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            double est = 0.0;
#pragma unroll
            for (int c = 0; c < L::NCLS; ++c) {
                const double dot = fma(limbs_to_f64(acc[rt][c]), cs[rt][c], ck[rt][c]);
                const double scale = c < L::NG ? (double)nu[c] * sc.inv_sqrt_d[c] : (double)rho * sc.qjl;
                est = fma(scale, dot, est);
            }
            const int qq = 4 * rt + gl;
            if (qq < G && key < n) ob[(size_t)qq * n + key] = (float)est;
        }
    }
}

}  // namespace tq
