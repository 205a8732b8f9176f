/*
 * TurboQuant CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 reference of what the packed-key encode/score path
 * computes. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the product path never does.
 *
 * Everything here follows the method as the source pages describe it:
 *   - turboquant-pytorch write-up (discuss.pytorch.kr, "turboquant-pytorch 소개"),
 *     section "turboquant-pytorch의 2단계 알고리즘 구조": stage 1 rotates each vector
 *     with a random orthogonal matrix and quantises every rotated coordinate on its
 *     own with a Lloyd-Max codebook precomputed for the bell-shaped (normal)
 *     coordinate distribution; stage 2 projects the stage-1 residual with a random
 *     Gaussian matrix and keeps one sign bit per projection, which makes the
 *     inner-product estimate unbiased (the QJL step);
 *   - tambur.pub article on TurboQuant: an MSE-only quantiser biases inner
 *     products, the 1-bit residual correction removes that bias;
 *   - same write-up, usage example: compress(vectors) then
 *     inner_product(query, compressed) estimates query @ vectors.T with the query
 *     kept at full precision.
 *
 * Where the pages leave a step open, the plainest reading is taken; each such
 * reading is marked READING below:
 *   - the rotation is the Q factor of a Householder QR of an i.i.d. N(0,1)
 *     matrix, columns sign-fixed so the triangular factor has a positive
 *     diagonal; coordinate j of the rotated vector is row j of Q times x;
 *   - the codebook is Lloyd-Max for N(0,1) and is applied to the rotated
 *     coordinates scaled to unit variance, z = sqrt(d_g) * (R x)_j / |x|;
 *   - each vector (and each channel group) keeps its norm as float32, the
 *     residual keeps its norm rho as float32; the format variant with 16-bit norms
 *     stores the binary16 rounding of those float32 values, and the reconstruction
 *     that the residual is taken against uses the stored (rounded) norm, so the
 *     sketch corrects exactly what a reader of the bytes rebuilds;
 *   - the sign-sketch scale is sqrt(pi/2)/m * rho (Gaussian sign identity);
 *   - bucket index = number of thresholds t with z >= t (ties go up), with the
 *     decision taken on z rounded to float32 against float32 thresholds;
 *   - sign bit = [p >= 0] with p rounded to float32 (so 0 and -0 give 1).
 *
 * Packed bank format (the layout is this project's own; the pages only say the
 * format is bit-packed codes plus sign metadata):
 *   keys are grouped in tiles of 16; n_pad = 16*ceil(n/16); slots n..n_pad-1 hold
 *   the encoding of the zero vector. A key's record is W 32-bit words:
 *     for each group g: for plane p < b_g: d_g/32 words; word k bit t is bit p of
 *     the bucket index of rotated coordinate 32k+t of group g;
 *     then m/32 sign words; word k bit t is the sign bit of projection row 32k+t.
 *   bits[tile][w][i] (uint32) holds word w of key 16*tile+i.
 *   norms[key][g] (float32), rnorms[key] (float32).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EARG (-1)

typedef struct {
    int d, m, ng;
    int gdim[2], gbits[2];
    const int *chan; /* [d]: group 0 channels then group 1 channels; NULL = identity */
    int norm16;      /* 1: norms stored at IEEE binary16 precision (format variant) */
} orc_cfg;

static int cfg_chan(const orc_cfg *c, int pos) { return c->chan ? c->chan[pos] : pos; }

static int cfg_words(const orc_cfg *c) {
    int w = c->m / 32;
    for (int g = 0; g < c->ng; ++g) w += c->gbits[g] * (c->gdim[g] / 32);
    return w;
}

static int cfg_check(const orc_cfg *c) {
    if (c->ng < 1 || c->ng > 2 || c->d <= 0 || c->d > 1024 || c->m < 0 || c->m > 1024 || c->m % 32) return ORC_EARG;
    if (c->norm16 != 0 && c->norm16 != 1) return ORC_EARG;
    int s = 0;
    for (int g = 0; g < c->ng; ++g) {
        if (c->gdim[g] <= 0 || c->gdim[g] % 32 || c->gbits[g] < 1 || c->gbits[g] > 4) return ORC_EARG;
        s += c->gdim[g];
    }
    return s == c->d ? ORC_OK : ORC_EARG;
}

int orc_words_per_key(const orc_cfg *c) { return cfg_check(c) ? ORC_EARG : cfg_words(c); }

/* Threads of the OpenMP loops from here on (the benchmark times the oracle on one core
 * too); returns the previous count, or 1 without OpenMP. */
int orc_set_threads(int n) {
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    if (n > 0) omp_set_num_threads(n);
    return prev;
#else
    (void)n;
    return 1;
#endif
}

/* ------------------------------------------------------------------------------ */
/* Lloyd-Max codebook for the standard normal (stage 1's "precomputed codebook").   */
/* ------------------------------------------------------------------------------ */

static double npdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }
static double ncdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* A 1-D distribution Lloyd's algorithm runs on: the standard normal (pts == NULL),
 * or a weighted empirical set of points. */
typedef struct {
    const double *pts, *w;
    long n;
} orc_dist;

/* Mass, first and second moment of the distribution on the cell [a, b). */
static void cell_moments(const orc_dist *D, double a, double b, double *m0, double *m1, double *m2) {
    if (!D->pts) {
        double p = ncdf(b) - ncdf(a);
        double apa = isinf(a) ? 0.0 : a * npdf(a), bpb = isinf(b) ? 0.0 : b * npdf(b);
        *m0 = p;
        *m1 = npdf(a) - npdf(b);
        *m2 = p - (bpb - apa);
        return;
    }
    double s0 = 0, s1 = 0, s2 = 0;
    for (long i = 0; i < D->n; ++i) {
        double x = D->pts[i];
        if (x >= a && x < b) {
            double w = D->w ? D->w[i] : 1.0;
            s0 += w;
            s1 += w * x;
            s2 += w * x * x;
        }
    }
    *m0 = s0;
    *m1 = s1;
    *m2 = s2;
}

/* Lloyd's two optimality conditions iterated to a fixed point: every threshold is
 * the midpoint of its two neighbouring centroids; every centroid is the mean of
 * the distribution restricted to its cell (an empty cell keeps its centroid).
 * c[L] holds the start on entry and the fixed point on exit. */
static int lloyd(const orc_dist *D, int L, double *c, double *thr, double *mse_out, int max_iter) {
    int it = 0;
    for (; it < max_iter; ++it) {
        double delta = 0.0, nc[64];
        for (int k = 0; k < L; ++k) {
            double a = k == 0 ? -INFINITY : 0.5 * (c[k - 1] + c[k]);
            double b = k == L - 1 ? INFINITY : 0.5 * (c[k] + c[k + 1]);
            double m0, m1, m2;
            cell_moments(D, a, b, &m0, &m1, &m2);
            nc[k] = m0 > 0 ? m1 / m0 : c[k];
            delta = fmax(delta, fabs(nc[k] - c[k]));
        }
        for (int k = 0; k < L; ++k) c[k] = nc[k];
        if (delta <= 1e-15) break;
    }
    double mse = 0.0;
    for (int k = 0; k < L; ++k) {
        double a = k == 0 ? -INFINITY : 0.5 * (c[k - 1] + c[k]);
        double b = k == L - 1 ? INFINITY : 0.5 * (c[k] + c[k + 1]);
        double m0, m1, m2;
        cell_moments(D, a, b, &m0, &m1, &m2);
        mse += m2 - 2.0 * c[k] * m1 + c[k] * c[k] * m0;
    }
    for (int k = 0; k + 1 < L; ++k) thr[k] = 0.5 * (c[k] + c[k + 1]);
    if (mse_out) *mse_out = mse;
    return it;
}

/* Lloyd-Max codebook for N(0,1) with 2^bits levels (the "precomputed codebook" of
 * stage 1). Started from a symmetric grid; N(0,1) is symmetric, so the exact fixed
 * point is too, and the result is symmetrised to remove floating-point drift
 * (this makes the middle threshold exactly 0). */
int orc_codebook(int bits, double *cent, double *thr, double *mse_out, int *iters_out) {
    if (bits < 1 || bits > 6) return ORC_EARG;
    const int L = 1 << bits;
    double c[64], t[64];
    for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L;
    orc_dist D = {NULL, NULL, 0};
    int it = lloyd(&D, L, c, t, NULL, 1000000);
    for (int k = 0; k < L / 2; ++k) {
        double a = 0.5 * (c[L - 1 - k] - c[k]);
        c[k] = -a;
        c[L - 1 - k] = a;
    }
    double mse;
    lloyd(&D, L, c, t, &mse, 0); /* zero iterations: thresholds and MSE of c */
    for (int k = 0; k < L; ++k) cent[k] = c[k];
    for (int k = 0; k + 1 < L; ++k) thr[k] = t[k];
    if (mse_out) *mse_out = mse;
    if (iters_out) *iters_out = it;
    return ORC_OK;
}

/* The same iteration on a weighted empirical set (w may be NULL = unit weights).
 * cent[L]: start on entry, fixed point on exit. */
int orc_lloyd_empirical(const double *pts, const double *w, long n, int L, double *cent, double *thr,
                        double *mse_out, int max_iter) {
    if (L < 1 || L > 64 || n < 1) return ORC_EARG;
    orc_dist D = {pts, w, n};
    return lloyd(&D, L, cent, thr, mse_out, max_iter);
}

/* Bucket index of one coordinate: the number of thresholds t with z >= t. */
int orc_bucketize(float z, const float *thr, int L) {
    int idx = 0;
    for (int t = 0; t < L - 1; ++t) idx += z >= thr[t];
    return idx;
}

/* ------------------------------------------------------------------------------ */
/* Random orthogonal rotation: Householder QR of a Gaussian matrix, sign-fixed.     */
/* ------------------------------------------------------------------------------ */

/* gauss: d x d row-major. rot: d x d row-major output, rot = Q diag(sign(diag(Rqr))). */
int orc_rotation(int d, const float *gauss, double *rot) {
    if (d <= 0) return ORC_EARG;
    double *A = (double *)malloc(sizeof(double) * d * d);
    double *Q = (double *)malloc(sizeof(double) * d * d);
    double *v = (double *)malloc(sizeof(double) * d);
    for (int i = 0; i < d * d; ++i) A[i] = gauss[i];
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) Q[i * d + j] = i == j ? 1.0 : 0.0;
    for (int k = 0; k < d - 1; ++k) {
        double nx = 0.0;
        for (int i = k; i < d; ++i) nx += A[i * d + k] * A[i * d + k];
        nx = sqrt(nx);
        if (nx == 0.0) continue;
        double alpha = A[k * d + k] >= 0 ? -nx : nx; /* reflect x onto alpha*e1 */
        for (int i = 0; i < d; ++i) v[i] = 0.0;
        for (int i = k; i < d; ++i) v[i] = A[i * d + k];
        v[k] -= alpha;
        double vv = 0.0;
        for (int i = k; i < d; ++i) vv += v[i] * v[i];
        if (vv == 0.0) continue;
        /* A <- H A, H = I - 2 v v^T / (v^T v) */
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            for (int i = k; i < d; ++i) s += v[i] * A[i * d + j];
            s *= 2.0 / vv;
            for (int i = k; i < d; ++i) A[i * d + j] -= s * v[i];
        }
        /* Q <- Q H */
        for (int i = 0; i < d; ++i) {
            double s = 0.0;
            for (int j = k; j < d; ++j) s += Q[i * d + j] * v[j];
            s *= 2.0 / vv;
            for (int j = k; j < d; ++j) Q[i * d + j] -= s * v[j];
        }
    }
    for (int j = 0; j < d; ++j) {
        double sg = A[j * d + j] < 0 ? -1.0 : 1.0;
        for (int i = 0; i < d; ++i) rot[i * d + j] = Q[i * d + j] * sg;
    }
    free(A);
    free(Q);
    free(v);
    return ORC_OK;
}

/* The IEEE 754 binary16 value nearest to x (ties to even), returned as a float: 11
 * significant bits for |x| >= 2^-14, a multiple of 2^-24 below that, infinity from
 * 65520 (the midpoint above the largest finite value, 65504) up. Scaling by a power of
 * two and rint (round-to-nearest-even, the default mode) are exact in double. */
static float round_binary16(float x) {
    if (x == 0.0f || isnan(x) || isinf(x)) return x;
    const double a = fabs((double)x);
    if (a >= 65520.0) return x > 0 ? INFINITY : -INFINITY;
    int e;
    (void)frexp(a, &e); /* a = f 2^e, f in [0.5, 1): leading bit 2^(e-1) */
    const int lead = e - 1 < -14 ? -14 : e - 1;
    const double quantum = ldexp(1.0, lead - 10);
    const double r = rint(a / quantum) * quantum;
    return (float)(x > 0 ? r : -r);
}

/* A stored norm: float32, or (format variant) the binary16 rounding of that float32. */
static float stored_norm(const orc_cfg *c, double v) {
    const float f = (float)v;
    return c->norm16 ? round_binary16(f) : f;
}

float orc_round_binary16(float x) { return round_binary16(x); }

/* ------------------------------------------------------------------------------ */
/* Encode: stage 1 (rotate, quantise per coordinate) + stage 2 (residual signs).    */
/* ------------------------------------------------------------------------------ */

static void put_bit(uint32_t *bits, int W, long key, int word, int bit, int val) {
    long tile = key / 16, i = key % 16;
    uint32_t *w = &bits[(tile * W + word) * 16 + i];
    if (val) *w |= (uint32_t)1u << bit;
}

static int get_bit(const uint32_t *bits, int W, long key, int word, int bit) {
    long tile = key / 16, i = key % 16;
    return (int)((bits[(tile * W + word) * 16 + i] >> bit) & 1u);
}

/* rot: group rotations concatenated (d_0 x d_0 then d_1 x d_1), fp64.
 * proj: S, m x d float32 (original channel order). cent/thr: per group, 16/15 slots.
 * keys: n x d float32. Writes n_pad keys (zero-vector encodings in the padding). */
/* As orc_encode, also returning (nullable) the fp64 quantities each decision was taken on:
 * z_out[key][pos] (unit-variance rotated coordinates, group order) and p_out[key][i]
 * (sketch projections of the residual), for keys < n. */
int orc_encode_trace(const orc_cfg *c, const double *rot, const float *proj, const double *cent, const float *thr,
                     const float *keys, long n, uint32_t *bits, float *norms, float *rnorms, double *z_out,
                     double *p_out);

int orc_encode(const orc_cfg *c, const double *rot, const float *proj, const double *cent, const float *thr,
               const float *keys, long n, uint32_t *bits, float *norms, float *rnorms) {
    return orc_encode_trace(c, rot, proj, cent, thr, keys, n, bits, norms, rnorms, NULL, NULL);
}

int orc_encode_trace(const orc_cfg *c, const double *rot, const float *proj, const double *cent, const float *thr,
                     const float *keys, long n, uint32_t *bits, float *norms, float *rnorms, double *z_out,
                     double *p_out) {
    if (cfg_check(c)) return ORC_EARG;
    const int d = c->d, m = c->m, W = cfg_words(c);
    const long n_pad = 16 * ((n + 15) / 16);
    memset(bits, 0, sizeof(uint32_t) * (size_t)n_pad * W);
#pragma omp parallel for schedule(dynamic, 64)
    for (long key = 0; key < n_pad; ++key) {
        double x[1024], xhat[1024], y[1024], r[1024];
        for (int k = 0; k < d; ++k) x[k] = key < n ? (double)keys[key * d + k] : 0.0;
        for (int k = 0; k < d; ++k) xhat[k] = 0.0;
        int off = 0, word0 = 0;
        const double *Rg = rot;
        for (int g = 0; g < c->ng; ++g) {
            const int dg = c->gdim[g], L = 1 << c->gbits[g];
            double nu2 = 0.0;
            for (int k = 0; k < dg; ++k) {
                double v = x[cfg_chan(c, off + k)];
                nu2 += v * v;
            }
            const double nu = sqrt(nu2);
            const float nu_s = stored_norm(c, nu);
            norms[key * c->ng + g] = nu_s;
            for (int j = 0; j < dg; ++j) {
                double s = 0.0;
                for (int k = 0; k < dg; ++k) s += Rg[j * dg + k] * x[cfg_chan(c, off + k)];
                y[j] = s;
            }
            double coef[1024];
            for (int j = 0; j < dg; ++j) {
                double z = nu > 0.0 ? sqrt((double)dg) * y[j] / nu : 0.0;
                if (z_out && key < n) z_out[key * d + off + j] = z;
                int idx = orc_bucketize((float)z, thr + g * 15, L);
                for (int p = 0; p < c->gbits[g]; ++p)
                    put_bit(bits, W, key, word0 + p * (dg / 32) + j / 32, j % 32, (idx >> p) & 1);
                coef[j] = cent[g * 16 + idx];
            }
            /* xhat_g = (nu_stored / sqrt(d_g)) R_g^T c[idx]: what a decoder rebuilds from the bytes */
            for (int k = 0; k < dg; ++k) {
                double s = 0.0;
                for (int j = 0; j < dg; ++j) s += Rg[j * dg + k] * coef[j];
                xhat[cfg_chan(c, off + k)] = ((double)nu_s / sqrt((double)dg)) * s;
            }
            word0 += c->gbits[g] * (dg / 32);
            off += dg;
            Rg += (long)dg * dg;
        }
        if (m > 0) {
            double rho2 = 0.0;
            for (int k = 0; k < d; ++k) {
                r[k] = x[k] - xhat[k];
                rho2 += r[k] * r[k];
            }
            rnorms[key] = stored_norm(c, sqrt(rho2));
            for (int i = 0; i < m; ++i) {
                double p = 0.0;
                for (int k = 0; k < d; ++k) p += (double)proj[(long)i * d + k] * r[k];
                if (p_out && key < n) p_out[key * m + i] = p;
                put_bit(bits, W, key, word0 + i / 32, i % 32, (float)p >= 0.0f);
            }
        } else if (rnorms) {
            rnorms[key] = 0.0f;
        }
    }
    return ORC_OK;
}

/* Bucket indices of one key, unpacked from the bank: idx[pos] in grouped order. */
static void unpack_codes(const orc_cfg *c, const uint32_t *bits, long key, int *idx) {
    const int W = cfg_words(c);
    int off = 0, word0 = 0;
    for (int g = 0; g < c->ng; ++g) {
        const int dg = c->gdim[g];
        for (int j = 0; j < dg; ++j) {
            int v = 0;
            for (int p = 0; p < c->gbits[g]; ++p) v |= get_bit(bits, W, key, word0 + p * (dg / 32) + j / 32, j % 32) << p;
            idx[off + j] = v;
        }
        word0 += c->gbits[g] * (dg / 32);
        off += dg;
    }
}

int orc_unpack(const orc_cfg *c, const uint32_t *bits, long n, int32_t *codes, uint8_t *signs) {
    if (cfg_check(c)) return ORC_EARG;
    const int W = cfg_words(c);
    int cw = 0;
    for (int g = 0; g < c->ng; ++g) cw += c->gbits[g] * (c->gdim[g] / 32);
    for (long key = 0; key < n; ++key) {
        int idx[1024];
        unpack_codes(c, bits, key, idx);
        for (int j = 0; j < c->d; ++j) codes[key * c->d + j] = idx[j];
        for (int i = 0; i < c->m; ++i) signs[key * c->m + i] = (uint8_t)get_bit(bits, W, key, cw + i / 32, i % 32);
    }
    return ORC_OK;
}

/* Decoder of the stage-1 part: xhat in the original channel order (fp64). */
int orc_decode(const orc_cfg *c, const double *rot, const double *cent, const uint32_t *bits, const float *norms,
               long n, double *out) {
    if (cfg_check(c)) return ORC_EARG;
    const int d = c->d;
#pragma omp parallel for schedule(dynamic, 64)
    for (long key = 0; key < n; ++key) {
        int idx[1024];
        unpack_codes(c, bits, key, idx);
        int off = 0;
        const double *Rg = rot;
        for (int g = 0; g < c->ng; ++g) {
            const int dg = c->gdim[g];
            const double sc = (double)norms[key * c->ng + g] / sqrt((double)dg);
            for (int k = 0; k < dg; ++k) {
                double s = 0.0;
                for (int j = 0; j < dg; ++j) s += Rg[j * dg + k] * cent[g * 16 + idx[off + j]];
                out[key * d + cfg_chan(c, off + k)] = sc * s;
            }
            off += dg;
            Rg += (long)dg * dg;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Score: the asymmetric estimator; the query stays at full precision.              */
/*   est = sum_g (nu_g/sqrt(d_g)) <R_g q_g, c_g[idx_g]>                               */
/*       + sqrt(pi/2)/m * rho * <S q, 2*bits - 1>                                      */
/* ------------------------------------------------------------------------------ */

/* Rotated and projected query: qr[pos] (grouped order, length d), qs[i] (length m). */
static void prep_query(const orc_cfg *c, const double *rot, const float *proj, const float *q, double *qr, double *qs) {
    int off = 0;
    const double *Rg = rot;
    for (int g = 0; g < c->ng; ++g) {
        const int dg = c->gdim[g];
        for (int j = 0; j < dg; ++j) {
            double s = 0.0;
            for (int k = 0; k < dg; ++k) s += Rg[j * dg + k] * (double)q[cfg_chan(c, off + k)];
            qr[off + j] = s;
        }
        off += dg;
        Rg += (long)dg * dg;
    }
    for (int i = 0; i < c->m; ++i) {
        double s = 0.0;
        for (int k = 0; k < c->d; ++k) s += (double)proj[(long)i * c->d + k] * (double)q[k];
        qs[i] = s;
    }
}

static double est_one(const orc_cfg *c, const double *cent, const uint32_t *bits, const float *norms,
                      const float *rnorms, long key, const double *qr, const double *qs) {
    const int W = cfg_words(c);
    int idx[1024];
    unpack_codes(c, bits, key, idx);
    double est = 0.0;
    int off = 0, cw = 0;
    for (int g = 0; g < c->ng; ++g) {
        const int dg = c->gdim[g];
        double s = 0.0;
        for (int j = 0; j < dg; ++j) s += qr[off + j] * cent[g * 16 + idx[off + j]];
        est += ((double)norms[key * c->ng + g] / sqrt((double)dg)) * s;
        cw += c->gbits[g] * (dg / 32);
        off += dg;
    }
    if (c->m > 0) {
        double s = 0.0;
        for (int i = 0; i < c->m; ++i) s += qs[i] * (get_bit(bits, W, key, cw + i / 32, i % 32) ? 1.0 : -1.0);
        est += sqrt(M_PI / 2.0) / (double)c->m * (double)rnorms[key] * s;
    }
    return est;
}

/* scores[g][key] for all G queries and n keys of one bank. */
int orc_score(const orc_cfg *c, const double *rot, const float *proj, const double *cent, const uint32_t *bits,
              const float *norms, const float *rnorms, long n, const float *q, int G, double *scores) {
    if (cfg_check(c)) return ORC_EARG;
    double *qr = (double *)malloc(sizeof(double) * (size_t)G * c->d);
    double *qs = (double *)malloc(sizeof(double) * (size_t)G * (c->m > 0 ? c->m : 1));
    for (int g = 0; g < G; ++g) prep_query(c, rot, proj, q + (long)g * c->d, qr + (long)g * c->d, qs + (long)g * c->m);
#pragma omp parallel for schedule(dynamic, 256)
    for (long key = 0; key < n; ++key)
        for (int g = 0; g < G; ++g)
            scores[(long)g * n + key] = est_one(c, cent, bits, norms, rnorms, key, qr + (long)g * c->d, qs + (long)g * c->m);
    free(qr);
    free(qs);
    return ORC_OK;
}

/* Scores of selected (query, key) pairs: out[t] = est(q[qi[t]], key ki[t]). */
int orc_score_pairs(const orc_cfg *c, const double *rot, const float *proj, const double *cent, const uint32_t *bits,
                    const float *norms, const float *rnorms, const float *q, int G, const int32_t *qi,
                    const int64_t *ki, long npairs, double *out) {
    if (cfg_check(c)) return ORC_EARG;
    double *qr = (double *)malloc(sizeof(double) * (size_t)G * c->d);
    double *qs = (double *)malloc(sizeof(double) * (size_t)G * (c->m > 0 ? c->m : 1));
#pragma omp parallel for
    for (int g = 0; g < G; ++g) prep_query(c, rot, proj, q + (long)g * c->d, qr + (long)g * c->d, qs + (long)g * c->m);
#pragma omp parallel for schedule(dynamic, 64)
    for (long t = 0; t < npairs; ++t)
        out[t] = est_one(c, cent, bits, norms, rnorms, ki[t], qr + (long)qi[t] * c->d, qs + (long)qi[t] * c->m);
    free(qr);
    free(qs);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Top-k of estimated scores per query: larger score first, equal scores by lower   */
/* key index (vector search over the estimates).                                     */
/* ------------------------------------------------------------------------------ */

typedef struct {
    double s;
    long i;
} orc_item;

static int item_cmp(const void *a, const void *b) {
    const orc_item *x = (const orc_item *)a, *y = (const orc_item *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);
}

/* scores: G x n (fp64). vals/idx: G x k. Full sort per query. */
int orc_topk(const double *scores, long n, int G, int k, double *vals, int64_t *idx) {
    if (k < 1 || k > n) return ORC_EARG;
#pragma omp parallel for
    for (int g = 0; g < G; ++g) {
        orc_item *it = (orc_item *)malloc(sizeof(orc_item) * n);
        for (long i = 0; i < n; ++i) {
            it[i].s = scores[(long)g * n + i];
            it[i].i = i;
        }
        qsort(it, n, sizeof(orc_item), item_cmp);
        for (int t = 0; t < k; ++t) {
            vals[(long)g * k + t] = it[t].s;
            idx[(long)g * k + t] = it[t].i;
        }
        free(it);
    }
    return ORC_OK;
}
