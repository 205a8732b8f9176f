// C-ABI host library of the gfx950 TurboQuant packed-key path: argument checks, host
// parameter construction (codebook, rotation), workspace planning and kernel dispatch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/tq.h"
#include "tq_encode.h"
#include "tq_encode_gemm.h"
#include "tq_score.h"
#include "tq_topk.h"
#include "tq_attend.h"
#include "tq_measure.h"

using namespace tq;

// ----------------------------------------------------------------------------------------
// Lloyd-Max codebook for N(0,1), computed on the positive half-line (the density is
// symmetric, so the optimum is): positive centroids c_1 < ... < c_{L/2}, thresholds
// 0 = t_0 < t_1 < ... ; iterate t_k = (c_k + c_{k+1})/2 and c_k = E[X | t_{k-1} <= X < t_k].
// Tail masses use erfc so that outer cells keep full relative precision.
// (turboquant-pytorch write-up, stage 1: a Lloyd-Max codebook precomputed for the normal
// distribution of the rotated coordinates.)
// ----------------------------------------------------------------------------------------
static double upper_mass(double x) { return 0.5 * erfc(x / sqrt(2.0)); }  // P(X >= x)
static double density(double x) { return exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }

extern "C" int tq_make_codebook(int bits, float *centroids, float *thresholds, double *mse_out) {
    if (bits < 1 || bits > 4 || !centroids || (bits > 0 && !thresholds)) return TQ_ERR_ARG;
    const int L = 1 << bits, H = L / 2;
    double c[8], t[9];
    for (int k = 0; k < H; ++k) c[k] = 3.0 * (k + 0.5) / H;  // start: even grid on (0, 3)
    t[0] = 0.0;
    for (int iter = 0; iter < 1000000; ++iter) {
        for (int k = 1; k < H; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        t[H] = INFINITY;
        double change = 0.0;
        for (int k = 0; k < H; ++k) {
            const double a = t[k], b = t[k + 1];
            const double mass = upper_mass(a) - (isinf(b) ? 0.0 : upper_mass(b));
            const double first = density(a) - (isinf(b) ? 0.0 : density(b));
            const double nc = first / mass;
            change = fmax(change, fabs(nc - c[k]));
            c[k] = nc;
        }
        if (change < 1e-16) break;
    }
    for (int k = 1; k < H; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    t[H] = INFINITY;
    // MSE over both halves: 2 * sum_k E[(X - c_k)^2 ; cell k]
    double mse = 0.0;
    for (int k = 0; k < H; ++k) {
        const double a = t[k], b = t[k + 1];
        const double m0 = upper_mass(a) - (isinf(b) ? 0.0 : upper_mass(b));
        const double m1 = density(a) - (isinf(b) ? 0.0 : density(b));
        const double m2 = m0 + a * density(a) - (isinf(b) ? 0.0 : b * density(b));
        mse += 2.0 * (m2 - 2.0 * c[k] * m1 + c[k] * c[k] * m0);
    }
    for (int k = 0; k < H; ++k) {
        centroids[H + k] = (float)c[k];
        centroids[H - 1 - k] = -(float)c[k];
    }
    for (int k = 0; k < H; ++k) {
        const float tk = (float)t[k];
        thresholds[H - 1 + k] = tk;
        if (k > 0) thresholds[H - 1 - k] = -tk;
    }
    if (mse_out) *mse_out = mse;
    return TQ_OK;
}

// ----------------------------------------------------------------------------------------
// Lloyd-Max codebook for the exact distribution of a rotated coordinate of a unit vector in
// R^d, in the same units (z = sqrt(d) t). A coordinate t of a uniformly random unit vector
// has density proportional to (1 - t^2)^((d-3)/2) on [-1, 1]; the normal distribution is
// its limit for large d (turboquant-pytorch write-up, stage 1: the rotated coordinates
// follow a bell curve, and the codebook is fitted to that distribution). Same iteration as
// above on z in [0, sqrt(d)]: the first moment of a cell in closed form, its mass and
// second moment by composite Gauss-Legendre quadrature (16 panels x 16 points per cell).
// ----------------------------------------------------------------------------------------
namespace {
struct SphereMarginal {
    double d, e, scale;  // density scale * (1 - z^2/d)^e on |z| < sqrt(d), e = (d - 3)/2
    explicit SphereMarginal(int dim) : d(dim), e(0.5 * (dim - 3)) {
        scale = exp(lgamma(0.5 * dim) - lgamma(0.5 * (dim - 1))) / sqrt(M_PI * dim);
    }
    double pdf(double z) const {
        const double x = z * z / d;  // log1p keeps (1 - x)^e accurate for large d
        return x >= 1.0 ? 0.0 : scale * exp(e * log1p(-x));
    }
    // integral over [a, b] of z * pdf(z): scale * d / (d - 1) * [(1 - z^2/d)^(e + 1)] from b to a
    double first(double a, double b) const {
        auto g = [&](double z) {
            const double x = z * z / d;
            return x >= 1.0 ? 0.0 : exp((e + 1.0) * log1p(-x));
        };
        return scale * d / (d - 1.0) * (g(a) - g(b));
    }
    // integrals over [a, b] of z^p * pdf(z), p = 0 and 2
    void masses(double a, double b, double &m0, double &m2) const {
        static const double x16[8] = {0.0950125098376374, 0.2816035507792589, 0.4580167776572274,
                                      0.6178762444026438, 0.7554044083550030, 0.8656312023878318,
                                      0.9445750230732326, 0.9894009349916499};
        static const double w16[8] = {0.1894506104550685, 0.1826034150449236, 0.1691565193950025,
                                      0.1495959888165767, 0.1246289712555339, 0.0951585116824928,
                                      0.0622535239386479, 0.0271524594117541};
        m0 = m2 = 0.0;
        const int panels = 16;
        const double h = (b - a) / panels;
        for (int pnl = 0; pnl < panels; ++pnl) {
            const double mid = a + (pnl + 0.5) * h, half = 0.5 * h;
            for (int k = 0; k < 8; ++k)
                for (int sgn = -1; sgn <= 1; sgn += 2) {
                    const double z = mid + sgn * half * x16[k], f = pdf(z) * w16[k] * half;
                    m0 += f;
                    m2 += f * z * z;
                }
        }
    }
};
}  // namespace

extern "C" int tq_make_codebook_sphere(int bits, int d, float *centroids, float *thresholds, double *mse_out) {
    if (bits < 1 || bits > 4 || d < 3 || d > (1 << 24) || !centroids || !thresholds) return TQ_ERR_ARG;
    const SphereMarginal sm(d);
    const int L = 1 << bits, H = L / 2;
    // the outer cell ends at sqrt(d), or at 40 when sqrt(d) is larger: the density there is
    // below exp(-z^2 (d - 3) / (2 d)) <= exp(-200) for d >= 4, so the quadrature panels stay
    // where the mass is
    const double top = fmin(sqrt((double)d), 40.0);
    double c[8], t[9];
    for (int k = 0; k < H; ++k) c[k] = fmin(3.0, top) * (k + 0.5) / H;  // start: even grid
    t[0] = 0.0;
    for (int iter = 0; iter < 200000; ++iter) {
        for (int k = 1; k < H; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
        t[H] = top;
        double change = 0.0;
        for (int k = 0; k < H; ++k) {
            double m0, m2;
            sm.masses(t[k], t[k + 1], m0, m2);
            const double nc = sm.first(t[k], t[k + 1]) / m0;
            change = fmax(change, fabs(nc - c[k]));
            c[k] = nc;
        }
        if (change < 1e-13) break;  // far below float resolution
    }
    for (int k = 1; k < H; ++k) t[k] = 0.5 * (c[k - 1] + c[k]);
    t[H] = top;
    double mse = 0.0;
    for (int k = 0; k < H; ++k) {
        double m0, m2;
        sm.masses(t[k], t[k + 1], m0, m2);
        mse += 2.0 * (m2 - 2.0 * c[k] * sm.first(t[k], t[k + 1]) + c[k] * c[k] * m0);
    }
    for (int k = 0; k < H; ++k) {
        centroids[H + k] = (float)c[k];
        centroids[H - 1 - k] = -(float)c[k];
    }
    for (int k = 0; k < H; ++k) {
        const float tk = (float)t[k];
        thresholds[H - 1 + k] = tk;
        if (k > 0) thresholds[H - 1 - k] = -tk;
    }
    if (mse_out) *mse_out = mse;
    return TQ_OK;
}

// ----------------------------------------------------------------------------------------
// Randomised Walsh-Hadamard rotation: R = H_d diag(s) / sqrt(d) with H_d the Sylvester
// Hadamard matrix (entry (j, k) = (-1)^popcount(j & k)) and s_k = sign(signs[k]); d a power
// of two. An orthogonal rotation that a fast transform applies in O(d log d) (tistory series
// part 11, on community GPU implementations: structured Walsh-Hadamard rotations are being
// tried to speed up the rotation).
// ----------------------------------------------------------------------------------------
extern "C" int tq_make_rotation_hadamard(int d, const float *signs, float *rot) {
    if (d <= 0 || d > 4096 || (d & (d - 1)) || !signs || !rot) return TQ_ERR_ARG;
    const float inv = (float)(1.0 / sqrt((double)d));
    for (int k = 0; k < d; ++k)
        if (!(signs[k] != 0.0f)) return TQ_ERR_ARG;  // zero or NaN: no sign
    for (int j = 0; j < d; ++j)
        for (int k = 0; k < d; ++k) {
            const bool neg = (__builtin_popcount((unsigned)(j & k)) & 1) != (signs[k] < 0.0f);
            rot[(size_t)j * d + k] = neg ? -inv : inv;
        }
    return TQ_OK;
}

// ----------------------------------------------------------------------------------------
// Random orthogonal rotation: modified Gram-Schmidt (applied twice per column) on the
// columns of the Gaussian matrix. The resulting triangular factor has a positive
// diagonal by construction, which fixes the column signs: this is the unique
// sign-fixed Q factor of `gauss` (turboquant-pytorch write-up, stage 1).
// ----------------------------------------------------------------------------------------
extern "C" int tq_make_rotation(int d, const float *gauss, float *rot) {
    if (d <= 0 || d > 4096 || !gauss || !rot) return TQ_ERR_ARG;
    std::vector<double> Q((size_t)d * d);  // column-major: column j at Q[j*d]
    for (int j = 0; j < d; ++j) {
        double *v = &Q[(size_t)j * d];
        for (int i = 0; i < d; ++i) v[i] = gauss[(size_t)i * d + j];
        const double n0 = sqrt([&] { double s = 0; for (int i = 0; i < d; ++i) s += v[i] * v[i]; return s; }());
        for (int pass = 0; pass < 2; ++pass)
            for (int k = 0; k < j; ++k) {
                const double *u = &Q[(size_t)k * d];
                double r = 0.0;
                for (int i = 0; i < d; ++i) r += u[i] * v[i];
                for (int i = 0; i < d; ++i) v[i] -= r * u[i];
            }
        double nv = 0.0;
        for (int i = 0; i < d; ++i) nv += v[i] * v[i];
        nv = sqrt(nv);
        if (!(nv > 1e-10 * (n0 > 0 ? n0 : 1.0))) return TQ_ERR_ARG;  // rank-deficient
        for (int i = 0; i < d; ++i) v[i] /= nv;
    }
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) rot[(size_t)i * d + j] = (float)Q[(size_t)j * d + i];
    return TQ_OK;
}

// ----------------------------------------------------------------------------------------
// argument checks and geometry
// ----------------------------------------------------------------------------------------
static inline bool misaligned16(const void *ptr) { return ((uintptr_t)ptr & 15) != 0; }

// The scorers, top-k and attention read bank arrays with 16-byte loads.
static inline bool bank_misaligned(const tq_bank *b) {
    return misaligned16(b->bits) || misaligned16(b->norms) || misaligned16(b->rnorms);
}

static int check_params(const tq_params *p) {
    if (!p) return TQ_ERR_ARG;
    if (p->n_groups < 1 || p->n_groups > 2) return TQ_ERR_ARG;
    int sum = 0;
    for (int g = 0; g < p->n_groups; ++g) {
        if (p->group_dim[g] <= 0 || p->group_dim[g] % 32) return TQ_ERR_ARG;
        if (p->group_bits[g] < 1 || p->group_bits[g] > 3) return TQ_ERR_ARG;
        sum += p->group_dim[g];
        const int L = 1 << p->group_bits[g];
        for (int i = 0; i < L; ++i) {
            if (!isfinite(p->centroids[g][i])) return TQ_ERR_ARG;
            if (p->centroids[g][L - 1 - i] != -p->centroids[g][i]) return TQ_ERR_UNSUPPORTED;  // symmetric only
            if (i + 1 < L && !(p->centroids[g][i] < p->centroids[g][i + 1])) return TQ_ERR_ARG;
        }
        for (int i = 0; i + 1 < L; ++i)
            if (!(p->centroids[g][i] <= p->thresholds[g][i] && p->thresholds[g][i] <= p->centroids[g][i + 1]))
                return TQ_ERR_ARG;
    }
    if (sum != p->d || p->d > 1024) return TQ_ERR_ARG;
    // m = 0: codes and norms only (the MSE-only quantiser, e.g. for stored values)
    if (p->m != 0 && (p->m < 32 || p->m > 1024 || p->m % 32)) return TQ_ERR_ARG;
    if (!p->rot || (p->m > 0 && !p->proj)) return TQ_ERR_ARG;
    if (misaligned16(p->rot) || misaligned16(p->proj)) return TQ_ERR_ARG;  // read as 16-byte rows
    if (p->norm_dtype != TQ_F32 && p->norm_dtype != TQ_F16) return TQ_ERR_ARG;
    return TQ_OK;
}

static bool half_norms(const tq_params *p) { return p->norm_dtype == TQ_F16; }

static int words_per_key(const tq_params *p) {
    int w = p->m / 32;
    for (int g = 0; g < p->n_groups; ++g) w += p->group_bits[g] * p->group_dim[g] / 32;
    return w;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

extern "C" int tq_bank_layout(const tq_params *p, int64_t n, int64_t *wpk, int64_t *n_pad, int64_t *bpk) {
    const int rc = check_params(p);
    if (rc) return rc;
    if (n < 0) return TQ_ERR_ARG;
    const int W = words_per_key(p);
    if (wpk) *wpk = W;
    if (n_pad) *n_pad = 16 * ((n + 15) / 16);
    if (bpk) *bpk = 4 * (int64_t)W + (half_norms(p) ? 2 : 4) * ((int64_t)p->n_groups + 1);
    return TQ_OK;
}

// ----------------------------------------------------------------------------------------
// layout dispatch: the scorer is compiled for these (groups, dims, bits, m)
// ----------------------------------------------------------------------------------------
#define TQ_LAYOUTS(X)            \
    X(1, 128, 1, 0, 0, 128)      \
    X(1, 128, 2, 0, 0, 128)      \
    X(1, 128, 3, 0, 0, 128)      \
    X(1, 64, 1, 0, 0, 64)        \
    X(1, 64, 2, 0, 0, 64)        \
    X(1, 256, 1, 0, 0, 256)      \
    X(1, 256, 2, 0, 0, 256)      \
    X(1, 256, 3, 0, 0, 256)      \
    X(1, 768, 1, 0, 0, 768)      \
    X(1, 768, 2, 0, 0, 768)      \
    X(1, 768, 3, 0, 0, 768)      \
    X(2, 32, 2, 96, 1, 128)

static bool layout_is(const tq_params *p, int ng, int d0, int b0, int d1, int b1, int m) {
    if (p->n_groups != ng || p->m != m || p->group_dim[0] != d0 || p->group_bits[0] != b0) return false;
    if (ng > 1 && (p->group_dim[1] != d1 || p->group_bits[1] != b1)) return false;
    return true;
}

// Calls f(Layout{}) for the matching layout; returns TQ_ERR_UNSUPPORTED if none.
template <class F>
static int with_layout(const tq_params *p, F &&f) {
#define TQ_TRY(ng, d0, b0, d1, b1, m) \
    if (layout_is(p, ng, d0, b0, d1, b1, m)) return f(Layout<ng, d0, b0, d1, b1, m>{});
    TQ_LAYOUTS(TQ_TRY)
#undef TQ_TRY
    return TQ_ERR_UNSUPPORTED;
}

// As with_layout, for the kernels that read a bank's norms: the layout as stored, wrapped
// in HalfNorms for the 16-bit norm format.
template <class F>
static int with_bank_layout(const tq_params *p, F &&f) {
    const bool h = half_norms(p);
    return with_layout(p, [&](auto l) -> int {
        if (h) return f(HalfNorms<decltype(l)>{});
        return f(l);
    });
}

// query-operand workspace: frags [banks][Gpad/4][NF][64][16 B], consts [banks][Gpad][NCLS][2] f64
struct PrepPlan {
    int Gpad, NF, NCLS;
    size_t frag_bytes, const_off, total;
};
static PrepPlan prep_plan(int NF, int NCLS, int64_t banks, int32_t G) {
    PrepPlan pl;
    pl.Gpad = 4 * ((G + 3) / 4);
    pl.NF = NF;
    pl.NCLS = NCLS;
    pl.frag_bytes = (size_t)banks * (pl.Gpad / 4) * NF * 1024;
    pl.const_off = align256(pl.frag_bytes);
    pl.total = pl.const_off + align256((size_t)banks * pl.Gpad * NCLS * 16);
    return pl;
}

// Encoder workspace: S' (fp32) always; for d or m above 128 also the bf16 pieces of R_g and
// S', one residual chunk and the per-tile |u|^2 partial sums.
struct EncWs {
    size_t sp, r3[2], s3, U, rho, total;
    int J;  // partial-sum slots per key row
};
static bool enc_large(const tq_params *p) { return p->d > ENCS_DMAX || p->m > ENCS_DMAX; }
static EncWs enc_ws_layout(const tq_params *p, int64_t banks, int64_t n) {
    EncWs w;
    memset(&w, 0, sizeof(w));
    size_t off = align256((size_t)p->m * p->d * 4);
    if (enc_large(p)) {
        for (int g = 0; g < p->n_groups; ++g) {
            w.r3[g] = off;
            off += align256((size_t)3 * p->group_dim[g] * p->group_dim[g] * 2);
            w.J += 2 * ((p->group_dim[g] + EG_TILE - 1) / EG_TILE);
        }
        w.s3 = off;
        off += align256((size_t)3 * p->m * p->d * 2);
        const int64_t rows = banks * 16 * ((n + 15) / 16);
        const int64_t urows = std::min<int64_t>(EG_CHUNK, (rows + EG_TILE - 1) / EG_TILE * EG_TILE);
        w.U = off;
        off += align256((size_t)urows * p->d * 4);
        w.rho = off;
        off += align256((size_t)w.J * EG_CHUNK * 4);
    }
    w.total = off;
    return w;
}

// LDS-operand scorer / top-k: row tiles per work-group, query blocks, key chunks
struct LdsPlan {
    int qblocks, kchunks, chunk_tiles;
    int64_t grid;
};
template <class L>
static LdsPlan lds_plan(int64_t banks, int64_t n, int Gpad) {
    LdsPlan pl;
    constexpr int RQ = lds_rows<L>();
    pl.qblocks = (Gpad / 4 + RQ - 1) / RQ;
    const int64_t n_tiles = (n + 15) / 16;
    // about 1024 work-groups (one per compute unit at a time, four rounds), each wave
    // keeping at least a few tiles
    int64_t kc = (1024 + banks * pl.qblocks - 1) / (banks * pl.qblocks);
    int64_t max_kc = n_tiles / (4 * LDS_WAVES);
    if (max_kc < 1) max_kc = 1;
    if (kc > max_kc) kc = max_kc;
    if (kc < 1) kc = 1;
    // a chunk's bit words within a 32-bit byte range (the streamed kernel reads them through
    // one buffer resource per work-group)
    const int64_t min_kc = (n_tiles * L::W * 64 + INT32_MAX - 1) / INT32_MAX;
    if (kc < min_kc) kc = min_kc;
    pl.chunk_tiles = (int)((n_tiles + kc - 1) / kc);
    pl.kchunks = (int)((n_tiles + pl.chunk_tiles - 1) / pl.chunk_tiles);
    pl.grid = banks * pl.kchunks * pl.qblocks;
    return pl;
}

// top-k partial lists: [banks][G][kchunks * LDS_WAVES][k] values, then indices
static size_t topk_part_bytes(int64_t banks, int32_t G, int kchunks, int32_t k) {
    return align256((size_t)banks * G * kchunks * LDS_WAVES * k * 4);
}

// attention workspace: logits [banks][G][n] | scorer workspace | chunk partials
// [banks][G][chunks][2 + AT_DMAX]
struct AttnWs {
    size_t score_off, score_bytes, part_off, total;
};
static AttnWs attn_ws_layout(size_t score_bytes, int64_t banks, int64_t n, int32_t G) {
    AttnWs w;
    w.score_off = align256((size_t)banks * G * n * 4);
    w.score_bytes = score_bytes;
    w.part_off = w.score_off + align256(score_bytes);
    const int64_t chunks = (n + AT_CHUNK - 1) / AT_CHUNK;
    w.total = w.part_off + align256((size_t)banks * G * chunks * (2 + AT_DMAX) * 4);
    return w;
}

extern "C" size_t tq_workspace_bytes(int op, const tq_params *p, int64_t banks, int64_t n, int32_t G, int32_t k) {
    if (check_params(p) || banks < 0 || n < 0) return 0;
    if (op == TQ_OP_ENCODE) return enc_ws_layout(p, banks, n).total;
    if (G < 1) return 0;
    if (op == TQ_OP_ATTEND) {
        if (p->m == 0 || n < 1) return 0;
        const size_t sb = tq_workspace_bytes(TQ_OP_SCORE, p, banks, n, G, 0);
        return sb ? attn_ws_layout(sb, banks, n, G).total : 0;
    }
    size_t out = 0;
    const int rc = with_layout(p, [&](auto l) {
        using L = decltype(l);
        out = prep_plan(L::NF, L::NCLS, banks, G).total;
        return TQ_OK;
    });
    if (rc) return 0;
    if (op == TQ_OP_SCORE) return out;
    if (op == TQ_OP_TOPK) {
        if (k < 1 || k > 64) return 0;
        size_t part = 0;
        with_layout(p, [&](auto l) {
            using L = decltype(l);
            const LdsPlan lp = lds_plan<L>(banks, n, 4 * ((G + 3) / 4));
            part = 2 * topk_part_bytes(banks, G, lp.kchunks, k);
            return TQ_OK;
        });
        return out + part;
    }
    return 0;
}

static int launch_status() { return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE; }

static EncArgs enc_args(const tq_params *p) {
    EncArgs a;
    memset(&a, 0, sizeof(a));
    a.d = p->d;
    a.m = p->m;
    a.ng = p->n_groups;
    int off = 0, word = 0;
    for (int g = 0; g < p->n_groups; ++g) {
        a.gdim[g] = p->group_dim[g];
        a.gbits[g] = p->group_bits[g];
        a.goff[g] = off;
        a.gword[g] = word;
        off += p->group_dim[g];
        word += p->group_bits[g] * p->group_dim[g] / 32;
        for (int i = 0; i < 16; ++i) a.cent[g][i] = p->centroids[g][i];
        for (int i = 0; i < 15; ++i) a.thr[g][i] = p->thresholds[g][i];
        a.sqrt_d[g] = sqrt((double)p->group_dim[g]);
    }
    a.sword = word;
    a.W = word + p->m / 32;
    a.nh = half_norms(p) ? 1 : 0;
    return a;
}

// The persistent encoder's instance for these parameters: compiled for two channel groups,
// or for one group of a fixed codebook width; for d = m = 128 (the KV-cache head size) also
// for that size, and for 3-bit value banks (d = 128, m = 0).
template <typename KT>
static decltype(&encode_split_kernel<KT, 2>) split_encoder(const tq_params *p) {
    const bool d128 = p->d == 128 && p->m == 128;
    if (p->n_groups == 2) return d128 ? &encode_split_kernel<KT, 2, 0, 128> : &encode_split_kernel<KT, 2>;
    if (d128) {
        switch (p->group_bits[0]) {
            case 1: return &encode_split_kernel<KT, 1, 1, 128>;
            case 2: return &encode_split_kernel<KT, 1, 2, 128>;
            default: return &encode_split_kernel<KT, 1, 3, 128>;
        }
    }
    if (p->d == 128 && p->m == 0 && p->group_bits[0] == 3)  // 3-bit MSE-only value banks
        return &encode_split_kernel<KT, 1, 3, 128, 0>;
    switch (p->group_bits[0]) {
        case 1: return &encode_split_kernel<KT, 1, 1>;
        case 2: return &encode_split_kernel<KT, 1, 2>;
        default: return &encode_split_kernel<KT, 1, 3>;
    }
}

static void launch_prep_proj(const tq_params *p, const EncArgs &a, float *sp, hipStream_t st) {
    if (p->m == 0) return;  // no sketch, no S'
    const int bx = p->d <= 64 ? 64 : (p->d <= 128 ? 128 : 256);
    hipLaunchKernelGGL(enc_prep_proj_kernel, dim3((unsigned)((p->d + bx - 1) / bx), (unsigned)p->m), dim3(bx), 0, st,
                       p->proj, p->rot, p->group_chan, a, sp);
}

extern "C" int tq_encode(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t n, const tq_bank *out,
                         void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (banks < 0 || n < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_ARG;
    if (banks == 0 || n == 0) return TQ_OK;
    if (!keys || !out || !out->bits || !out->norms || !out->rnorms) return TQ_ERR_ARG;
    const EncWs ew = enc_ws_layout(p, banks, n);
    if (ew.total && (!workspace || ws_bytes < ew.total || ((uintptr_t)workspace & 255))) return TQ_ERR_WORKSPACE;
    if (p->m == 0 && enc_large(p)) return TQ_ERR_UNSUPPORTED;  // MSE-only keys up to 128 dimensions
    const int64_t n_tiles = (n + 15) / 16;
    if (banks * n_tiles > INT32_MAX) return TQ_ERR_UNSUPPORTED;
    // d, m <= 128 with aligned words: the persistent bf16-split encoder
    const bool split = p->d <= ENCS_DMAX && p->m <= ENCS_DMAX && ((uintptr_t)out->bits % 16) == 0 &&
                       ((uintptr_t)keys % (dtype == TQ_F32 ? 16 : 8)) == 0;
    hipStream_t st = (hipStream_t)stream;
    const EncArgs a = enc_args(p);
    float *sp = (float *)workspace;
    const long tot = (long)p->m * p->d;
    launch_prep_proj(p, a, sp, st);
    if ((rc = launch_status())) return rc;
    if (split) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const int64_t total = banks * n_tiles;
        const dim3 pgrid((unsigned)std::min<int64_t>(total, std::max(cus, 1)));
        if (dtype == TQ_F32)
            hipLaunchKernelGGL(split_encoder<float>(p), pgrid, dim3(ENCS_WAVES * 64), 0, st, (const float *)keys,
                               (long)n, (int)n_tiles, (int)total, p->rot, sp, p->group_chan, a, out->bits, out->norms,
                               out->rnorms, EncSlots{nullptr, 0});
        else
            hipLaunchKernelGGL(split_encoder<uint16_t>(p), pgrid, dim3(ENCS_WAVES * 64), 0, st,
                               (const uint16_t *)keys, (long)n, (int)n_tiles, (int)total, p->rot, sp, p->group_chan,
                               a, out->bits, out->norms, out->rnorms, EncSlots{nullptr, 0});
        return launch_status();
    }
    // larger keys with 16-byte aligned rows: the two-GEMM encoder, chunk by chunk
    if (enc_large(p) && ((uintptr_t)keys % 16) == 0) {
        char *ws = (char *)workspace;
        for (int g = 0, goff = 0; g < p->n_groups; goff += p->group_dim[g] * p->group_dim[g], ++g) {
            const long cnt = (long)p->group_dim[g] * p->group_dim[g];
            hipLaunchKernelGGL(enc_split3_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st,
                               p->rot + goff, cnt, (uint16_t *)(ws + ew.r3[g]));
        }
        hipLaunchKernelGGL(enc_split3_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, (const float *)sp,
                           tot, (uint16_t *)(ws + ew.s3));
        if ((rc = launch_status())) return rc;
        const int64_t total = banks * n_tiles;
        const bool d768 = p->n_groups == 1 && p->d == 768 && p->m == 768;  // the search geometry
        for (int64_t tc = 0; tc < total; tc += EG_CHUNK / 16) {
            const int rows = (int)std::min<int64_t>(EG_CHUNK, (total - tc) * 16);
            const int kblocks = (rows + EG_KT - 1) / EG_KT;
            int jbase = 0;
            for (int g = 0; g < p->n_groups; ++g) {
                const int ntile = (p->group_dim[g] + EG_TILE - 1) / EG_TILE;
                const dim3 grid((unsigned)(kblocks * ntile));
                const uint16_t *r3 = (const uint16_t *)(ws + ew.r3[g]);
                if (dtype == TQ_F32)
                    hipLaunchKernelGGL((d768 ? enc_gemm_rot_kernel<float, 768> : enc_gemm_rot_kernel<float, 0>), grid,
                                       dim3(EG_THREADS), 0, st, (const float *)keys, p->group_chan, r3, a, g, (long)tc,
                                       rows, (int)n_tiles, (long)n, jbase, (float *)(ws + ew.U),
                                       (float *)(ws + ew.rho), out->bits, out->norms);
                else
                    hipLaunchKernelGGL((enc_gemm_rot_kernel<uint16_t, 0>), grid, dim3(EG_THREADS), 0, st,
                                       (const uint16_t *)keys, p->group_chan, r3, a, g, (long)tc, rows, (int)n_tiles,
                                       (long)n, jbase, (float *)(ws + ew.U), (float *)(ws + ew.rho), out->bits,
                                       out->norms);
                jbase += 2 * ntile;
            }
            const dim3 pgrid((unsigned)(kblocks * ((p->m + EG_TILE - 1) / EG_TILE)));
            hipLaunchKernelGGL((d768 ? enc_gemm_prj_kernel<768> : enc_gemm_prj_kernel<0>), pgrid, dim3(EG_THREADS), 0,
                               st, (const float *)(ws + ew.U), (const uint16_t *)(ws + ew.s3), a, (long)tc, rows,
                               ew.J, (const float *)(ws + ew.rho), out->bits, out->rnorms);
            if ((rc = launch_status())) return rc;
        }
        return TQ_OK;
    }
    const size_t smem = enc_smem_bytes(p->d, p->m);
    if (smem > 150 * 1024) return TQ_ERR_UNSUPPORTED;
    const dim3 grid((unsigned)(banks * n_tiles));
    if (dtype == TQ_F32) {
        (void)hipFuncSetAttribute((const void *)encode_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(encode_kernel<float>, grid, dim3(256), smem, st, (const float *)keys, (long)n, (int)n_tiles,
                           p->rot, sp, p->group_chan, a, out->bits, out->norms, out->rnorms,
                           EncSlots{nullptr, 0});
    } else {
        (void)hipFuncSetAttribute((const void *)encode_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(encode_kernel<uint16_t>, grid, dim3(256), smem, st, (const uint16_t *)keys, (long)n,
                           (int)n_tiles, p->rot, sp, p->group_chan, a, out->bits, out->norms,
                           out->rnorms, EncSlots{nullptr, 0});
    }
    return launch_status();
}

// Argument checks shared by the two append entry points (nothing is enqueued).
static int check_append(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                        const int32_t *pos, int64_t n_cap, const tq_bank *out) {
    int rc = check_params(p);
    if (rc) return rc;
    if (banks < 0 || count < 0 || n_cap < 0 || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_ARG;
    if (banks == 0 || count == 0 || n_cap == 0) return TQ_OK;
    if (!keys || !pos || !out || !out->bits || !out->norms || !out->rnorms) return TQ_ERR_ARG;
    const int64_t n_tiles = (count + 15) / 16, cap_tiles = (n_cap + 15) / 16;
    if (banks * n_tiles > INT32_MAX || cap_tiles > INT32_MAX) return TQ_ERR_UNSUPPORTED;
    if (enc_smem_bytes(p->d, p->m) > 150 * 1024) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

// The launches of an append, arguments already checked: the S' fold into sp (when fold),
// then the encoder placing each key in its slot.
static int launch_append(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                         const int32_t *pos, int64_t n_cap, const tq_bank *out, bool fold, float *sp, hipStream_t st) {
    int rc;
    const int64_t n_tiles = (count + 15) / 16, cap_tiles = (n_cap + 15) / 16;
    const size_t smem = enc_smem_bytes(p->d, p->m);
    const bool split = p->d <= ENCS_DMAX && p->m <= ENCS_DMAX && ((uintptr_t)keys % (dtype == TQ_F32 ? 16 : 8)) == 0;
    const EncArgs a = enc_args(p);
    if (fold) {
        launch_prep_proj(p, a, sp, st);
        if ((rc = launch_status())) return rc;
    }
    const EncSlots slots{pos, (int)cap_tiles};
    if (split) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        const int64_t total = banks * n_tiles;
        const dim3 pgrid((unsigned)std::min<int64_t>(total, std::max(cus, 1)));
        if (dtype == TQ_F32)
            hipLaunchKernelGGL(split_encoder<float>(p), pgrid, dim3(ENCS_WAVES * 64), 0, st, (const float *)keys,
                               (long)count, (int)n_tiles, (int)total, p->rot, sp, p->group_chan, a, out->bits,
                               out->norms, out->rnorms, slots);
        else
            hipLaunchKernelGGL(split_encoder<uint16_t>(p), pgrid, dim3(ENCS_WAVES * 64), 0, st,
                               (const uint16_t *)keys, (long)count, (int)n_tiles, (int)total, p->rot, sp,
                               p->group_chan, a, out->bits, out->norms, out->rnorms, slots);
        return launch_status();
    }
    const dim3 grid((unsigned)(banks * n_tiles));
    if (dtype == TQ_F32) {
        (void)hipFuncSetAttribute((const void *)encode_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(encode_kernel<float>, grid, dim3(256), smem, st, (const float *)keys, (long)count,
                           (int)n_tiles, p->rot, sp, p->group_chan, a, out->bits, out->norms,
                           out->rnorms, slots);
    } else {
        (void)hipFuncSetAttribute((const void *)encode_kernel<uint16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(encode_kernel<uint16_t>, grid, dim3(256), smem, st, (const uint16_t *)keys, (long)count,
                           (int)n_tiles, p->rot, sp, p->group_chan, a, out->bits, out->norms,
                           out->rnorms, slots);
    }
    return launch_status();
}

extern "C" int tq_encode_append(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                                const int32_t *pos, int64_t n_cap, const tq_bank *out, int flags, void *workspace,
                                size_t ws_bytes, void *stream) {
    int rc = check_append(p, keys, dtype, banks, count, pos, n_cap, out);
    if (rc) return rc;
    if (flags & ~TQ_APPEND_PREPARED) return TQ_ERR_ARG;
    if (banks == 0 || count == 0 || n_cap == 0) return TQ_OK;
    const size_t ws_need = enc_ws_layout(p, banks, count).total;
    if (ws_need && (!workspace || ws_bytes < ws_need || ((uintptr_t)workspace & 255))) return TQ_ERR_WORKSPACE;
    return launch_append(p, keys, dtype, banks, count, pos, n_cap, out, !(flags & TQ_APPEND_PREPARED),
                         (float *)workspace, (hipStream_t)stream);
}

// ----------------------------------------------------------------------------------------
// Append without allocation: the folded projection S' (m x d floats) lives in a file-scope
// device array instead of a caller workspace. Each device holds its own copy of the array;
// its device address is looked up once per device (the host-side name is only a handle
// for that lookup and is never passed to a kernel).
// ----------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

static constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex scratch_mu;
static void *scratch_ptr[SCRATCH_MAX_DEVICES];

// The current device's address of `scratch`, or nullptr if the lookup fails.
static void *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

extern "C" int tq_encode_append_noalloc(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                                        const int32_t *pos, int64_t n_cap, const tq_bank *out, void *stream) {
    int rc = check_append(p, keys, dtype, banks, count, pos, n_cap, out);
    if (rc) return rc;
    // the layouts whose only scratch is S': d, m <= 128, at most 64 KiB
    if (p->d > ENCS_DMAX || p->m > ENCS_DMAX || (size_t)p->m * p->d * 4 > TQ_NOALLOC_SCRATCH_BYTES)
        return TQ_ERR_UNSUPPORTED;
    if (banks == 0 || count == 0 || n_cap == 0) return TQ_OK;
    float *sp = (float *)scratch_on_current_device();
    if (!sp) return TQ_ERR_DEVICE;
    return launch_append(p, keys, dtype, banks, count, pos, n_cap, out, true, sp, (hipStream_t)stream);
}

static PrepArgs prep_args(const tq_params *p) {
    PrepArgs pa;
    memset(&pa, 0, sizeof(pa));
    for (int g = 0; g < p->n_groups; ++g) {
        const int b = p->group_bits[g], L = 1 << b;
        double total = 0.0;
        for (int s = 0; s < walsh_planes(b); ++s) {
            const int mask = walsh_mask(b, s);
            double acc = 0.0;
            for (int idx = 0; idx < L; ++idx) {
                double chi = 1.0;
                for (int bit = 0; bit < b; ++bit)
                    if (mask & (1 << bit)) chi *= ((idx >> bit) & 1) ? 1.0 : -1.0;
                acc += (double)p->centroids[g][idx] * chi;
            }
            const double chat = acc / L;
            pa.walsh[g][s] = 2.0 * chat;
            total += chat;
        }
        pa.cmax[g] = total;
    }
    return pa;
}

extern "C" int tq_prepare_queries(const tq_params *p, const float *q, int64_t banks, int32_t G, void *workspace,
                                  size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (p->m == 0) return TQ_ERR_UNSUPPORTED;  // the estimator needs the sign sketch
    if (banks < 0 || G < 1) return TQ_ERR_ARG;
    if (banks == 0) return TQ_OK;
    if (!q) return TQ_ERR_ARG;
    return with_layout(p, [&](auto l) {
        using L = decltype(l);
        const PrepPlan pl = prep_plan(L::NF, L::NCLS, banks, G);
        if (!workspace || ws_bytes < pl.total || ((uintptr_t)workspace & 255)) return (int)TQ_ERR_WORKSPACE;
        if (banks * pl.Gpad > INT32_MAX) return (int)TQ_ERR_UNSUPPORTED;
        int8_t *frags = (int8_t *)workspace;
        double *consts = (double *)((char *)workspace + pl.const_off);
        hipLaunchKernelGGL(qprep_kernel<L>, dim3((unsigned)(banks * pl.Gpad / 4)), dim3(1024), 0, (hipStream_t)stream, q,
                           p->rot, p->proj, p->group_chan, prep_args(p), (int)G, pl.Gpad, frags, consts);
        return launch_status();
    });
}

static ScoreScale score_scale(const tq_params *p) {
    ScoreScale s;
    s.inv_sqrt_d[0] = 1.0 / sqrt((double)p->group_dim[0]);
    s.inv_sqrt_d[1] = p->n_groups > 1 ? 1.0 / sqrt((double)p->group_dim[1]) : 0.0;
    s.qjl = sqrt(M_PI / 2.0) / (double)p->m;
    return s;
}

// tiles per batch in the scorer: fewer when more registers hold operands
template <class L, int RT>
constexpr int score_tb() {
    return (RT == 1 && L::NG == 1) ? 4 : (RT <= 2 ? 2 : 1);
}

// the decode scorers keep RT x NF operand fragments (4 VGPRs each) in registers
template <class L, int RT>
constexpr bool vgpr_operands_fit() {
    return RT * L::NF <= 40;
}

template <class L, int RT>
static int launch_score(const tq_bank *in, int64_t banks, int64_t n, int32_t G, const PrepPlan &pl, const void *ws,
                        float *scores, const ScoreScale &sc, hipStream_t st) {
    if constexpr (!vgpr_operands_fit<L, RT>()) {
        return TQ_ERR_UNSUPPORTED;
    } else {
    const int64_t n_tiles = (n + 15) / 16;
    const int64_t target_waves = 256 * 16;
    int64_t tpw = (banks * n_tiles + target_waves - 1) / target_waves;
    if (tpw < 1) tpw = 1;
    const int64_t wpb = (n_tiles + tpw - 1) / tpw;
    const int64_t waves = banks * wpb;
    if ((waves + 3) / 4 > INT32_MAX) return TQ_ERR_UNSUPPORTED;
    const int8_t *frags = (const int8_t *)ws;
    const double *consts = (const double *)((const char *)ws + pl.const_off);
    hipLaunchKernelGGL((score_kernel<L, RT, score_tb<L, RT>()>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                       in->bits, (const typename L::NormT *)in->norms, (const typename L::NormT *)in->rnorms, frags, consts, scores, (int)banks, (long)n, (int)n_tiles, (int)G,
                       pl.Gpad, (int)tpw, (int)wpb, sc);
    return launch_status();
    }
}

// Fused query preparation + scoring (one launch). Work-groups of 16 waves, about one per
// compute unit, each owning a contiguous range of one bank's tiles.
template <class L, int RT>
static constexpr bool fused_fits() {
    // LDS for the prologue, and operand registers within the per-wave budget of the
    // work-group size (16 waves: 128 VGPRs; 8 waves: 256)
    return sizeof(FusedLds<L, RT>) <= 160 * 1024 && (RT == 1 ? L::NF <= 10 : RT * L::NF <= 24);
}

template <class L, int RT>
static int launch_fused(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G,
                        float *scores, hipStream_t st) {
    if constexpr (!fused_fits<L, RT>()) {
        return TQ_ERR_UNSUPPORTED;
    } else {
        const int64_t n_tiles = (n + 15) / 16;
        int64_t wpb = (256 + banks - 1) / banks;                // aim at one work-group per compute unit
        constexpr int WAVES = fused_waves<RT>();
        const int64_t max_wpb = (n_tiles + WAVES - 1) / WAVES;  // at least a tile per wave
        if (wpb > max_wpb) wpb = max_wpb;
        if (wpb < 1) wpb = 1;
        const int64_t tpw = (n_tiles + wpb - 1) / wpb;
        wpb = (n_tiles + tpw - 1) / tpw;
        if (banks * wpb > INT32_MAX) return TQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL((score_fused_kernel<L, RT, score_tb<L, RT>()>), dim3((unsigned)(banks * wpb)),
                           dim3(WAVES * 64), 0, st, in->bits, (const typename L::NormT *)in->norms, (const typename L::NormT *)in->rnorms, q, p->rot, p->proj,
                           p->group_chan, prep_args(p), scores, (int)banks, (long)n, (int)n_tiles, (int)G, (int)wpb,
                           (int)tpw, score_scale(p));
        return launch_status();
    }
}

// Ring-staged fused scorer (G <= 4): needs a ring of at least 4 tiles per wave next to the
// prologue's LDS, and the operand registers of one row tile.
template <class L>
static constexpr bool ring_fits() {
    return ring_slots<L>() >= 4 && L::NF <= 10 && RingTile<L>::LOADS * (ring_slots<L>() - 1) <= 63;
}

template <class L>
static int launch_ring(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G,
                       float *scores, hipStream_t st) {
    if constexpr (!ring_fits<L>()) {
        return TQ_ERR_UNSUPPORTED;
    } else {
        const int64_t n_tiles = (n + 15) / 16;
        int64_t wpb = (256 + banks - 1) / banks;  // aim at one work-group per compute unit
        const int64_t max_wpb = (n_tiles + RING_WAVES - 1) / RING_WAVES;
        if (wpb > max_wpb) wpb = max_wpb;
        if (wpb < 1) wpb = 1;
        const int64_t tpw = (n_tiles + wpb - 1) / wpb;
        wpb = (n_tiles + tpw - 1) / tpw;
        if (banks * wpb > INT32_MAX || 4 * n > INT32_MAX) return TQ_ERR_UNSUPPORTED;
        hipLaunchKernelGGL((score_ring_kernel<L, ring_slots<L>()>), dim3((unsigned)(banks * wpb)),
                           dim3(RING_WAVES * 64), 0, st, in->bits, (const typename L::NormT *)in->norms, (const typename L::NormT *)in->rnorms, q, p->rot, p->proj,
                           p->group_chan, prep_args(p), scores, (int)banks, (long)n, (int)n_tiles, (int)G, (int)wpb,
                           (int)tpw, score_scale(p));
        return launch_status();
    }
}

// Scorer / top-k with the prepared operands staged in LDS (any G, any layout whose
// operands of one row tile fit). TOPK: partial lists into part_v / part_i.
template <class L, bool TOPK>
static int launch_lds(const tq_bank *in, int64_t banks, int64_t n, int32_t G, const PrepPlan &pp, const void *ws,
                      float *scores, int32_t k, float *part_v, int *part_i, const ScoreScale &sc, hipStream_t st) {
    if constexpr (!lds_fits<L>()) {
        return TQ_ERR_UNSUPPORTED;
    } else {
        const LdsPlan lp = lds_plan<L>(banks, n, pp.Gpad);
        if (lp.grid > INT32_MAX || (int64_t)G * n > ((int64_t)1 << 62)) return TQ_ERR_UNSUPPORTED;
        const int8_t *frags = (const int8_t *)ws;
        const double *consts = (const double *)((const char *)ws + pp.const_off);
        hipLaunchKernelGGL((score_lds_kernel<L, lds_rows<L>(), TOPK>), dim3((unsigned)lp.grid), dim3(LDS_WAVES * 64),
                           0, st, in->bits, (const typename L::NormT *)in->norms, (const typename L::NormT *)in->rnorms, frags, consts, (long)n, (int)((n + 15) / 16), (int)G,
                           pp.Gpad, lp.qblocks, lp.kchunks, lp.chunk_tiles, sc, scores, (int)k, part_v, part_i);
        return launch_status();
    }
}

extern "C" int tq_score_prepared(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, int32_t G,
                                 const void *workspace, float *scores, void *stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (p->m == 0) return TQ_ERR_UNSUPPORTED;  // the estimator needs the sign sketch
    if (banks < 0 || n < 0 || G < 1) return TQ_ERR_ARG;
    if (banks == 0 || n == 0) return TQ_OK;
    if (!in || !in->bits || !in->norms || !in->rnorms || !scores || bank_misaligned(in)) return TQ_ERR_ARG;
    if (!workspace || ((uintptr_t)workspace & 255)) return TQ_ERR_WORKSPACE;
    const ScoreScale sc = score_scale(p);
    return with_bank_layout(p, [&](auto l) {
        using L = decltype(l);
        const PrepPlan pl = prep_plan(L::NF, L::NCLS, banks, G);
        hipStream_t st = (hipStream_t)stream;
        int r = TQ_ERR_UNSUPPORTED;
        switch (pl.Gpad / 4) {
            case 1: r = launch_score<L, 1>(in, banks, n, G, pl, workspace, scores, sc, st); break;
            case 2: r = launch_score<L, 2>(in, banks, n, G, pl, workspace, scores, sc, st); break;
            case 3: r = launch_score<L, 3>(in, banks, n, G, pl, workspace, scores, sc, st); break;
            case 4: r = launch_score<L, 4>(in, banks, n, G, pl, workspace, scores, sc, st); break;
            default: break;
        }
        if (r != TQ_ERR_UNSUPPORTED) return r;
        // many queries, or operands too large for registers: operands in LDS
        return launch_lds<L, false>(in, banks, n, G, pl, workspace, scores, 0, nullptr, nullptr, sc, st);
    });
}

extern "C" int tq_score(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G,
                        float *scores, void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (p->m == 0) return TQ_ERR_UNSUPPORTED;  // the estimator needs the sign sketch
    if (banks < 0 || n < 0 || G < 1) return TQ_ERR_ARG;
    if (banks == 0 || n == 0) return TQ_OK;
    if (!in || !in->bits || !in->norms || !in->rnorms || !scores || !q || bank_misaligned(in)) return TQ_ERR_ARG;
    hipStream_t st = (hipStream_t)stream;
    rc = G > 16 ? (int)TQ_ERR_UNSUPPORTED : with_bank_layout(p, [&](auto l) {
        using L = decltype(l);
        switch ((G + 3) / 4) {
            case 1: {
                // four queries per bank: the ring-staged scorer where it fits
                const int r = G == 4 ? launch_ring<L>(p, in, banks, n, q, G, scores, st) : TQ_ERR_UNSUPPORTED;
                return r != TQ_ERR_UNSUPPORTED ? r : launch_fused<L, 1>(p, in, banks, n, q, G, scores, st);
            }
            case 2: return launch_fused<L, 2>(p, in, banks, n, q, G, scores, st);
            case 3: return launch_fused<L, 3>(p, in, banks, n, q, G, scores, st);
            default: return launch_fused<L, 4>(p, in, banks, n, q, G, scores, st);
        }
    });
    if (rc != TQ_ERR_UNSUPPORTED) return rc;
    // many queries, or layouts too large for the fused prologue: prepare into the
    // workspace, then score
    if ((rc = tq_prepare_queries(p, q, banks, G, workspace, ws_bytes, stream))) return rc;
    return tq_score_prepared(p, in, banks, n, G, workspace, scores, stream);
}

extern "C" int tq_topk(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G,
                       int32_t k, float *vals, int32_t *idx, void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(p);
    if (rc) return rc;
    if (p->m == 0) return TQ_ERR_UNSUPPORTED;  // the estimator needs the sign sketch
    if (banks < 0 || n < 0 || G < 1 || k < 1 || k > 64 || k > n) return TQ_ERR_ARG;
    if (banks == 0) return TQ_OK;
    if (n > INT32_MAX) return TQ_ERR_UNSUPPORTED;  // key indices are returned as int32
    if (!in || !in->bits || !in->norms || !in->rnorms || !q || !vals || !idx || bank_misaligned(in)) return TQ_ERR_ARG;
    if (!workspace || ((uintptr_t)workspace & 255)) return TQ_ERR_WORKSPACE;
    if (ws_bytes < tq_workspace_bytes(TQ_OP_TOPK, p, banks, n, G, k)) return TQ_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const ScoreScale sc = score_scale(p);
    return with_bank_layout(p, [&](auto l) {
        using L = decltype(l);
        if constexpr (!lds_fits<L>()) {
            return (int)TQ_ERR_UNSUPPORTED;
        } else {
            const PrepPlan pp = prep_plan(L::NF, L::NCLS, banks, G);
            const LdsPlan lp = lds_plan<L>(banks, n, pp.Gpad);
            if (banks * G > INT32_MAX / 2) return (int)TQ_ERR_UNSUPPORTED;
            const size_t pb = topk_part_bytes(banks, G, lp.kchunks, k);
            float *part_v = (float *)((char *)workspace + pp.total);
            int *part_i = (int *)((char *)workspace + pp.total + pb);
            int r = tq_prepare_queries(p, q, banks, G, workspace, ws_bytes, stream);
            if (r) return r;
            if ((r = launch_lds<L, true>(in, banks, n, G, pp, workspace, nullptr, k, part_v, part_i, sc, st))) return r;
            const int64_t queries = banks * G;
            hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)((queries + 3) / 4)), dim3(256), 0, st, part_v, part_i,
                               (long)queries, lp.kchunks * LDS_WAVES, (int)k, vals, (int *)idx);
            return launch_status();
        }
    });
}

// ----------------------------------------------------------------------------------------
// decompression and decode attention
// ----------------------------------------------------------------------------------------
static DecArgs dec_args(const tq_params *p) {
    DecArgs a;
    memset(&a, 0, sizeof(a));
    a.d = p->d;
    a.ng = p->n_groups;
    a.W = words_per_key(p);
    int off = 0, word = 0;
    for (int g = 0; g < p->n_groups; ++g) {
        a.gdim[g] = p->group_dim[g];
        a.gbits[g] = p->group_bits[g];
        a.goff[g] = off;
        a.gword[g] = word;
        off += p->group_dim[g];
        word += p->group_bits[g] * p->group_dim[g] / 32;
        for (int i = 0; i < (1 << p->group_bits[g]); ++i) a.cent[g][i] = p->centroids[g][i];
        a.inv_sqrt_d[g] = (float)(1.0 / sqrt((double)p->group_dim[g]));
    }
    a.nh = half_norms(p) ? 1 : 0;
    return a;
}

extern "C" int tq_decode(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, float *out, void *stream) {
    const int rc = check_params(p);
    if (rc) return rc;
    if (banks < 0 || n < 0) return TQ_ERR_ARG;
    if (banks == 0 || n == 0) return TQ_OK;
    if (!in || !in->bits || !in->norms || !out) return TQ_ERR_ARG;
    if (misaligned16(in->bits) || misaligned16(in->norms)) return TQ_ERR_ARG;
    const int64_t n_tiles = (n + 15) / 16;
    if (banks * n_tiles > INT32_MAX) return TQ_ERR_UNSUPPORTED;
    const DecArgs a = dec_args(p);
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)(banks * n_tiles)), dim3(256), (size_t)16 * p->d * 4,
                       (hipStream_t)stream, in->bits, in->norms, (long)n, (int)n_tiles, p->rot, p->group_chan, a, out);
    return launch_status();
}

// Walsh coefficients a_P of a symmetric codebook in the bit-plane basis the attention kernel
// uses (planes: bit 0, bit 1, bit 2, and the xor of the three for 3 bits):
// c[idx] = sum_P a_P s_P(idx), s_P = +-1. False if the codebook is not reproduced.
static bool attn_args(const tq_params *p, AttnArgs *a) {
    memset(a, 0, sizeof(*a));
    a->d = p->d;
    a->ng = p->n_groups;
    a->W = words_per_key(p);
    int off = 0, word = 0;
    for (int g = 0; g < p->n_groups; ++g) {
        const int b = p->group_bits[g], L = 1 << b;
        a->gdim[g] = p->group_dim[g];
        a->gbits[g] = b;
        a->goff[g] = off;
        a->gword[g] = word;
        off += p->group_dim[g];
        word += b * p->group_dim[g] / 32;
        a->inv_sqrt_d[g] = 1.0 / sqrt((double)p->group_dim[g]);
        auto sgn = [&](int P, int idx) -> double {
            if (P < 3) return ((idx >> P) & 1) ? 1.0 : -1.0;
            return (((idx ^ (idx >> 1) ^ (idx >> 2)) & 1) ? 1.0 : -1.0);  // s0 s1 s2 = 2 (b0^b1^b2) - 1
        };
        const int planes = b == 3 ? 4 : b;
        double al[4] = {0.0, 0.0, 0.0, 0.0};
        for (int P = 0; P < planes; ++P)
            for (int idx = 0; idx < L; ++idx) al[P] += (double)p->centroids[g][idx] * sgn(P, idx) / L;
        for (int idx = 0; idx < L; ++idx) {
            double r = 0.0;
            for (int P = 0; P < planes; ++P) r += al[P] * sgn(P, idx);
            const double c = p->centroids[g][idx];
            if (fabs(r - c) > 1e-6 * (1.0 + fabs(c))) return false;
        }
        for (int P = 0; P < planes; ++P) {
            a->coef[g][P] = 2.0 * al[P];
            a->bias[g] += al[P];
        }
    }
    return true;
}

extern "C" int tq_attend(const tq_params *kp, const tq_bank *keys, const tq_params *vp, const tq_bank *values,
                         int64_t banks, int64_t n, const int32_t *lengths, const float *q, int32_t G, float scale,
                         float *out, void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_params(kp);
    if (rc) return rc;
    if ((rc = check_params(vp))) return rc;
    if (kp->m == 0) return TQ_ERR_UNSUPPORTED;  // the logits come from the estimator
    if (banks < 0 || n < 1 || G < 1 || !isfinite(scale)) return TQ_ERR_ARG;
    if (vp->d > AT_DMAX) return TQ_ERR_UNSUPPORTED;
    if (banks == 0) return TQ_OK;
    if (!keys || !keys->bits || !keys->norms || !keys->rnorms || !values || !values->bits || !values->norms || !q ||
        !out)
        return TQ_ERR_ARG;
    if (bank_misaligned(keys) || misaligned16(values->bits) || misaligned16(values->norms)) return TQ_ERR_ARG;
    if (!workspace || ((uintptr_t)workspace & 255)) return TQ_ERR_WORKSPACE;
    const size_t need = tq_workspace_bytes(TQ_OP_ATTEND, kp, banks, n, G, 0);
    if (!need) return TQ_ERR_UNSUPPORTED;
    if (ws_bytes < need) return TQ_ERR_WORKSPACE;
    const int64_t chunks = (n + AT_CHUNK - 1) / AT_CHUNK;
    if (banks * chunks > INT32_MAX || banks * G > INT32_MAX || (G + 3) / 4 > 65535) return TQ_ERR_UNSUPPORTED;
    AttnArgs a;
    if (!attn_args(vp, &a)) return TQ_ERR_UNSUPPORTED;
    const AttnWs w = attn_ws_layout(tq_workspace_bytes(TQ_OP_SCORE, kp, banks, n, G, 0), banks, n, G);
    float *logits = (float *)workspace;
    float *part = (float *)((char *)workspace + w.part_off);
    if ((rc = tq_score(kp, keys, banks, n, q, G, logits, (char *)workspace + w.score_off, w.score_bytes, stream)))
        return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t n_tiles = (n + 15) / 16;
    const dim3 grid((unsigned)(banks * chunks), (unsigned)((G + 3) / 4));
    auto chunk_kernel = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(AT_THREADS), 0, st, logits, values->bits, (const void *)values->norms,
                           (long)n, (int)n_tiles, (int)G, (int)chunks, scale, lengths, a, part);
    };
    const bool nh = half_norms(vp);
    if (vp->n_groups == 2)
        nh ? chunk_kernel(attn_chunk_kernel<2, true, 0>) : chunk_kernel(attn_chunk_kernel<2, false, 0>);
    else if (vp->group_bits[0] == 3)
        nh ? chunk_kernel(attn_chunk_kernel<1, true, 3>) : chunk_kernel(attn_chunk_kernel<1, false, 3>);
    else
        nh ? chunk_kernel(attn_chunk_kernel<1, true, 0>) : chunk_kernel(attn_chunk_kernel<1, false, 0>);
    if ((rc = launch_status())) return rc;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(banks * G)), dim3(AT_MERGE_WAVES * 64), 0, st, part,
                       (int)chunks, vp->rot,
                       vp->group_chan, a, out);
    return launch_status();
}

extern "C" int tq_fp32_logits(const float *keys, int64_t banks, int64_t n, int32_t d, const float *q, int32_t G,
                              float *scores, void *stream) {
    if (banks < 0 || n < 0 || d <= 0 || d % 4 || G < 1) return TQ_ERR_ARG;
    if (banks == 0 || n == 0) return TQ_OK;
    if (!keys || !q || !scores) return TQ_ERR_ARG;
    if (d > 256 || G > 32) return TQ_ERR_UNSUPPORTED;
    return launch_fp32_logits(keys, banks, n, d, q, G, scores, (hipStream_t)stream) ? TQ_ERR_DEVICE : TQ_OK;
}

extern "C" int tq_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes == 0) return TQ_OK;
    if (!src || !dst || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) || (bytes & 15)) return TQ_ERR_ARG;
    return launch_copy(src, dst, bytes, (hipStream_t)stream) ? TQ_ERR_DEVICE : TQ_OK;
}

extern "C" const char *tq_status_string(int status) {
    switch (status) {
        case TQ_OK: return "ok";
        case TQ_ERR_ARG: return "invalid argument";
        case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case TQ_ERR_DEVICE: return "device launch failed";
        case TQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}
