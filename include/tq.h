/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant packed-key library.
 *
 * The method (turboquant-pytorch write-up on discuss.pytorch.kr, section on the
 * two-stage algorithm; tambur.pub article on TurboQuant; tistory series part 11,
 * section 3 on format-aware kernels):
 *   stage 1: rotate each key with a random orthogonal matrix and quantise every
 *            rotated coordinate on its own against a Lloyd-Max codebook that is
 *            precomputed for the normal distribution the rotation produces;
 *   stage 2: project the stage-1 residual with a Gaussian matrix S and keep one
 *            sign bit per projection row (QJL), plus the residual's norm;
 *   scoring: unbiased inner-product estimates of full-precision queries against
 *            the packed keys (attention logits, vector-search scores), optionally
 *            reduced to a per-query top-k.
 *
 * Conventions for every entry point:
 *   - All pointers marked (device) are device memory owned by the caller; the
 *     library never allocates, frees or retains them. (host) pointers are host
 *     memory read or written before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Device work is
 *     enqueued asynchronously on it; argument checks run first and return a
 *     negative status with nothing enqueued.
 *   - Returns TQ_OK (0) or a negative tq_status. TQ_ERR_DEVICE reports a failed
 *     launch (the HIP error is not cleared). tq_status_string() names a code.
 *   - Results are bit-identical from run to run for identical inputs.
 *   - Calls are thread-safe. The only state the library keeps is, per device, the
 *     address of the device array used by tq_encode_append_noalloc (looked up once).
 *   - Non-finite inputs give unspecified (but memory-safe) results.
 *   - The matrices (rot, proj) and the bank arrays read by the scorers, top-k, decode and
 *     attention are read with 16-byte loads: their pointers must be 16-byte aligned
 *     (TQ_ERR_ARG otherwise). Allocations from hipMalloc or torch are.
 *
 * Packed bank format (one "bank" = the keys of one (layer, batch, kv-head), or a
 * whole search database). With W = sum_g b_g*d_g/32 + m/32 words per key and
 * n_pad = 16*ceil(n/16):
 *   bits   (uint32) [banks][n_pad/16][W][16]: element [b][t][w][i] is word w of key
 *          16*t+i. Word order inside a key: for each channel group g, for each
 *          codebook bit-plane p < b_g, d_g/32 words (word k, bit t = bit p of the
 *          bucket index of rotated coordinate 32k+t of group g); then m/32 sign
 *          words (word k, bit t = [row 32k+t of S times the residual >= 0]).
 *   norms  [banks][n_pad][n_groups]: |x_g| per group.
 *   rnorms [banks][n_pad]: |residual| (0 for the MSE-only quantiser, m = 0).
 *   Both norm arrays hold float32 values, or with tq_params.norm_dtype == TQ_F16 the
 *   IEEE binary16 roundings of those float32 values (2 bytes each: the format variant
 *   with 16-bit norms; the stage-1 residual is then taken against the reconstruction
 *   from the rounded norm, so the sketch corrects the rounding too).
 *   Slots n..n_pad-1 hold the encoding of the zero vector.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_ERR_ARG = -1,         /* null pointer, bad size, inconsistent parameters */
    TQ_ERR_UNSUPPORTED = -2, /* a valid request the library has no kernel for */
    TQ_ERR_DEVICE = -3,      /* a HIP launch failed */
    TQ_ERR_WORKSPACE = -4    /* workspace missing or smaller than tq_workspace_bytes() */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef enum { TQ_OP_ENCODE = 0, TQ_OP_SCORE = 1, TQ_OP_TOPK = 2, TQ_OP_ATTEND = 3 } tq_op;

/* tq_encode_append flags. TQ_APPEND_PREPARED: the workspace already holds this call's
 * folded projection S' = S P_chan blockdiag(R_g)^T, written by an earlier tq_encode or
 * tq_encode_append with the same parameters into the same workspace; it is not formed again. */
enum { TQ_APPEND_PREPARED = 1 };

/* Parameters of one encoding. Dimensions and the codebooks are host values;
 * the matrices are (device) pointers read by the kernels.
 *   d            key dimension; d = group_dim[0] (+ group_dim[1])
 *   m            sign-sketch rows (QJL): a multiple of 32 in [32, 1024], or 0 for the
 *                MSE-only quantiser (codes and norms only; such banks can be decoded and
 *                attended over as values, not scored: TQ_ERR_UNSUPPORTED)
 *   n_groups     1, or 2 for a split of the channels into two groups that are
 *                rotated and quantised separately (mixed bit widths)
 *   group_dim    channels per group, multiples of 32
 *   group_bits   codebook bits per group, 1..3 (the total budget per channel is
 *                group_bits + the shared 1-bit sketch)
 *   centroids    per group, 2^bits Lloyd-Max centroids in ascending order, in
 *                unit-variance units (tq_make_codebook); must be symmetric,
 *                c[L-1-i] == -c[i]
 *   thresholds   per group, the 2^bits - 1 decision thresholds (midpoints)
 *   group_chan   (device) int32[d]: group 0's channels ascending, then group 1's;
 *                NULL = identity (required NULL when n_groups == 1)
 *   rot          (device) float32: group 0's d_0 x d_0 rotation row-major, then
 *                group 1's; rotated coordinate j of group g = row j . x_g
 *   proj         (device) float32 [m][d] row-major: S, columns in channel order (NULL
 *                when m == 0)
 *   norm_dtype   storage of the bank's norm arrays: TQ_F32 (0), or TQ_F16 for the
 *                16-bit norm format variant (turboquant-pytorch write-up, results: the
 *                compressed cache size it reports at 3 bits is met with 16-bit norms).
 *                Every encoder writes it and every reader takes it, for all layouts.
 *                Other values: TQ_ERR_ARG. */
typedef struct {
    int32_t d, m, n_groups;
    int32_t group_dim[2];
    int32_t group_bits[2];
    float centroids[2][16];
    float thresholds[2][15];
    const int32_t *group_chan;
    const float *rot;
    const float *proj;
    int32_t norm_dtype;
} tq_params;

/* (device) arrays of one or more banks, laid out as described above. */
typedef struct {
    uint32_t *bits;
    void *norms;  /* float32, or binary16 (tq_params.norm_dtype) */
    void *rnorms;
} tq_bank;

/* Lloyd-Max codebook for N(0,1) with 2^bits levels, 1 <= bits <= 4, computed on
 * the host in fp64 and rounded to float (turboquant-pytorch write-up, stage 1:
 * the codebook is precomputed for the normal distribution of the rotated
 * coordinates). centroids[2^bits], thresholds[2^bits - 1] (host); mse_out
 * (host, nullable) receives the fp64 mean squared error. Deterministic. */
int tq_make_codebook(int bits, float *centroids, float *thresholds, double *mse_out);

/* Lloyd-Max codebook, in the same z units, for the exact distribution of one coordinate
 * of a uniformly random unit vector in R^d (density proportional to (1 - z^2/d)^((d-3)/2)
 * on |z| < sqrt(d); the normal distribution is its large-d limit). 1 <= bits <= 4,
 * 3 <= d <= 2^24, else TQ_ERR_ARG. Host fp64; outputs as tq_make_codebook (symmetric). */
int tq_make_codebook_sphere(int bits, int d, float *centroids, float *thresholds, double *mse_out);

/* Randomised Walsh-Hadamard rotation (tistory series part 11, on community GPU
 * implementations: structured Walsh-Hadamard rotations are tried to speed up the rotation):
 * rot (host) receives d x d floats, entry (j, k) =
 * (-1)^popcount(j & k) * sign(signs[k]) / sqrt(d). d a power of two, at most 4096; signs
 * (host) float[d], each nonzero. TQ_ERR_ARG otherwise. The matrix is orthogonal and goes to
 * tq_params.rot like any other rotation. */
int tq_make_rotation_hadamard(int d, const float *signs, float *rot);

/* Random orthogonal rotation (same write-up, stage 1): the Q factor of a QR
 * decomposition of the d x d matrix `gauss` (host, row-major, expected i.i.d.
 * N(0,1)), with column signs fixed so that the triangular factor has a positive
 * diagonal. Host fp64 computation; rot (host) receives d x d floats row-major.
 * TQ_ERR_ARG if gauss is rank-deficient. */
int tq_make_rotation(int d, const float *gauss, float *rot);

/* Bank geometry for n keys: 32-bit words per key, n_pad, and bytes per key of the
 * three arrays together (words*4 + (n_groups + 1)*4, or *2 with 16-bit norms). Host only. */
int tq_bank_layout(const tq_params *p, int64_t n, int64_t *words_per_key, int64_t *n_pad, int64_t *bytes_per_key);

/* Device workspace bytes needed by `op` (a tq_op) for these sizes; 0 on bad
 * arguments. Pass at least this much, 256-byte aligned, to the call. An encode of an
 * MSE-only layout (m = 0) with d <= 128 needs none (workspace may then be NULL). */
size_t tq_workspace_bytes(int op, const tq_params *p, int64_t banks, int64_t n, int32_t G, int32_t k);

/* Encode (stages 1 and 2) keys (device) [banks][n][d] of dtype TQ_F32 or TQ_BF16
 * into `out` (device arrays sized by tq_bank_layout for `banks` banks). Uses
 * `workspace` (device) of tq_workspace_bytes(TQ_OP_ENCODE, ...). An MSE-only layout
 * (m = 0: stage 1 alone, e.g. stored values) is supported up to d = 128
 * (TQ_ERR_UNSUPPORTED above). */
int tq_encode(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t n, const tq_bank *out,
              void *workspace, size_t ws_bytes, void *stream);

/* Streaming append (online encoding: the quantiser is data-oblivious, so a new key is
 * encoded on its own, with nothing recomputed for the keys already stored; turboquant-pytorch
 * write-up, two-stage algorithm section). Encodes `count` new keys per bank, keys (device)
 * [banks][count][d] of dtype TQ_F32 or TQ_BF16, into slots pos[b] .. pos[b] + count - 1 of
 * bank b of `out`, whose arrays are sized by tq_bank_layout for n_cap slots per bank.
 * pos (device) int32[banks]. A key whose slot falls outside [0, n_cap_pad) (n_cap_pad =
 * 16 * ceil(n_cap / 16)) is skipped; no other slot is written. Slots are encoded as
 * tq_encode encodes them (up to the decision band of the fp32-level contractions). Uses
 * `workspace` (device) of tq_workspace_bytes(TQ_OP_ENCODE, p, banks, count, ...) bytes;
 * flags: 0 or TQ_APPEND_PREPARED (any other bit: TQ_ERR_ARG). Scoring a bank filled this way
 * uses n = n_cap: slots never written hold whatever the arrays held (tq_attend's lengths
 * restrict attention to each bank's filled prefix). TQ_ERR_UNSUPPORTED when
 * the per-tile LDS footprint (16 keys x (8 d + 2 (d + m)) bytes) exceeds 150 KiB. */
int tq_encode_append(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                     const int32_t *pos, int64_t n_cap, const tq_bank *out, int flags, void *workspace,
                     size_t ws_bytes, void *stream);

/* Streaming append for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): tq_encode_append with
 * flags = 0, except that the folded projection S' is formed in a device array the library
 * holds for the life of the process (one per device, TQ_NOALLOC_SCRATCH_BYTES) instead of in
 * a caller workspace. The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). Arguments, slots and results as tq_encode_append; layouts with
 * d > 128 or m > 128 (whose encoder needs more scratch than the array holds):
 * TQ_ERR_UNSUPPORTED. Every call on a device shares that device's array and re-forms S' in
 * it, so calls that may overlap on one device (several streams, several host threads) race
 * and must be serialised by the caller; calls in order on one stream do not. TQ_ERR_DEVICE
 * if the array's device address cannot be obtained. */
#define TQ_NOALLOC_SCRATCH_BYTES 65536
int tq_encode_append_noalloc(const tq_params *p, const void *keys, int dtype, int64_t banks, int64_t count,
                             const int32_t *pos, int64_t n_cap, const tq_bank *out, void *stream);

/* Query preparation (per query: R_g q_g and S q, once, as the estimator's
 * operands; same write-up, usage example: the query stays at full precision).
 * q (device) float32 [banks][G][d]. Writes the prepared operands into
 * `workspace` (device), of tq_workspace_bytes(TQ_OP_SCORE, ...) bytes, for
 * tq_score_prepared (tq_score and tq_topk run it themselves when they need it). */
int tq_prepare_queries(const tq_params *p, const float *q, int64_t banks, int32_t G, void *workspace,
                       size_t ws_bytes, void *stream);

/* Estimated inner products of prepared queries (any G) against packed banks:
 *   est = sum_g (nu_g / sqrt(d_g)) <R_g q_g, c_g[idx_g]>
 *       + sqrt(pi/2) / m * rho * <S q, 2*signs - 1>
 * (turboquant-pytorch write-up: stage 2 makes this estimate unbiased; usage
 * example: inner_product(query, compressed)). scores (device) float32
 * [banks][G][n]; query row g of bank b uses bank b (GQA: the caller arranges the
 * G query heads sharing a kv head as one bank's queries). */
int tq_score_prepared(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, int32_t G,
                      const void *workspace, float *scores, void *stream);

/* The same estimates from unprepared queries q (device) float32 [banks][G][d]. For up
 * to 16 queries per bank and operands that fit in registers the preparation runs inside
 * the scoring kernel (one launch) and `workspace` is not touched; otherwise this is
 * tq_prepare_queries followed by tq_score_prepared and `workspace` (device) must hold
 * tq_workspace_bytes(TQ_OP_SCORE, ...) bytes, 256-byte aligned. */
int tq_score(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G,
             float *scores, void *workspace, size_t ws_bytes, void *stream);

/* Per query, the k largest estimates (vector search over the packed database;
 * tambur.pub article, vector-search paragraph), largest first, equal estimates
 * by lower key index; the estimates are those tq_score returns (fp32), ranked as
 * fp32. vals (device) float32 [banks][G][k], idx (device) int32 [banks][G][k].
 * q (device) float32 [banks][G][d], any G >= 1. 1 <= k <= 64 and k <= n, else
 * TQ_ERR_ARG; n > INT32_MAX (indices past the int32 range): TQ_ERR_UNSUPPORTED.
 * The score rows are never written to memory: the prepared query operands and the
 * per-wave partial top-k lists live in `workspace` (device) of
 * tq_workspace_bytes(TQ_OP_TOPK, ...) bytes, 256-byte aligned (TQ_ERR_WORKSPACE
 * otherwise). TQ_ERR_UNSUPPORTED for a layout whose operands exceed 150 KiB of LDS
 * per row of four queries. */
int tq_topk(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, const float *q, int32_t G, int32_t k,
            float *vals, int32_t *idx, void *workspace, size_t ws_bytes, void *stream);

/* Decompression of the stage-1 part (turboquant-pytorch write-up, usage example: decompress;
 * the MSE quantiser's reconstruction): out (device) float32 [banks][n][d], per stored vector
 * and channel group x_hat_g = (nu_g / sqrt(d_g)) R_g^T c_g[idx_g], in channel order. The sign
 * sketch, if any, is not used. fp32 arithmetic (relative error about d_g * 2^-24). */
int tq_decode(const tq_params *p, const tq_bank *in, int64_t banks, int64_t n, float *out, void *stream);

/* Decode attention over a packed KV cache (same write-up, usage example: keys held by the
 * inner-product quantiser, values by the MSE quantiser): for bank b and query row g,
 *   out[b][g] = sum_{i < len_b} softmax_i(scale * est(q[b][g], key_i)) * x_hat(value_i),
 * est as tq_score returns it (fp32) and x_hat as tq_decode forms it. keys: banks of n slots
 * under kp (m > 0); values: banks of the same n slots under vp (any m; the sketch is ignored),
 * d_v = vp->d <= 128 (else TQ_ERR_UNSUPPORTED). lengths (device) int32[banks], nullable: bank
 * b attends over its first len_b = min(max(lengths[b], 0), n) slots (a growing cache filled
 * by tq_encode_append; slots past len_b may hold anything, NaN included); NULL = all n. A
 * bank with len_b = 0 gets out = 0. q (device) float32 [banks][G][kp->d], out (device) float32
 * [banks][G][d_v]. n >= 1, finite scale, else TQ_ERR_ARG. The logits of all n slots are formed
 * into `workspace` (device) of tq_workspace_bytes(TQ_OP_ATTEND, kp, banks, n, G, 0) bytes,
 * 256-byte aligned (TQ_ERR_WORKSPACE otherwise), then reduced per chunk of 512 slots (softmax
 * weights in 30-bit fixed point, exact integer products) and merged in fp64. */
int tq_attend(const tq_params *kp, const tq_bank *keys, const tq_params *vp, const tq_bank *values, int64_t banks,
              int64_t n, const int32_t *lengths, const float *q, int32_t G, float scale, float *out, void *workspace,
              size_t ws_bytes, void *stream);

/* Measurement kernels (not part of the method):
 * fp32 logits against unquantized keys, scores[b][g][i] = q[b][g] . keys[b][i]
 * (keys, q, scores device float32; the comparison the tambur.pub article makes
 * between 4-bit keys and 32-bit keys), and a plain device-to-device copy used to
 * calibrate the achievable HBM bandwidth and the traffic counters. */
int tq_fp32_logits(const float *keys, int64_t banks, int64_t n, int32_t d, const float *q, int32_t G, float *scores,
                   void *stream);
int tq_copy(const void *src, void *dst, size_t bytes, void *stream);

const char *tq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
