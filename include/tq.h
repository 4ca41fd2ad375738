/*
 * tq.h -- C ABI of the TurboQuant KV-cache library (libtq.so), MI355X / gfx950.
 *
 * The method (pages cited by site and section):
 *  - Encode [admirer.cn memory-wall article, section 2, stage one]: each key or
 *    value vector is rotated by one seeded Haar-random orthogonal matrix, its
 *    length is stored, and every rotated coordinate is quantized by a pure
 *    threshold lookup into a Lloyd-Max codebook precomputed for the known law
 *    of a rotated unit vector's coordinates -- no scale, no zero point.
 *  - Keys add [same article, stage two; intelliparadigm "3-bit" article,
 *    section 2.1.2] a 1-bit QJL sketch z = [S r > 0] of the quantization
 *    residual r, with S an m x d Gaussian matrix, so that the inner product
 *    estimate becomes unbiased.
 *  - Decode [cc-newplayer explainer, technical breakdown items 2 and 4]: the
 *    query stays uncompressed; it is rotated once, scored against the packed
 *    codes plus the QJL correction, softmax-ed, and the dequantized values are
 *    summed in the rotated domain and rotated back once.
 *
 * Conventions shared by every call:
 *  - d = head_dim, b' = mse_bits (bits per rotated coordinate), L = 2^b',
 *    m = qjl_dim (0 for values and for MSE-only keys).
 *  - Rotation: y = Pi x (Pi row-major d x d).  QJL: p = S r (S row-major m x d).
 *  - Packed codes: code j of a vector occupies bits [j*b', (j+1)*b') of the
 *    vector's bit stream, least significant bit first; stream bit k is bit
 *    k%32 of little-endian uint32 word k/32.  A vector has d*b'/32 code words.
 *    With split widths (tq_codebook_build_split) code j starts at bit
 *    sum_{i<j} width_i instead: the first w coordinates are b'+1 bits wide,
 *    and a vector has (d*b' + w)/32 code words.
 *    Sign bit i (= [p_i > 0]) is stream bit i of the vector's m/32 sign words.
 *  - Cache layout (structure of arrays, all device memory, row-major):
 *      codes[B][H_kv][t_cap][d*b'/32]  uint32
 *      signs[B][H_kv][t_cap][m/32]     uint32   (keys with m > 0 only)
 *      norms[B][H_kv][t_cap]           float    nu = ||x||
 *      res_norms[B][H_kv][t_cap]       float    gamma = ||r|| (keys, m > 0)
 *    Row index of (b, h, t) is (b*H_kv + h)*t_cap + t.
 *  - `stream` is a hipStream_t of the codebook's device (NULL = its default
 *    stream).  Encode and decode only enqueue work: they return before the GPU
 *    finishes, and a device fault shows up at the caller's next synchronization.
 *  - Ownership: the caller owns every buffer passed in; the library owns only
 *    the codebook handle (host tables + one device table buffer).  Encode and
 *    decode allocate nothing.
 *  - Errors: every argument is validated on the host before any HIP call; a
 *    failed check returns a negative status and enqueues nothing.
 *    tq_last_error() returns a message for the calling thread's last failure.
 *  - Thread safety: all calls are reentrant; a codebook is immutable after
 *    build and may be shared by threads and streams.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment or combination      */
  TQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. d != 128 on GPU) */
  TQ_ERR_ALLOC = -3,       /* host or device allocation failed (build only)    */
  TQ_ERR_DEVICE = -4       /* a HIP call or kernel launch failed               */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

typedef struct tq_codebook tq_codebook; /* opaque */

/* Build the setup tables once [memory-wall article §2 stage one: the codebooks
 * are computed ahead of time and stored; inference only looks them up].
 *   head_dim   d >= 2 (host-only mode); the GPU path supports d == 128.
 *   mse_bits   b' in 1..4.
 *   qjl_dim    m: 0 (no QJL) or a multiple of 32; the GPU path supports 0 or 128.
 *   rot_seed   seed of the Haar rotation's Gaussian matrix.
 *   qjl_seed   seed of S (ignored when m == 0).
 *   device     HIP device ordinal, or -1 for a host-only handle (export works,
 *              encode/decode return TQ_ERR_INVALID_ARG).
 *   out        receives the handle; free it with tq_codebook_free.
 * Tables: Lloyd-Max centroids of the density f_d(t) ~ (1-t^2)^((d-3)/2) on
 * [-1,1] (symmetric; Lloyd iteration in double until no centroid moves by
 * 1e-15) rounded to
 * fp32, thresholds = fp32 of the midpoints; Pi = Q diag(sign(diag R)) of the
 * Householder QR of a d x d Gaussian matrix; S = m x d Gaussian.  Gaussians
 * come from SplitMix64 (state = seed) turned into Box-Muller pairs (cos first),
 * filled row-major; see DESIGN notes in the source for the exact definition. */
tq_status tq_codebook_build(int32_t head_dim, int32_t mse_bits, int32_t qjl_dim,
                            uint64_t rot_seed, uint64_t qjl_seed, int32_t device,
                            tq_codebook **out);

/* Split bit widths [cc-newplayer explainer, technical breakdown item 1: an
 * average of about 2.5 bits per element; intelliparadigm "3-bit" article,
 * §2.1 (a 2.5-bit intermediate) and §5.1 (3.5 bits)]: the pages give
 * fractional averages without their construction; here rotated coordinates
 * 0 .. wide_coords - 1 take the (mse_bits + 1)-bit Lloyd-Max codebook of f_d
 * and the others the mse_bits-bit one, for mse_bits + wide_coords/d bits per
 * coordinate (keys add their 1-bit sketch).  Every rotated coordinate follows
 * f_d, so the expected distortion is the coordinate-weighted mean of the two
 * widths' distortions whichever coordinates are wide.
 *   mse_bits      b' in 1..3 when wide_coords > 0.
 *   wide_coords   0 (a uniform codebook, as tq_codebook_build) .. d; the GPU
 *                 path supports 0 and 64 (else TQ_ERR_UNSUPPORTED).
 * Other arguments as in tq_codebook_build; Pi and S are the same for the same
 * seeds.  Records pack the codes at running offsets (see the top).  On the
 * GPU a split codebook encodes (tq_encode_kv, tq_append_decode) and is read by
 * the single-query matrix-core decode: tq_decode_attention(_static),
 * tq_append_decode and tq_attention_logits with t_cap a multiple of 4 and
 * 16-byte aligned norm arrays, the key and value codebooks both split; other
 * reads (chunks of several queries, other t_cap) return TQ_ERR_UNSUPPORTED. */
tq_status tq_codebook_build_split(int32_t head_dim, int32_t mse_bits, int32_t wide_coords, int32_t qjl_dim,
                                  uint64_t rot_seed, uint64_t qjl_seed, int32_t device, tq_codebook **out);

/* wide_coords and the wide width (mse_bits + 1, or 0 for a uniform codebook);
 * either pointer may be NULL. */
tq_status tq_codebook_split_info(const tq_codebook *cb, int32_t *wide_coords, int32_t *wide_bits);

/* The wide codebook's fp32 centroids[2L] and thresholds[2L-1] (host pointers,
 * either may be NULL); TQ_ERR_INVALID_ARG for a uniform codebook.
 * tq_codebook_export gives the b'-bit codebook of the other coordinates. */
tq_status tq_codebook_export_wide(const tq_codebook *cb, float *centroids, float *thresholds);

/* Release a handle (NULL is accepted).  The caller must make sure no enqueued
 * work still uses it. */
tq_status tq_codebook_free(tq_codebook *cb);

/* Parameters of a handle; any output pointer may be NULL. */
tq_status tq_codebook_info(const tq_codebook *cb, int32_t *head_dim, int32_t *mse_bits,
                           int32_t *qjl_dim, int32_t *device);

/* Copy the host tables out (host pointers; any may be NULL):
 * centroids[L], thresholds[L-1], rotation[d*d] (row-major, y = Pi x),
 * qjl[m*d] (row-major; must be NULL when m == 0). */
tq_status tq_codebook_export(const tq_codebook *cb, float *centroids, float *thresholds,
                             float *rotation, float *qjl);

/* Same tables in float64 (the values before rounding to fp32). */
tq_status tq_codebook_export_f64(const tq_codebook *cb, double *centroids, double *thresholds,
                                 double *rotation, double *qjl);

/* Words per cache row: code_words = (d*b' + wide_coords)/32 rounded up,
 * sign_words = m/32 (either may be NULL). */
tq_status tq_record_words(const tq_codebook *cb, int32_t *code_words, int32_t *sign_words);

/* Encode n vectors online into cache rows [memory-wall article §2: stage one
 * for all vectors, stage two for keys (m > 0)].
 *   x             device, n rows of d elements of x_dtype, row r at x + r*x_row_stride
 *                 elements (x_row_stride >= d; 16-byte aligned rows).
 *   dst_row       device int64[n] giving the cache row of input row i, or NULL
 *                 for row i -> cache row i.  Rows whose destination lies outside
 *                 [0, cache_rows) are skipped (nothing written).
 *   cache_rows    number of rows the output arrays hold (>= n when dst_row == NULL).
 *   codes         device uint32[cache_rows][code_words] (tq_record_words).
 *   signs         device uint32[cache_rows][m/32]; NULL iff m == 0.
 *   norms         device float[cache_rows]: nu = ||x||.
 *   res_norms     device float[cache_rows]: gamma = ||y - c[idx]||; NULL iff m == 0.
 *   dbg_rot       NULL, or device float[n][d]: the rotated unit vector y = Pi x/nu
 *                 exactly as quantized (indexed by input row).
 *   dbg_proj      NULL, or device float[n][m]: p = S r exactly as signed (m > 0).
 * Per vector: nu = ||x||; y = Pi x / nu (y = 0 when nu == 0); code_j =
 * #{i : y_j >= t_i} (NaN -> 0); keys: r = y - c[code], gamma = ||r||,
 * sign_i = [ (S r)_i > 0 ].  With split widths coordinate j uses its own
 * width's thresholds and centroids.  Pure function of (x, codebook): re-running it on
 * the same rows is idempotent.  n == 0 is a no-op. */
tq_status tq_encode_kv(const tq_codebook *cb, const void *x, tq_dtype x_dtype, int64_t n,
                       int64_t x_row_stride, const int64_t *dst_row, int64_t cache_rows,
                       uint32_t *codes, uint32_t *signs, float *norms, float *res_norms,
                       float *dbg_rot, float *dbg_proj, void *stream);

/* One compressed cache tensor set, laid out as described at the top. */
typedef struct {
  const uint32_t *codes;
  const uint32_t *signs;     /* keys with m > 0, else NULL */
  const float *norms;
  const float *res_norms;    /* keys with m > 0, else NULL */
  int64_t t_cap;             /* tokens per (batch, kv head) row block */
} tq_cache;

/* Bytes of device workspace tq_decode_attention needs for these sizes. */
tq_status tq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int64_t t_cap, size_t *bytes);

/* Single-query decode attention over the compressed cache [cc-newplayer
 * explainer item 4: Q uncompressed, attention with dequantization].
 *   kcb, vcb      key codebook (its Pi, S, centroids) and value codebook
 *                 (vcb->m must be 0); both on the same device, same d.
 *   q             device [batch][n_q_heads][d] of q_dtype (contiguous).
 *   k, v          host structs holding device pointers; k->t_cap == v->t_cap.
 *   seq_len       device int32[batch]: tokens to attend per sequence; values are
 *                 clamped to [0, t_cap].
 *   n_q_heads     n_kv_heads times 1, 2, 4 or 8 (else TQ_ERR_UNSUPPORTED); q head h
 *                 reads kv head h / (H_q/H_kv).
 *   softmax_scale <= 0 selects 1/sqrt(d).
 *   out           device [batch][n_q_heads][d] of out_dtype; a sequence with
 *                 seq_len 0 gets zeros.  bf16 output is the round-to-nearest-even
 *                 of the fp32 result.
 *   dbg_scores    NULL or device float[batch][n_q_heads][t_cap]: the scaled
 *                 logits l_t for t < seq_len (other entries untouched).
 *   workspace     device scratch of at least tq_decode_workspace_bytes bytes,
 *                 256-byte aligned; its contents on entry do not matter.  Calls
 *                 that share a workspace must not overlap in time.
 * Score: l_t = scale * nu_t * ( <Pi q, c_k[code_t]> + sqrt(pi/2)/m * gamma_t *
 * <S Pi q, 2 z_t - 1> ); output o = Pi_v^T sum_t softmax(l)_t nu^v_t c_v[code^v_t].
 * Deterministic: the same inputs give bitwise-identical outputs. */
tq_status tq_decode_attention(const tq_codebook *kcb, const tq_codebook *vcb, const void *q,
                              tq_dtype q_dtype, const tq_cache *k, const tq_cache *v,
                              const int32_t *seq_len, int32_t batch, int32_t n_q_heads,
                              int32_t n_kv_heads, float softmax_scale, void *out,
                              tq_dtype out_dtype, float *dbg_scores, void *workspace,
                              size_t workspace_bytes, void *stream);

/* tq_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch is a static device array of
 * 16 MiB inside the library, one copy per GPU, held until the process ends;
 * this call itself calls no hipMalloc, hipFree or other allocating routine.
 * Arguments, results and errors are those of tq_decode_attention (same kernels,
 * bitwise the same output), except that sizes whose workspace
 * (tq_decode_workspace_bytes) exceeds 16 MiB return TQ_ERR_INVALID_ARG and
 * launch nothing.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and must be
 * serialized by the caller.  The scratch's contents on entry do not matter. */
tq_status tq_decode_attention_static(const tq_codebook *kcb, const tq_codebook *vcb, const void *q,
                                     tq_dtype q_dtype, const tq_cache *k, const tq_cache *v,
                                     const int32_t *seq_len, int32_t batch, int32_t n_q_heads,
                                     int32_t n_kv_heads, float softmax_scale, void *out, tq_dtype out_dtype,
                                     float *dbg_scores, void *stream);

/* Attention of a chunk of n_new new tokens' queries over the compressed cache
 * (chunked prefill, or several decode tokens verified at once), each query
 * causal: query j of sequence b sits at position p = seq_len[b] - n_new + j
 * and attends over cached positions 0 .. p [admirer.cn memory-wall article,
 * section 1: every new token attends over the keys and values of all tokens
 * before it; section 2: the attention runs on the compressed cache].  The new
 * tokens' own K and V must already be in the cache (tq_encode_kv).
 *   q             device [batch][n_q_heads][n_new][d] of q_dtype (contiguous).
 *   seq_len       device int32[batch]: cached tokens including the n_new new
 *                 ones; query j attends over clamp(seq_len[b] - n_new + j + 1,
 *                 0, t_cap) tokens (zero output when that is 0).
 *   n_new         >= 1, with n_new * n_kv_heads <= 65535, batch <= 65535 and
 *                 batch * n_q_heads * n_new <= 2^24 (else TQ_ERR_INVALID_ARG).
 *   out           device [batch][n_q_heads][n_new][d] of out_dtype.
 *   workspace     at least tq_chunk_workspace_bytes bytes for the same sizes,
 *                 256-byte aligned; calls that share it must not overlap in time.
 * Other arguments as in tq_decode_attention.
 * With n_new * (n_q_heads / n_kv_heads) < 16 the queries run through the
 * decode kernel: n_new = 1 equals tq_decode_attention bit for bit, and query
 * j equals tq_decode_attention of that query alone with seq_len[b] - n_new +
 * j + 1 tokens up to the order of the split sums (bitwise when both launches
 * pick the same token-chunk length).  From 16 query rows per kv head on, the
 * matrix cores compute the query rotation with fp16 hi/lo operands (22
 * significant bits) and the scores and the value sum with bf16 hi/lo operand
 * splits (two or three products per fp32 product, about 2^-16 relative error
 * per product); the outputs agree with the single-query path to about 1e-4
 * (max-abs over unit-scale outputs). */
tq_status tq_chunk_attention(const tq_codebook *kcb, const tq_codebook *vcb, const void *q, tq_dtype q_dtype,
                             const tq_cache *k, const tq_cache *v, const int32_t *seq_len, int32_t batch,
                             int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new, float softmax_scale, void *out,
                             tq_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace tq_chunk_attention needs for these sizes. */
tq_status tq_chunk_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t n_new,
                                   int64_t t_cap, size_t *bytes);

/* One step of a decode loop, enqueued on `stream` with no host synchronization
 * (so a caller can capture it in a graph and replay it): the new key and value
 * of every (b, kv head) are appended to the caches, the queries attend over
 * the grown cache, and seq_len grows by one [admirer.cn memory-wall article,
 * section 1: each generated token appends its K and V and attends over all of
 * them; intelliparadigm "3-bit" article, section 3.2: the cache is written
 * sequentially and read at attention].
 *   k_new, v_new  device [batch][n_kv_heads][d] of kv_dtype (contiguous); row
 *                 (b, h) is encoded into cache row (b*n_kv_heads + h)*t_cap +
 *                 seq_len[b] of k and v (keys with kcb, values with vcb).
 *   seq_len       device int32[batch], read and then advanced on the device:
 *                 a sequence with 0 <= seq_len[b] < t_cap gets the new token
 *                 and seq_len[b] + 1; one at t_cap (full) attends over its t_cap
 *                 tokens and is neither written nor advanced.
 *   k, v          the caches, written at the appended rows (the const in
 *                 tq_cache does not apply here).
 * Other arguments as in tq_decode_attention (no dbg_scores).  Results equal
 * tq_encode_kv of the new rows into those rows followed by tq_decode_attention
 * with seq_len + 1, bit for bit. */
tq_status tq_append_decode(const tq_codebook *kcb, const tq_codebook *vcb, const void *k_new, const void *v_new,
                           tq_dtype kv_dtype, const void *q, tq_dtype q_dtype, const tq_cache *k, const tq_cache *v,
                           int32_t *seq_len, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                           float softmax_scale, void *out, tq_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Scaled attention logits of every cached token, without the softmax and the
 * value sum: the key phase of tq_decode_attention on its own [admirer.cn
 * memory-wall article, section 2: the attention logits computed from the
 * compressed key cache, the operation the pages time against a JAX baseline
 * at each bit width; intelliparadigm "3-bit" article, section 2.1.2: inner
 * products estimated from the codes and the QJL signs].
 *   kcb           key codebook (its Pi, S, centroids), on a GPU device.
 *   q             device [batch][n_q_heads][d] of q_dtype (contiguous).
 *   k             host struct holding device pointers to the key cache.
 *   seq_len       device int32[batch]: tokens per sequence, clamped to [0, t_cap].
 *   n_q_heads     n_kv_heads times 1, 2, 4 or 8 (else TQ_ERR_UNSUPPORTED).
 *   softmax_scale <= 0 selects 1/sqrt(d).
 *   logits        device float[batch][n_q_heads][t_cap] (caller-owned):
 *                 entry t < seq_len[b] gets l_t; the others are not written.
 *   workspace     device scratch of at least tq_decode_workspace_bytes bytes for
 *                 the same sizes, 256-byte aligned; calls that share it must not
 *                 overlap in time.
 * l_t = scale * nu_t * ( <Pi q, c_k[code_t]> + sqrt(pi/2)/m * gamma_t *
 * <S Pi q, 2 z_t - 1> ), bit for bit the l_t that tq_decode_attention returns
 * in dbg_scores for the same inputs.  Errors: TQ_ERR_INVALID_ARG for NULL or
 * misaligned pointers, bad sizes or a short workspace; nothing is launched then. */
tq_status tq_attention_logits(const tq_codebook *kcb, const void *q, tq_dtype q_dtype, const tq_cache *k,
                              const int32_t *seq_len, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                              float softmax_scale, float *logits, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Static name of a status code. */
const char *tq_status_string(tq_status s);

/* Message describing the calling thread's most recent failed call ("" if none). */
const char *tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
