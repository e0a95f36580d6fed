/*
 * tq.h -- C ABI of libtq: a packed KV-cache codec (RoPE, randomized Hadamard rotation,
 * Lloyd-Max scalar codes, 1-bit QJL residual sketch), decode attention over the packed
 * cache and inner-product top-k search over packed vectors, for AMD MI355X (gfx950).
 *
 * Sources (page titles; the section or passage on each page):
 *   [TurboESM]   "TurboESM: Ultra-Efficient 3-Bit KV Cache Quantization for Protein
 *                Language Models with Orthogonal Rotation and QJL Correction", technical
 *                summary: 2.A RoPE before the orthogonal rotation Pi and the invariance of
 *                (Pi R_i q)^T (Pi R_j k); 2.C Lloyd-Max look-up tables; 2.D 1-bit residual
 *                correction; 2.E one fused decode pass (dequantize, correct, inverse
 *                rotation, online softmax).
 *   [TurboQuant] news summary of the TurboQuant post: "Etape 1" random rotation then a
 *                per-coordinate scalar quantizer; "Etape 2"/"QJL" sign bits of a
 *                Johnson-Lindenstrauss projection of the residual with an estimator that
 *                pairs a full-precision query with the 1-bit data; vector search section
 *                (top-k by estimated inner product, recall 1@k).
 *   [NSNQuant]   technical summary, section 2: randomized Hadamard transform.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller allocates and frees every buffer (host and device).  The
 *     library never allocates, keeps no global state and is reentrant.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Device work is
 *     enqueued asynchronously on it; buffers must stay valid until it completes.
 *   - Errors: every argument, shape and capacity check runs on the host before anything
 *     is enqueued; a failing check returns its status and enqueues nothing.  A failed
 *     kernel launch returns TQ_EDEVICE.  No C++ exception crosses this interface.
 *   - A norm too large for fp16 is stored as 65504 and sets bit 0 of the cache header's
 *     flags word (byte offset 8), which stays set until tq_cache_init.
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
  TQ_EINVAL = 1,        /* NULL pointer, negative size, inconsistent shapes */
  TQ_EUNSUPPORTED = 2,  /* valid but not implemented: d, bits or m outside the supported set */
  TQ_ECAPACITY = 3,     /* start_pos + n_new or length beyond the cache capacity */
  TQ_ENOSPACE = 4,      /* output or workspace buffer smaller than required */
  TQ_EDEVICE = 5        /* a HIP launch or runtime call failed */
} tq_status;

/* Element types of the K, V and query inputs.  Entry points take the value as an int32_t
 * (any other value is TQ_EINVAL), so a C caller's out-of-range integer is checked rather
 * than loaded as an enum. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Codec parameters.  d: vector dimension; bits_k: scalar bits of keys / database
 * vectors (1..4); bits_v: scalar bits of values (0 = keys only, else 1..4); m: QJL rows
 * (0 = no residual sketch, else a multiple of 32, at most 2048); seed: draws the rotation
 * signs D and the Gaussian projection S. */
typedef struct {
  int32_t d, bits_k, bits_v, m;
  uint64_t seed;
} tq_codec_desc;

/* Packed cache shape: `batch` x `kv_heads` units of `capacity` token slots each
 * (batch x kv_heads <= 65535 and capacity <= 2^30; a larger shape is TQ_EUNSUPPORTED and
 * tq_cache_bytes returns 0 for it).
 * nsn = 1 selects the NSN pre-transform ([NSNQuant] section 1: tokens normalized to norm
 * sqrt(d), the channel mean shifted out, normalized again) for keys and values: each
 * token v is stored as the codec of w = v - s1 o with s1 = ||v|| / sqrt(d) kept in fp16
 * and o the unit's channel mean (tq_nsn_set_means); the codec's own norm and direction
 * are NSN's second normalization.  Requires bits_v > 0 and d = 64 or 128; nsn = 0 is the
 * plain codec.
 * polar = 1 selects PolarQuant ([TurboQuant] news summary, "PolarQuant") as stage 1 in
 * place of the per-coordinate codes: the rotated vector's adjacent coordinates are turned
 * into (radius, angle) pairs, the radii paired again recursively down to one radius (the
 * norm, fp16) and d - 1 angles, each angle coded on a fixed grid (tq_make_polar_grid):
 * 4 bits for a level-1 angle, 2 bits above, 3 d - 2 bits in all; keys keep the QJL sketch
 * of their residual.  Requires d = 64 or 128, bits_k = 3, bits_v = 0 or 3, nsn = 0. */
typedef struct {
  int32_t batch, kv_heads, d, capacity, bits_k, bits_v, m;
  int32_t nsn;
  int32_t polar;
} tq_cache_desc;

typedef void *tq_stream_t; /* hipStream_t */

/* Version string of the library and of the packed format ("libtq <x.y> format 1"). */
const char *tq_version(void);

/* Human-readable name of a status code (static storage; "unknown status" for a value
 * that is not a tq_status). */
const char *tq_status_str(int32_t s);

/* Lloyd-Max codebook ([TurboQuant] "Etape 1" and the reader comment on Lloyd-Max
 * boundaries; [TurboESM] 2.C) for one coordinate of a uniformly random unit vector in
 * R^d, density proportional to (1 - x^2)^((d-3)/2) on [-1, 1], computed in fp64 on the
 * host.  The codec stores each centroid rounded to fp16; `centroids` (2^bits values,
 * ascending) receives those stored values and `bounds` (2^bits - 1 values) the exact
 * midpoints between consecutive stored centroids, which are the encoder's decision
 * boundaries.  The density is even, so the codebook is made exactly odd after the fp64
 * iteration: c[2^bits - 1 - k] = -c[k].  Supported: 8 <= d <= 4096, 1 <= bits <= 4.
 * Host only, synchronous. */
tq_status tq_make_codebook(int32_t d, int32_t bits, float *centroids, float *bounds);

/* Same computation, returning the fp64 Lloyd-Max centroids and boundaries before the
 * fp16 rounding (for checking the iteration itself). */
tq_status tq_make_codebook_f64(int32_t d, int32_t bits, double *centroids, double *bounds);

/* PolarQuant angle grid of one level in fp64.  Level 1 (an angle atan2(y_{2i+1}, y_{2i})
 * in [0, 2 pi), uniform for a rotated vector): 16 equal cells, centroids (k + 1/2) pi / 8,
 * boundaries k pi / 8.  Level l >= 2 (atan2(r_{2i+1}, r_{2i}) of two radii of the level
 * below, in [0, pi/2], with sin^2 psi ~ Beta(m/2, m/2), m = 2^(l-1), density proportional
 * to sin^(m-1)(2 psi)): the 4-cell Lloyd-Max grid, iterated in fp64 with composite
 * Gauss-Legendre cell integrals to a change below 1e-13.  centroids: 16 or 4 values,
 * bounds: 15 or 3, ascending.  The codec table stores each centroid's cos and sin in fp32
 * and the boundaries in fp64 for the levels of d.  Host only. */
tq_status tq_make_polar_grid(int32_t level, double *centroids, double *bounds);

/* Size in bytes of the codec table built by tq_codec_build (0 if the desc is invalid). */
size_t tq_codec_bytes(const tq_codec_desc *desc);

/* Build the codec table on the host into `host_out` (tq_codec_bytes(desc) bytes): key
 * and value codebooks, the rotation signs D_j and the m x d Gaussian projection S, all
 * drawn from desc->seed.  The caller copies the table to device memory once and passes
 * that copy as `codec_dev` to the device entry points; it must have been built with the
 * same d, bits_k, bits_v and m as the cache it is used with.
 * Draws: SplitMix64 (Steele, Lea & Flood 2014) as a counter generator, output k of the
 * generator seeded with `seed` being mix(seed + (k + 1) * 0x9E3779B97F4A7C15); D_j uses
 * k = 2^32 + j and is -1 when the top bit is set; S_ij is the Box-Muller cosine branch
 * with uniforms from k = 2^33 + 2(i d + j) and the next k, in fp64, rounded to fp32. */
tq_status tq_codec_build(const tq_codec_desc *desc, void *host_out, size_t bytes);

/* Size in bytes of a packed cache (header + key bits + key norms [+ value codes + value
 * norms] [+ NSN means]), format version 1:
 *   header  256 B: u32 magic 0x564B5154, u32 version 1, u32 flags, u32 0, then the desc
 *           (eight i32, nsn last).
 *   Kbits   [batch][kv_heads][capacity][(bits_k d + m)/8]: bit p of each key code as
 *           plane p (coordinate j at byte j/8, bit j%8), planes p = 0..bits_k-1, then the
 *           m QJL sign bits.
 *   Knorm   [batch][kv_heads][capacity] x {fp16 ||y||, fp16 ||r||}.
 *   Vcodes  [batch][kv_heads][ceil(capacity/32)][d][4 bits_v bytes]: per 32-token tile and
 *           coordinate, token i's value code in bits [bits_v i, bits_v (i+1)) of a
 *           little-endian integer.
 *   Vnorm   [batch][kv_heads][capacity] fp16 ||y||.
 *   PolarQuant caches: a Kbits record is the 3 d / 8 bytes of angle codes (level-1 code i
 *           in bits [4 i, 4 i + 4), then levels 2, 3, ... in order, 2 bits per code, from
 *           bit 2 d; 2 zero bits last) followed by the m QJL sign bits; Vcodes holds token
 *           records of the same 3 d / 8 angle bytes, [batch][kv_heads][capacity].
 *   NSN caches: Knorm records are {fp16 ||y||, fp16 ||r||, fp16 s1, 0} (8 bytes), Vnorm
 *           records {fp16 ||y||, fp16 s1} (4 bytes), and a last region holds per unit
 *           [o_K, o_V, Pi o_K, Pi o_V], fp32 [d] each (the keys' mean taken after RoPE).
 * Regions start at multiples of 256 bytes.  Returns 0 if the desc is invalid. */
size_t tq_cache_bytes(const tq_cache_desc *desc);

/* Write the cache header (magic, version, desc) and clear the flags word; for an NSN
 * cache also set the means to zero.  Token slots are not touched.  Enqueued on
 * `stream`. */
tq_status tq_cache_init(const tq_cache_desc *desc, void *cache_dev, tq_stream_t stream);

/* Append tokens [start_pos, start_pos + n_new) of every (batch, kv-head) unit to the
 * packed cache ([TurboESM] 2.A-2.D; [TurboQuant] "Etape 1", "Etape 2"):
 *   keys:   y = Pi RoPE(k, pos) with Pi = blockdiag(H_B) diag(D) / sqrt(B) (H_B Sylvester,
 *           B the largest power of two dividing d), RoPE half-split with
 *           theta_j = rope_base^(-2j/d) (rope_base == 0: none); n = ||y||; code_j = number
 *           of boundaries t with y_j/n >= t; r = y - fp16(n) c[code]; QJL bit i =
 *           [(S r)_i >= 0]; stored: planes, sign bits, fp16 n, fp16 ||r||.
 *   values: y = Pi v (no RoPE), codes with the value codebook, fp16 n.
 *   NSN caches: before the norm, s1 = ||y|| / sqrt(d) is rounded to fp16 and
 *           y = y - s1 (Pi o) with the unit's stored fp32 Pi o (keys o_K, values o_V);
 *           s1 is stored next to the norms.
 * k, v: device arrays [batch][kv_heads][n_new][d] of `dtype`, contiguous; v must be NULL
 * iff desc->bits_v == 0; both must be 16-byte aligned (TQ_EINVAL otherwise).
 * n_new == 0 is a no-op.  Writes never touch other slots. */
tq_status tq_quantize_kv(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                         const void *k, const void *v, int32_t dtype, int32_t start_pos,
                         int32_t n_new, float rope_base, tq_stream_t stream);

/* Workspace bytes tq_decode_attend needs for this shape (splits chosen by the library). */
size_t tq_decode_workspace_bytes(const tq_cache_desc *desc, int32_t q_heads, int32_t length);

/* Split count tq_decode_attend uses for this shape (for inspection). */
int32_t tq_decode_splits(const tq_cache_desc *desc, int32_t q_heads, int32_t length);

/* GQA decode attention of one query per (batch, q-head) over cached tokens [0, length)
 * ([TurboESM] 2.A and 2.E; [TurboQuant] QJL estimator):
 *   q_rot = Pi RoPE(q, q_pos); sq = S q_rot;
 *   score_t = n_t <q_rot, c_k[code_t]> + ||r_t|| sqrt(pi/2)/m <sq, 2 bits_t - 1>;
 *   p = softmax(scale * score) (scale == 0: 1/sqrt(d)), computed as an online softmax
 *   over token splits; o_rot = sum_t p_t n_v,t c_v[vcode_t]; out = Pi^T o_rot.
 * q-head h reads kv-head floor(h * kv_heads / q_heads); q_heads must be a multiple of
 * kv_heads.  q: device [batch][q_heads][d] of `dtype`.  out: device fp32
 * [batch][q_heads][d].  scores: NULL or device fp32 [batch][q_heads][length], receiving
 * the unscaled score_t.  out == NULL (scores required) computes the logits only: the
 * scores are written and no softmax, value or output work is done.  length == 0 writes
 * out = 0.  ws: device workspace of at least
 * tq_decode_workspace_bytes bytes, overwritten. */
tq_status tq_decode_attend(const tq_cache_desc *desc, const void *codec_dev,
                           const void *cache_dev, int32_t length, const void *q,
                           int32_t dtype, int32_t q_heads, int32_t q_pos, float rope_base,
                           float scale, float *out, float *scores, void *ws, size_t ws_bytes,
                           tq_stream_t stream);

/* As tq_decode_attend with an explicit token split count (0 = the library's choice);
 * the workspace must then be tq_decode_workspace_bytes_splits(desc, q_heads, splits). */
size_t tq_decode_workspace_bytes_splits(const tq_cache_desc *desc, int32_t q_heads,
                                        int32_t splits);
tq_status tq_decode_attend_splits(const tq_cache_desc *desc, const void *codec_dev,
                                  const void *cache_dev, int32_t length, const void *q,
                                  int32_t dtype, int32_t q_heads, int32_t q_pos,
                                  float rope_base, float scale, float *out, float *scores,
                                  int32_t splits, void *ws, size_t ws_bytes,
                                  tq_stream_t stream);

/* Instrumented forms for measurement: identical to tq_quantize_kv and
 * tq_decode_attend_splits, and in addition record the caller's hipEvent_t `ev_start`
 * right before and `ev_stop` right after the kernel that streams the packed cache (the
 * quantize kernel; the split-K decode kernel) on `stream`.  Either event may be NULL. */
tq_status tq_quantize_kv_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                  void *cache_dev, const void *k, const void *v,
                                  int32_t dtype, int32_t start_pos, int32_t n_new,
                                  float rope_base, void *ev_start, void *ev_stop,
                                  tq_stream_t stream);
tq_status tq_decode_attend_profiled(const tq_cache_desc *desc, const void *codec_dev,
                                    const void *cache_dev, int32_t length, const void *q,
                                    int32_t dtype, int32_t q_heads, int32_t q_pos,
                                    float rope_base, float scale, float *out, float *scores,
                                    int32_t splits, void *ws, size_t ws_bytes,
                                    void *ev_start, void *ev_stop, tq_stream_t stream);

/* Workspace bytes tq_decode_attend_window needs for this shape. */
size_t tq_decode_window_workspace_bytes(const tq_cache_desc *desc, int32_t q_heads, int32_t length);

/* Decode attention over the packed tokens [0, length) and a full-precision window of the
 * most recent tokens ([NSNQuant] section 4, implementation details, residuals: the KV
 * cache is a quantized part plus a full-precision residual, which is quantized and
 * appended once full).  win_k, win_v: device [batch][kv_heads][win_cap][d] of win_dtype,
 * the raw keys (before RoPE) and values of positions length, ..., length + win_len - 1 in
 * slots 0 .. win_len - 1; 0 <= win_len <= win_cap <= 4096, d = 64 or 128, bits_v > 0.
 * A window token scores exactly <RoPE(q, q_pos), RoPE(k, pos)> (equal to the rotated-basis
 * product, Pi being orthogonal: [TurboESM] 2.A); one softmax runs over both sets.  out,
 * scale, q and the rest as tq_decode_attend (out may be NULL for logits only); scores:
 * NULL or [batch][q_heads][length + win_len], packed tokens first.  ws: at least
 * tq_decode_window_workspace_bytes bytes.  Flushing a full window into the cache is
 * tq_quantize_kv(desc, codec, cache, win_k, win_v, win_dtype, length, win_cap, rope_base),
 * the window buffer being exactly that call's [batch][kv_heads][n_new][d] input. */
tq_status tq_decode_attend_window(const tq_cache_desc *desc, const void *codec_dev,
                                  const void *cache_dev, int32_t length, const void *win_k,
                                  const void *win_v, int32_t win_dtype, int32_t win_len,
                                  int32_t win_cap, const void *q, int32_t dtype, int32_t q_heads,
                                  int32_t q_pos, float rope_base, float scale, float *out,
                                  float *scores, void *ws, size_t ws_bytes, tq_stream_t stream);

/* One generation step with the window managed in place ([NSNQuant] section 4, residuals:
 * the full-precision residual is quantized and appended to the packed part once full).
 * *length packed tokens and *win_len window tokens (host in/out; 0 <= *win_len <= win_cap)
 * precede the new token, whose raw key and value new_k, new_v (device
 * [batch][kv_heads][d] of win_dtype) sit at position *length + *win_len.  If the window
 * is full (*win_len == win_cap) its rows are first quantized into the packed cache at
 * positions *length ... (the tq_quantize_kv launch above, 16-byte aligned buffers), and
 * the window starts empty; the new token is then stored into row *win_len of win_k, win_v
 * by the attention kernel itself, and q attends over the packed tokens and the window
 * with it, as tq_decode_attend_window.  On TQ_OK *length and *win_len hold the new counts
 * and scores (optional) has rows of *length + *win_len; on a validation error nothing
 * was launched and nothing changes.  ws: tq_decode_window_workspace_bytes for the
 * packed length after the step (the cache capacity always suffices). */
tq_status tq_decode_step(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                         int32_t *length, void *win_k, void *win_v, int32_t win_dtype,
                         int32_t *win_len, int32_t win_cap, const void *new_k, const void *new_v,
                         const void *q, int32_t dtype, int32_t q_heads, int32_t q_pos,
                         float rope_base, float scale, float *out, float *scores, void *ws,
                         size_t ws_bytes, tq_stream_t stream);

/* Workspace bytes tq_nsn_set_means needs for n tokens per unit. */
size_t tq_nsn_means_workspace_bytes(const tq_cache_desc *desc, int32_t n);

/* Channel means of an NSN cache ([NSNQuant] section 1, the shift step; section 4 puts
 * NSN on keys before RoPE, here after it as for the plain codec): for every unit,
 * o_K = mean over its n tokens of sqrt(d) RoPE(k, pos) / ||k|| (positions start_pos ...)
 * and o_V = mean of sqrt(d) v / ||v||, accumulated in fp64 in a fixed order and stored in
 * fp32, then Pi o_K and Pi o_V (fp64, stored in fp32).  A zero token counts as a zero
 * vector.  Later tq_quantize_kv calls on the cache shift their tokens by these means;
 * typically k, v are the prefill and the call precedes its tq_quantize_kv.  k, v:
 * [batch][kv_heads][n][d] of `dtype`, 16-byte aligned; n >= 1; ws: at least
 * tq_nsn_means_workspace_bytes.  TQ_EINVAL on a cache without nsn. */
tq_status tq_nsn_set_means(const tq_cache_desc *desc, const void *codec_dev, void *cache_dev,
                           const void *k, const void *v, int32_t dtype, int32_t start_pos,
                           int32_t n, float rope_base, void *ws, size_t ws_bytes,
                           tq_stream_t stream);

/* Bytes of the device scratch array behind tq_decode_attend_noalloc (per GPU). */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* tq_decode_attend without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It computes exactly what tq_decode_attend computes with the library's own
 * split count (the same kernels; outputs are bitwise equal), and calls no hipMalloc,
 * hipFree or other allocating routine.  The workspace lives in a file-scope device array of
 * TQ_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the process
 * ends; the first call on a device looks up its address (hipGetSymbolAddress, with that
 * device made current for the lookup).  Shapes whose workspace,
 * tq_decode_workspace_bytes(desc, q_heads, length), exceeds TQ_NOALLOC_SCRATCH_BYTES
 * return TQ_ENOSPACE and enqueue nothing.  All calls on one GPU share that GPU's array,
 * which keeps the last call's contents (nothing in it needs to start at zero): calls that
 * overlap on one GPU (different streams or threads without ordering between them) race,
 * so the caller orders them, e.g. on one stream.  Arguments, errors and the device
 * chosen (the device of `stream`; the current device for the null stream) are as
 * tq_decode_attend. */
tq_status tq_decode_attend_noalloc(const tq_cache_desc *desc, const void *codec_dev,
                                   const void *cache_dev, int32_t length, const void *q,
                                   int32_t dtype, int32_t q_heads, int32_t q_pos, float rope_base,
                                   float scale, float *out, float *scores, tq_stream_t stream);

/* Workspace bytes tq_search_topk needs. */
size_t tq_search_workspace_bytes(const tq_cache_desc *db, int32_t n_db, int32_t nq, int32_t k);

/* Inner-product top-k search over packed database vectors ([TurboQuant] vector search:
 * top-k by the estimated inner product).  The database is a cache with batch =
 * kv_heads = 1 and bits_v = 0 filled by tq_quantize_kv (rope_base = 0, v = NULL), slots
 * [0, n_db).  For each query (device fp32 [nq][d]) the score of vector x is the same
 * estimator as in tq_decode_attend (with q_rot = Pi q, no RoPE).  idx_out (device int32
 * [nq][k]) and score_out (device fp32 [nq][k]) receive the k best in descending score,
 * equal scores ordered by lower index; if k > n_db the tail is idx -1, score -inf.
 * 1 <= k <= 64.  With 3-bit codes, m == d, d a multiple of 128 up to 2048 and k <= 16
 * the code term runs on int8 matrix cores (each centroid of the odd codebook is a sum
 * of four +-1 terms of its code bits, and the query is a 32-bit fixed point in four
 * int8 digits); other shapes use an fp32 path.  Both carry fp32-level accuracy. */
tq_status tq_search_topk(const tq_cache_desc *db, const void *codec_dev, const void *db_cache,
                         int32_t n_db, const float *queries, int32_t nq, int32_t k,
                         int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes,
                         tq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
