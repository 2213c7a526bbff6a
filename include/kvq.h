/*
 * kvq.h -- C ABI of libkvq: rotated INT2 KV-cache quantization and decode
 * attention over the packed cache, for AMD MI355X (gfx950).
 *
 * Method sources (cited by title and section):
 *   [OptR]  "Output-Aware Rotation for INT2 KV-Cache Quantization"
 *   [Eval]  "Output-aware INT2 KV-cache rotation evaluation"
 *
 * General rules for every entry point
 *   - Pointers are device pointers unless an argument says "host".  All
 *     arrays are dense, row-major, with the shapes given below.
 *   - The caller owns every buffer.  The library allocates and frees no
 *     memory.  Its only process-wide state is a counter that tags each
 *     decode launch, the compute-unit count of each device (read once: it
 *     sizes the split plan, so workspace sizes are those of the device
 *     current when they are queried) and the device address of the
 *     no-allocation scratch array; all three are safe to use from several
 *     threads.
 *   - Work is enqueued on `stream` and is asynchronous; results are ready
 *     after the caller synchronizes that stream.
 *   - All arguments that can be checked on the host are checked before the
 *     first launch; on any error nothing is launched and nothing is written.
 *   - There is no implicit fallback: a request outside what is implemented
 *     returns KVQ_ERR_UNSUPPORTED, never a slower path ([Eval], contract).
 *   - Device-resident indices (slot_mapping, page_table, seq_lens) cannot be
 *     checked on the host.  Kernels never access memory out of bounds: a
 *     slot outside the cache is skipped by kvq_quantize; a page index outside
 *     the cache, or seq_len < 0 or > max_seq_len, makes kvq_decode_attn write
 *     NaN to every output of the affected sequence.
 *   - K, V, q, W_O and dense rotation matrices start at 16-byte aligned
 *     addresses (every hipMalloc or torch allocation does); the kernels read
 *     them with 16-byte vector loads, so an unaligned one returns
 *     KVQ_ERR_INVALID_ARGUMENT.
 *   - Head dimension and quantization group size are both 128 ([OptR],
 *     Appendix Table A; [Eval]: group size 128, per-token-group K/V).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_HEAD_DIM 128
#define KVQ_GROUP_SIZE 128
#define KVQ_VERSION 1

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad shape, bad value          */
  KVQ_ERR_UNSUPPORTED = 2,      /* well-formed but not implemented             */
  KVQ_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required  */
  KVQ_ERR_HIP = 4               /* a HIP launch reported an error              */
} kvq_status;

/* Element type of K, V, q and W_O (all four share it in one call). */
enum { KVQ_F32 = 0, KVQ_BF16 = 1 };

/* Rotation kinds ([OptR] §3.1 Eq. (4): z' = z R, row-vector convention).
 *   IDENTITY         R = I (no rotation; also the "pre-rotated input" mode).
 *   SIGNED_HADAMARD  R = diag(s) H / sqrt(128), H the Sylvester Hadamard
 *                    matrix, s in {-1,+1}^128 ([Eval]: signed-Hadamard
 *                    candidates).
 *   DENSE            any orthogonal R given as fp32 ([OptR] §4.2 Eq. (11):
 *                    learned rotations R0 exp(A - A^T)). */
enum { KVQ_ROT_IDENTITY = 0, KVQ_ROT_SIGNED_HADAMARD = 1, KVQ_ROT_DENSE = 2 };

/* Candidate-search objective units. */
enum { KVQ_SELECT_JOINT = 0, KVQ_SELECT_PER_HEAD = 1 };

/* Per-KV-head rotations of one side (K or V).
 *   signs:  int8 [H][128], each +1 or -1 (kind SIGNED_HADAMARD), else unused.
 *   matrix: fp32 [H][128][128], row-major, z'_j = sum_i z_i R[i][j]
 *           (kind DENSE), else unused. */
typedef struct {
  int32_t kind;
  const int8_t *signs;
  const float *matrix;
} kvq_rotation;

/* Packed paged INT2 cache ([OptR] §1 and §6: rotation keeps the cache shape
 * and the paged layout; [Eval]: 2-bit codes, group 128).
 *
 *   pages: uint8 [num_pages][num_kv_heads][72 * page_size]
 *
 * One block per (page, KV head) holds page_size = P tokens (P % 16 == 0):
 *   bytes [0, 32P)     K codes, token-major: token p at 32p; byte m holds
 *                      dims 4m..4m+3, dim 4m+e in bits 2e..2e+1.
 *   bytes [32P, 64P)   V codes, four tokens interleaved: byte m of token p
 *                      at 32P + 128*(p/4) + 4m + (p%4), same bit order.
 *   bytes [64P, 68P)   K metadata: token p at 64P + 4p: fp16 scale (bytes
 *                      0-1) then fp16 zero (bytes 2-3), little-endian.
 *   bytes [68P, 72P)   V metadata, same format.
 * A code q of a group with scale s and zero z dequantizes to q*s + z.
 * Slot index = page * P + position in page.  Codes of one (token, head) pair
 * take 64 bytes (K + V) and metadata 8 bytes: 72 bytes in all. */
typedef struct {
  uint8_t *pages;
  int64_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
} kvq_cache;

/* Bytes of a cache buffer (num_pages * num_kv_heads * 72 * page_size). */
size_t kvq_cache_bytes(int64_t num_pages, int32_t page_size, int32_t num_kv_heads);

/* ---------------------------------------------------------------------------
 * kvq_quantize -- cache write ([OptR] §6 Efficiency Analysis; Appendix
 * Eq. (20)-(21); §4.1 key reparameterization; §3.1 Q2).
 *
 * For every token t < num_tokens and KV head h:
 *   k' = (k[t][h] - key_mean[h]) R_K[h]      (key_mean NULL: no centering)
 *   v' = v[t][h] R_V[h]
 * each 128-group is quantized with clip ratio clip_k (keys) or clip_v
 * (values): lo = c*min, hi = c*max, s = fp16((hi - lo)/3), z = fp16(lo),
 * code = clamp(round_half_even((x - z) * (1/s)), 0, 3), all codes 0 when
 * s == 0; codes and metadata are written to slot slot_mapping[t].
 *
 *   k, v          [num_tokens][H][128], dtype KVQ_F32 or KVQ_BF16, H =
 *                 cache->num_kv_heads.
 *   slot_mapping  int64 [num_tokens], or NULL for slot = t.  Negative slots
 *                 are skipped (token not written).
 *   rot_k, rot_v  host pointers to rotation descriptors (device arrays).
 *   key_mean      fp32 [H][128] or NULL.
 *   clip_k/clip_v in (0, 1].
 *   cache         host pointer to the descriptor; cache->pages is written.
 * Inputs must be finite and give |lo| and (hi-lo)/3 within fp16 range;
 * otherwise the metadata holds fp16 infinities (defined as unsupported
 * input).  With IDENTITY rotations, no key_mean and KVQ_F32 inputs, codes and
 * metadata equal the fp32 definition above bit for bit.
 * Errors: INVALID_ARGUMENT (nulls, num_tokens < 0, clip outside (0,1],
 * page_size % 16 != 0, H < 1), UNSUPPORTED (unknown dtype or rotation kind),
 * HIP.
 * ------------------------------------------------------------------------- */
int kvq_quantize(const void *k, const void *v, int32_t dtype, int64_t num_tokens, const int64_t *slot_mapping,
                 const kvq_rotation *rot_k, const kvq_rotation *rot_v, const float *key_mean, float clip_k,
                 float clip_v, const kvq_cache *cache, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kvq_decode_attn -- decode attention straight from the packed cache
 * ([OptR] Appendix Eq. (21)-(22), (26): rotated query against stored rotated
 * keys; §3 Eq. (1)-(3): softmax over the cached tokens with scale
 * 1/sqrt(128), probability-weighted values, per-head W_O blocks; Appendix
 * Eq. (27)-(28): explicit inverse value rotation).
 *
 * Query row r (r < num_seqs * queries_per_seq) belongs to sequence
 * b = r / queries_per_seq.  For query head j (KV head h = j / (Hq / H)):
 *   q'     = q[r][j] R_K[h]
 *   p_t    = softmax_t(q' . k_hat_t / sqrt(128)),  t < seq_lens[b]
 *   o'     = sum_t p_t v_hat_t;   out_o[r][j] = o' R_V[h]^T
 *   out_y[r] = sum_j out_o[r][j] W_O[j*128 : j*128+128, :]
 * Token t of sequence b sits in page page_table[b][t / P] at position t % P.
 * Only tokens t < seq_lens[b] are used: the cache slots at or past a
 * sequence's length and the table entries of pages holding none of its
 * tokens may hold anything (a table entry outside [0, num_pages) for a page
 * that does hold tokens makes that sequence's outputs NaN).
 *
 *   q            [num_seqs * queries_per_seq][Hq][128], dtype.
 *   page_table   int32 [num_seqs][max_pages_per_seq], or NULL for page
 *                b * max_pages_per_seq + t / P (contiguous caches).
 *   seq_lens     int32 [num_seqs], each in [0, max_seq_len]; an empty
 *                sequence gives out_o = 0.
 *   max_seq_len  host bound on seq_lens, <= max_pages_per_seq * P.
 *   w_o          [Hq*128][d_model], dtype, or NULL (then out_y is not
 *                written and d_model is ignored).
 *   out_o        fp32 [rows][Hq][128];  out_y fp32 [rows][d_model] or NULL.
 *   workspace    device scratch of at least kvq_decode_workspace_bytes(...)
 *                bytes with the same shape arguments.
 *   num_splits   split-K parts per sequence (0 = automatic).
 *   events       host pointer to a kvq_decode_events, or NULL.
 * Limits: Hq % H == 0 (else INVALID_ARGUMENT); queries_per_seq * Hq / H <= 64
 * and max_seq_len <= 2^26, else UNSUPPORTED.
 * Kernels: page sizes that are powers of two (16, 32, 64, ...) run the
 * matrix-core decode (one launch: query rotation, split attention, merge,
 * inverse value rotation).  Other multiples of 16 run a vector-unit split
 * kernel and a separate merge launch, about 4x slower at the same size; the
 * causal and windowed variants below do not take such page sizes.
 * ------------------------------------------------------------------------- */
/* Optional timing hook of kvq_decode_attn: when non-NULL, split_start and
 * split_stop are recorded on `stream` immediately before and after the
 * split-K attention kernel (the step that reads the packed cache), so a caller
 * can time that kernel alone with hipEventElapsedTime; attn_stop is recorded
 * after the split merge and inverse value rotation (out_o complete), before
 * the W_O projection.  Any of the three may be NULL.  Work is unchanged. */
typedef struct {
  hipEvent_t split_start;
  hipEvent_t split_stop;
  hipEvent_t attn_stop;
} kvq_decode_events;

size_t kvq_decode_workspace_bytes(int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t max_seq_len, int32_t d_model, int32_t num_splits);

int kvq_decode_attn(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                    const kvq_cache *cache, const int32_t *page_table, int32_t max_pages_per_seq,
                    const int32_t *seq_lens, int32_t max_seq_len, const kvq_rotation *rot_k,
                    const kvq_rotation *rot_v, const void *w_o, int32_t d_model, float *out_o, float *out_y,
                    void *workspace, size_t workspace_bytes, int32_t num_splits, const kvq_decode_events *events,
                    hipStream_t stream);

/* kvq_decode_attn with causal queries (a chunk of the last query positions,
 * as in the pages' objective over the final 64 query positions of a
 * sequence, [OptR] Appendix, calibration data and output-space error): the
 * queries_per_seq rows of sequence b are its last positions, so row qi
 * attends tokens t < seq_lens[b] - (queries_per_seq - 1 - qi) only (a row
 * left with no token gives out_o = 0).  Same arguments, workspace and limits
 * as kvq_decode_attn; UNSUPPORTED for page sizes that are not a power of two. */
int kvq_decode_attn_causal(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                           int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                           int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                           const kvq_rotation *rot_k, const kvq_rotation *rot_v, const void *w_o, int32_t d_model,
                           float *out_o, float *out_y, void *workspace, size_t workspace_bytes, int32_t num_splits,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kvq_decode_attn_noalloc -- kvq_decode_attn for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results and limits as
 * kvq_decode_attn, without the workspace: the split partials, the W_O operand
 * copy and the arrival counters live in a device array of the library of
 * KVQ_NOALLOC_SCRATCH_BYTES, one per GPU, held from the first call on that
 * GPU until the process ends.  The call allocates and frees nothing.
 * Returns KVQ_ERR_WORKSPACE, launching nothing, when the shapes need more
 * than that (kvq_decode_workspace_bytes(...) > KVQ_NOALLOC_SCRATCH_BYTES).
 * Every call on one GPU uses the same array (nothing in it needs clearing
 * between calls): two calls that may run at the same time on one GPU (on
 * different streams, or from different threads) race and must not overlap.
 * ------------------------------------------------------------------------- */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

int kvq_decode_attn_noalloc(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                            int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                            int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            const kvq_rotation *rot_k, const kvq_rotation *rot_v, const void *w_o, int32_t d_model,
                            float *out_o, float *out_y, int32_t num_splits, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * BF16 sink and recent windows ([OptR] §5, implementation details: 64 sink
 * and 256 recent tokens stay in BF16, 2.32 bits per element at a 64K-token
 * context; §4: sink and recent tokens skip INT2 quantization, their keys
 * keep the same centering, their values stay unchanged in BF16).
 *
 * For a sequence of length L: positions [0, lo), lo = min(num_sink, L), are
 * sink tokens; positions [hi, L), hi = max(lo, L - num_recent), are recent
 * tokens; positions [lo, hi) are read from the INT2 cache.  A window token's
 * logit is q . (k - key_mean) / sqrt(128) (key_mean as at the cache write,
 * or none) and its value is v itself; one softmax covers all L positions.
 *
 *   sink_k, sink_v      bf16 [num_seqs][num_sink][H][128]
 *   recent_k, recent_v  bf16 [num_seqs][num_recent][H][128]: the token at
 *                       position p sits in slot p % num_recent (a ring: a
 *                       position leaves it when position p + num_recent is
 *                       written, by which time it has left the window)
 * Buffers are owned by the caller; pointers may be NULL for a size of zero.
 * Limits: num_sink % 16 == 0 and num_sink + num_recent <= 384.
 * ------------------------------------------------------------------------- */
typedef struct {
  void *sink_k, *sink_v;
  void *recent_k, *recent_v;
  int32_t num_seqs, num_kv_heads, num_sink, num_recent;
} kvq_windows;

/* Window write: token i (of num_tokens, k and v [num_tokens][H][128] in
 * dtype) of sequence seq_idx[i] at position positions[i] goes to the sink
 * when the position is below num_sink, else to its recent slot (skipped
 * when num_recent == 0); fp32 inputs are rounded to bf16 (nearest even).
 * seq_idx and positions are device int32 [num_tokens]; a token whose
 * sequence is outside [0, num_seqs) or whose position is negative is
 * skipped.  seq_lens (device int32 [num_seqs], or NULL) is each sequence's
 * length once this write is done: a token at or past it is skipped, and a
 * non-sink token goes to the ring only when its position is at least
 * seq_lens[b] - num_recent, so one call can
 * carry a whole prefill; with NULL every non-sink token goes to its slot, and
 * two tokens of one call must not share a slot (which of them the slot keeps
 * is then undefined).  INT2 codes are written by kvq_quantize as before
 * (positions in the windows may be written there too; the decode does not
 * read them). */
int kvq_window_write(const void *k, const void *v, int32_t dtype, int64_t num_tokens, const int32_t *seq_idx,
                     const int32_t *positions, const int32_t *seq_lens, const kvq_windows *windows,
                     hipStream_t stream);

/* kvq_decode_attn with the windows: the same arguments and workspace, plus
 * the windows (H = the cache's KV heads) and the keys' centering key_mean
 * (fp32 [H][128] or NULL, as given to kvq_quantize; 16-byte aligned, else
 * INVALID_ARGUMENT).  Returns UNSUPPORTED for page sizes that are not a power
 * of two. */
int kvq_decode_attn_windows(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                            int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                            int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            const kvq_rotation *rot_k, const kvq_rotation *rot_v, const kvq_windows *windows,
                            const float *key_mean, const void *w_o, int32_t d_model, float *out_o, float *out_y,
                            void *workspace, size_t workspace_bytes, int32_t num_splits, hipStream_t stream);

/* Bits per cached element of one sequence of length L with the windows: INT2
 * tokens 2.25 (2-bit codes and an fp16 scale and zero per 128), window tokens
 * 16 (host function). */
double kvq_bits_per_element(int64_t seq_len, int32_t num_sink, int32_t num_recent);

/* ---------------------------------------------------------------------------
 * kvq_fold_value_rotation -- value-rotation folding ([OptR] Appendix,
 * equivalent inference implementation, Eq. (29)-(31)): out block b =
 * R_V[h]^T w block b, for w = num_blocks blocks of 128 rows, [num_blocks *
 * 128][cols] in dtype, block b belonging to KV head h = b / blocks_per_head.
 *   W_O [Hq*128][d_model], blocks_per_head = Hq / H: kvq_decode_attn with an
 *       identity rot_v and the folded W_O gives the same out_y as rot_v with
 *       W_O (out_o is then o R_V, the rotated output).
 *   W_V in [H*128][d_in] rows (v = x W_V^T), blocks_per_head = 1: the
 *       folded W_V projects values that are already rotated (cache write
 *       with an identity rot_v).
 * fp32 sums, the result rounded to dtype (nearest even); out must not
 * overlap w.  One-time weight preparation (not a per-step kernel).
 * ------------------------------------------------------------------------- */
int kvq_fold_value_rotation(const void *w, int32_t dtype, int32_t num_blocks, int32_t blocks_per_head, int32_t cols,
                            const kvq_rotation *rot_v, void *out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kvq_candidate_nmse -- batched post-W_O NMSE over a grid of candidate
 * rotations and clip ratios, and selection of the best one ([Eval], observed
 * envelope: identity + signed-Hadamard candidates x clip grid, chosen by
 * post-W_O output NMSE; [OptR] §3.2 Eq. (7), (10): the post-W_O error).
 *
 * For candidate r (used for both K and V) and clip clips[i] (used for both):
 * quantize K (centered by key_mean when given) and V as kvq_quantize does,
 * decode every query over all num_tokens tokens, and compare with the
 * full-precision output of the raw, unrotated K and V:
 *   JOINT     (U = 1):  NMSE_q = ||y_hat_q - y_q||^2 / ||y_q||^2 over the
 *                       whole layer output y_q = sum_j o_qj W_O[j-block].
 *   PER_HEAD  (U = H):  NMSE_q,h = sum_{j in G_h} ||y_hat_qj - y_qj||^2 /
 *                       sum_{j in G_h} ||y_qj||^2, y_qj = o_qj W_O[j-block].
 *   out_nmse[u][r][i]  = mean over queries of NMSE (fp32, device)
 *   out_nmse_per_query[u][r][i][q] (device, may be NULL)
 *   out_best[u] = r * num_clips + i of the first minimum in (r, i) order.
 *
 *   k, v          [num_tokens][H][128], dtype;  q [num_queries][Hq][128].
 *   candidates    host array [num_candidates] of rotation descriptors.
 *   clips         host array [num_clips], each in (0, 1].
 *   w_o           [Hq*128][d_model], dtype.
 *   workspace     at least kvq_candidate_workspace_bytes(...) bytes.
 * Limits: num_queries * Hq / H <= 64, and Hq <= 64 in JOINT mode, else
 * UNSUPPORTED.
 * ------------------------------------------------------------------------- */
size_t kvq_candidate_workspace_bytes(int64_t num_tokens, int32_t num_kv_heads, int32_t num_q_heads,
                                     int32_t num_queries, int32_t num_candidates, int32_t num_clips,
                                     int32_t d_model);

int kvq_candidate_nmse(const void *k, const void *v, const void *q, int32_t dtype, int64_t num_tokens,
                       int32_t num_kv_heads, int32_t num_q_heads, int32_t num_queries,
                       const kvq_rotation *candidates, int32_t num_candidates, const float *clips,
                       int32_t num_clips, const float *key_mean, const void *w_o, int32_t d_model, int32_t mode,
                       float *out_nmse, float *out_nmse_per_query, int32_t *out_best, void *workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * OptR offline calibration ([OptR] Appendix "OptR Algorithm", Algorithm 1;
 * §4.1 key reparameterization; §4.2 Eq. (11): R = R0 exp(A - A^T); §4.3
 * Eq. (12)-(14): key loss KL(p || p^K) + lambda_K ||e_K||^2 / d_model; §4.4
 * Eq. (15)-(16): value loss under the selected key attention; §4.5 Eq. (17)-
 * (18): the INT2 path with a straight-through estimator; Appendix,
 * calibration details and Table A: Adam, 80 steps, learning rate 0.02,
 * held-out selection every 20 steps, the final 64 query positions, clip
 * ratios 0.96 / 0.92, 64 sink and 256 recent BF16 tokens, lambda_K = 1).
 *
 * Traces of one layer: per sequence b of length L_b, keys and values of
 * every position and the queries of its final num_queries positions (query t
 * of them sits at position L_b - num_queries + t and attends positions
 * s <= that one).  For each KV head h (query heads h G .. h G + G - 1, G =
 * Hq / H): the key mean (the mean of every cached key of the calibration
 * set, unless key_mean is given); then A_K from 0 by Adam on L_K over the
 * calibration set, the held-out L_K checked after every eval_every steps and
 * the first minimum kept; then A_V likewise on L_V, whose attention is that
 * of the selected key rotation.  Positions [0, min(num_sink, L)) and
 * [max(that, L - num_recent), L) stay unquantized (keys centered); the rest
 * go through rotation, clipping, INT2 rounding (the fp32 sequence of
 * kvq_quantize) and dequantization, with the gradient passed where a value
 * lies inside its group's clipping range [c min, c max] and blocked
 * elsewhere.  Post-W_O errors use query head j's rows j*128 .. j*128+127 of
 * W_O [Hq*128][d_model]; losses are means over every (query, query head)
 * pair of the set.  Arithmetic is fp64 except the INT2 quantizer (fp32).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_seqs;          /* 1 .. 64 */
  int32_t max_len;           /* row count of k and v per sequence */
  const int32_t *seq_lens;   /* host [num_seqs], each in [num_queries, max_len] */
  const void *k, *v;         /* [num_seqs][max_len][H][128], dtype (rows past a length unused) */
  const void *q;             /* [num_seqs][num_queries][Hq][128], dtype */
} kvq_trace_set;

typedef struct {
  double lambda_k;           /* weight of the post-W_O key error (1.0) */
  float clip_k, clip_v;      /* clip ratios in (0, 1] (0.96, 0.92), fp32 as in kvq_quantize */
  int32_t num_sink, num_recent;  /* BF16 window sizes (64, 256), >= 0 */
  int32_t steps;             /* Adam steps per phase (80) */
  double lr;                 /* Adam learning rate (0.02); betas 0.9, 0.999, eps 1e-8 */
  int32_t eval_every;        /* held-out checkpoint period (20); with fewer steps, the last step */
} kvq_optr_config;

size_t kvq_optr_workspace_bytes(const kvq_trace_set *calib, const kvq_trace_set *heldout, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t num_queries, int32_t d_model);

/* calib, heldout, cfg: host structs (arrays device, seq_lens host).
 *   w_o          [Hq*128][d_model], dtype.
 *   r0_k, r0_v   fp32 [H][128][128] base rotations (any orthogonal).
 *   key_mean     fp32 [H][128], or NULL to estimate it from calib.
 *   out_r_k/v    fp32 [H][128][128]: R0 exp(A - A^T) of the selected A.
 *   out_key_mean fp32 [H][128] or NULL: the centering used.
 *   out_log      fp64 [H][2][steps + C + 1] or NULL (C = steps / eval_every,
 *                at least 1): per phase (keys, values) the training loss of
 *                every step (at the generator before its update), the
 *                held-out loss at each checkpoint, and the selected step.
 * Errors: INVALID_ARGUMENT (shapes, lengths, config), UNSUPPORTED (dtype,
 * more than 64 sequences), WORKSPACE, HIP. */
int kvq_optr_calibrate(int32_t dtype, const kvq_trace_set *calib, const kvq_trace_set *heldout, int32_t num_kv_heads,
                       int32_t num_q_heads, int32_t num_queries, const void *w_o, int32_t d_model, const float *r0_k,
                       const float *r0_v, const float *key_mean, const kvq_optr_config *cfg, float *out_r_k,
                       float *out_r_v, float *out_key_mean, double *out_log, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* One objective and its gradient at a given generator, per KV head (the
 * building block of kvq_optr_calibrate, for checking it or driving another
 * optimizer): phase 0 = L_K at R0 exp(A - A^T) (r0 = the key base rotation),
 * phase 1 = L_V at R0 exp(A - A^T) (r0 = the value base rotation) under the
 * attention of the key rotation r_k_hat (fp32 [H][128][128]).
 *   a          fp64 [H][128][128] device;  key_mean fp32 [H][128] (required).
 *   out_loss   fp64 [H];  out_grad fp64 [H][128][128] = dL/dA.
 * Workspace: kvq_optr_workspace_bytes(set, NULL, ...). */
int kvq_optr_loss_grad(int32_t dtype, int32_t phase, const kvq_trace_set *set, int32_t num_kv_heads,
                       int32_t num_q_heads, int32_t num_queries, const void *w_o, int32_t d_model, const float *r0,
                       const double *a, const float *r_k_hat, const float *key_mean, const kvq_optr_config *cfg,
                       double *out_loss, double *out_grad, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Human-readable name of a kvq_status value (static string). */
const char *kvq_status_string(int status);
/* KVQ_VERSION of the built library. */
int kvq_version(void);

#ifdef __cplusplus
}
#endif
#endif
