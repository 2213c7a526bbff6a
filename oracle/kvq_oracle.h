/*
 * kvq_oracle.h -- plain, slow CPU oracle for rotated INT2 KV-cache quantization
 * and decode attention over the packed cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may build, load or call this code.  The
 * product path (the HIP library and its Python binding) never does, and this
 * code includes, links and calls nothing from the product path.
 *
 * Sources (all citations are to the pages the method is described on):
 *   [OptR]  "Output-Aware Rotation for INT2 KV-Cache Quantization" (paper deep
 *           dive page: full text of arXiv 2608.02691v2).
 *   [Eval]  "Output-aware INT2 KV-cache rotation evaluation" (project page
 *           with the observed 4,096-token envelope).
 *
 * Precision: every floating-point step is fp64, except the INT2 quantizer,
 * whose scale/zero are fp16 [Eval, observed envelope: fp16 scale/zero is part
 * of the recipe] and whose fp32 step sequence is this implementation's stated
 * reading of "group-wise affine INT2 with clipping ratio c" [OptR, §3.1 and
 * Appendix Table A].  The file is compiled with -O2 -ffp-contract=off and no
 * fast-math, so every fp32 operation rounds once, to nearest even.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQO_D 128 /* head dimension == quantization group size */

enum {
  KVQO_OK = 0,
  KVQO_ERR_ARG = 1,       /* bad shape, null pointer, out-of-range index   */
  KVQO_ERR_NONFINITE = 2, /* NaN/Inf input to the quantizer                */
  KVQO_ERR_RANGE = 3      /* scale or zero does not fit in fp16            */
};

enum { KVQO_ROT_IDENTITY = 0, KVQO_ROT_SIGNED_HADAMARD = 1, KVQO_ROT_DENSE = 2 };
enum { KVQO_SELECT_JOINT = 0, KVQO_SELECT_PER_HEAD = 1 };

/* fp32 -> fp16 bits, round to nearest even.  Returns KVQO_ERR_RANGE when the
 * rounded magnitude exceeds 65504, KVQO_ERR_NONFINITE for NaN/Inf. */
int kvqo_f32_to_f16(float x, uint16_t *bits);
float kvqo_f16_to_f32(uint16_t bits);

/* Sylvester Hadamard matrix of order n (power of two), entries +1/-1, built
 * by the doubling rule H(2m) = [[H(m), H(m)], [H(m), -H(m)]]. */
int kvqo_sylvester(int n, double *h);

/* Dense fp64 rotation R (row-vector convention z' = z R) for one head.
 * kind IDENTITY: R = I.  SIGNED_HADAMARD: R = diag(signs) H / sqrt(128).
 * DENSE: R = the given fp32 matrix (row-major [128][128]). */
int kvqo_rotation_matrix(int kind, const int8_t *signs, const float *matrix, double *r);

/* One INT2 group (n values, n >= 1): scale/zero and codes 0..3. */
int kvqo_quantize_group(const float *x, int n, float clip, uint8_t *codes, uint16_t *scale_bits,
                        uint16_t *zero_bits);

/* n groups of 128: x_hat = dequantized Q2 values, in_range = 1 where the
 * value lies inside the group's clipping range [c*min, c*max] (the
 * straight-through estimator of the OptR calibration passes gradients there). */
int kvqo_quantize_dequant_groups(const float *x, int64_t n, float clip, float *x_hat, uint8_t *in_range);

/* Paged packed cache, byte layout fixed by the C-ABI header of the library
 * (see the per-field comments in kvq_oracle.c, which restate it). */
typedef struct {
  uint8_t *pages;      /* [num_pages][num_kv_heads][72 * page_size] */
  int64_t num_pages;
  int32_t page_size;   /* tokens per page, multiple of 4 */
  int32_t num_kv_heads;
} kvqo_cache;

/* Rotations for all heads of one side (K or V). */
typedef struct {
  int32_t kind;
  const int8_t *signs;  /* [H][128] when kind == SIGNED_HADAMARD */
  const float *matrix;  /* [H][128][128] when kind == DENSE      */
} kvqo_rotation;

/* Cache write: rotate (and center keys), quantize every (token, head, K|V)
 * group, pack into slot slot_mapping[t] (identity when NULL).
 * k, v: [num_tokens][H][128] (bf16 inputs are passed widened to fp32). */
int kvqo_quantize(const float *k, const float *v, int64_t num_tokens, const int64_t *slot_mapping,
                  const kvqo_rotation *rot_k, const kvqo_rotation *rot_v, const float *key_mean,
                  float clip_k, float clip_v, kvqo_cache *cache);

/* Rotated values as fp32 (what the quantizer sees): out[t][h][:] */
int kvqo_rotate(const float *x, int64_t num_tokens, int32_t num_heads, const kvqo_rotation *rot,
                const float *mean, float *out);

/* Read back one group: codes[128], scale and zero bits. kv = 0 for K, 1 for V. */
int kvqo_read_group(const kvqo_cache *cache, int64_t slot, int32_t head, int kv, uint8_t *codes,
                    uint16_t *scale_bits, uint16_t *zero_bits);

/* Decode attention over the packed cache.
 * q: [num_seqs * queries_per_seq][Hq][128]; query row r belongs to sequence
 * r / queries_per_seq; page_table [num_seqs][max_pages] (NULL: page of token t
 * of sequence b is b * max_pages + t / page_size); seq_lens [num_seqs].
 * w_o: [Hq * 128][d_model] or NULL.  out_o: [rows][Hq][128]; out_y: [rows][d_model]. */
int kvqo_decode(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                const float *w_o, int32_t d_model, float *out_o, float *out_y);

/* Same decode but returning fp64 results (used by the candidate search). */
int kvqo_decode_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                    const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                    const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                    double *out_o);

/* Full-precision reference attention over raw K, V ([T][H][128]); every query
 * row attends all num_tokens tokens.  out_o: [rows][Hq][128] fp64. */
int kvqo_attention_ref(const float *q, int32_t rows, int32_t num_q_heads, const float *k,
                       const float *v, int64_t num_tokens, int32_t num_kv_heads, double *out_o);

/* Candidate search by post-W_O NMSE.  candidates: [C]; clips: [n_clip].
 * mode JOINT: one unit (the whole layer output); PER_HEAD: one unit per KV head.
 * out_nmse [U][C][n_clip] (mean over queries), out_nmse_q [U][C][n_clip][Nq]
 * (may be NULL), out_best [U] = r * n_clip + i of the first minimum. */
int kvqo_candidate_nmse(const float *k, const float *v, const float *q, int64_t num_tokens,
                        int32_t num_kv_heads, int32_t num_q_heads, int32_t num_queries,
                        const kvqo_rotation *candidates, int32_t num_candidates, const float *clips,
                        int32_t num_clips, const float *key_mean, const float *w_o, int32_t d_model,
                        int32_t mode, double *out_nmse, double *out_nmse_q, int32_t *out_best);

#ifdef __cplusplus
}
#endif

/* ------------------------------------------------------------------------ */
/* BF16 sink and recent windows ("Output-Aware Rotation for INT2 KV-Cache
 * Quantization", §5 setup: 64 sink and 256 recent tokens are kept in BF16,
 * and the effective cost is 2.32 bits per element at a 64K-token context;
 * §4: sink and recent tokens skip INT2 quantization, their keys keep the
 * same centering and their values stay unchanged in BF16; Appendix, key
 * reparameterization: the BF16 window keys keep the centering). */
typedef struct {
  const uint16_t *sink_k, *sink_v;     /* [num_seqs][num_sink][H][128] bf16 bits            */
  const uint16_t *recent_k, *recent_v; /* [num_seqs][num_recent][H][128] bf16 bits: the
                                          token at position p is in slot p % num_recent  */
  int32_t num_sink, num_recent;
  const float *key_mean;               /* [H][128] or NULL: the keys' centering mu        */
} kvqo_windows;

/* fp32 -> bf16 bits, round to nearest even (NaN stays NaN). */
uint16_t kvqo_f32_to_bf16(float x);

/* Window write of num_tokens tokens [num_tokens][H][128] (fp32; bf16 inputs
 * widened): token i of sequence seq_idx[i] at position positions[i] goes to
 * the sink when the position is below num_sink, else to recent slot
 * position % num_recent (when num_recent > 0; with seq_lens, the lengths
 * after the write, only when position >= seq_lens[b] - num_recent, and a
 * position at or past seq_lens[b] is not written); tokens are written in
 * index order; out-of-range indices are skipped. */
int kvqo_window_write(const float *k, const float *v, int64_t num_tokens, int32_t num_kv_heads,
                      const int32_t *seq_idx, const int32_t *positions, const int32_t *seq_lens, int32_t num_seqs,
                      uint16_t *sink_k,
                      uint16_t *sink_v, uint16_t *recent_k, uint16_t *recent_v, int32_t num_sink,
                      int32_t num_recent);

/* Decode with the windows, fp64: for a sequence of length L, positions below
 * lo = min(num_sink, L) are sink tokens, positions in [hi, L) with
 * hi = max(lo, L - num_recent) are recent tokens, and [lo, hi) are read from
 * the INT2 cache (as kvqo_decode_f64).  One softmax over all L positions;
 * a window token's logit is q . (k - mu) / sqrt(128) and its value is v
 * itself; INT2 tokens as kvqo_decode_f64. */
int kvqo_decode_windows_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                            const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                            const kvqo_windows *win, double *out_o);

/* Bits per cached element of a sequence of length L with the windows: each
 * INT2 token stores 2 bits per element plus an fp16 scale and zero per group
 * of 128 (2.25 bits per element), each window token 16 bits per element. */
double kvqo_bits_per_element(int64_t L, int32_t num_sink, int32_t num_recent);


/* Value-rotation folding ("Output-Aware Rotation for INT2 KV-Cache
 * Quantization", Appendix, equivalent inference implementation, Eq. (29)-(31):
 * the value rotation and its inverse are folded into the projection weights).
 * w holds num_blocks blocks of 128 rows, [num_blocks * 128][cols]; block b
 * belongs to KV head b / blocks_per_head, and out block b = R_V[h]^T w block b
 * (fp64 products in index order, rounded to fp32).  W_O [Hq*128][d_model]
 * (rows of query head j): blocks_per_head = Hq / H, then y = o' W_O-folded
 * for the rotated output o' = o R_V; W_V in [H*128][d_in] row layout (the
 * pages' W_{V,h}): blocks_per_head = 1, then x W_V-folded^T = (x W_V^T) R_V. */
int kvqo_fold_value_rotation(const float *w, int32_t num_blocks, int32_t blocks_per_head, int32_t cols,
                             const kvqo_rotation *rot_v, float *out);


/* Causal queries (the final query positions of a sequence, "Output-Aware
 * Rotation for INT2 KV-Cache Quantization", Appendix: the objective over the
 * final 64 query positions; causal attention distributions): row qi of
 * sequence b is position L - queries_per_seq + qi and attends the first
 * L - (queries_per_seq - 1 - qi) tokens; each row is kvqo_decode_f64 over
 * that prefix (no token: o = 0). */
int kvqo_decode_causal_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                           const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                           double *out_o);

#endif
