/*
 * kvq_oracle.c -- plain, slow CPU oracle.  TEST INFRASTRUCTURE ONLY: the test
 * suite, the smoke check and the benchmark's CPU-baseline leg are the only
 * callers.  Nothing here is shared with, included from, or called by the HIP
 * product path.
 *
 * Citations: [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization"
 * (paper deep-dive page); [Eval] = "Output-aware INT2 KV-cache rotation
 * evaluation" (project page).  Readings of passages that are silent or
 * garbled are marked READING and are listed in the design notes.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* fp16 <-> fp32.  READING: each group stores an fp16 scale and an fp16 zero.
 * 32 bits of metadata per 128-element group is what makes the 2.32
 * bits-per-element figure of [OptR, §5 Implementation Details] come out at
 * 64K context with the 64 + 256 BF16 window tokens of Appendix Table A.    */

int kvqo_f32_to_f16(float x, uint16_t *bits) {
  if (!isfinite(x)) return KVQO_ERR_NONFINITE;
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs((double)x);
  if (a == 0.0) {
    *bits = sign;
    return KVQO_OK;
  }
  int e2;
  (void)frexp(a, &e2);       /* a in [2^(e2-1), 2^e2)                        */
  int ex = e2 - 1;           /* exponent of the leading bit                   */
  if (ex < -14) ex = -14;    /* fp16 subnormal range: spacing 2^-24            */
  double quantum = ldexp(1.0, ex - 10);   /* spacing of fp16 values at ex     */
  double n = nearbyint(a / quantum);      /* exact quotient; ties to even     */
  if (n * quantum > 65504.0) return KVQO_ERR_RANGE;
  if (n >= 2048.0) {         /* rounding carried into the next binade         */
    n /= 2.0;
    ex += 1;
  }
  uint16_t h;
  if (n < 1024.0) {
    h = (uint16_t)n;         /* subnormal: value n * 2^-24                     */
  } else {
    h = (uint16_t)(((ex + 15) << 10) | ((int)n - 1024));
  }
  *bits = (uint16_t)(sign | h);
  return KVQO_OK;
}

float kvqo_f16_to_f32(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return (float)(s ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* Rotations.  [OptR, §3.1 Eq. (4)]: a cache vector z is rotated as zR before
 * quantization (row-vector convention).  [Eval, observed envelope]: identity
 * plus eight deterministic signed-Hadamard candidates.  READING: signed
 * Hadamard = diag(signs) * H / sqrt(128) with H the Sylvester matrix.
 * [OptR, §4.2 Eq. (11)]: learned rotations are dense orthogonal matrices
 * (here an input, already formed).                                          */

int kvqo_sylvester(int n, double *h) {
  if (n < 1 || (n & (n - 1))) return KVQO_ERR_ARG;
  h[0] = 1.0;
  for (int m = 1; m < n; m *= 2) {
    for (int i = 0; i < m; ++i) {
      for (int j = 0; j < m; ++j) {
        double x = h[(size_t)i * n + j];
        h[(size_t)i * n + (j + m)] = x;
        h[(size_t)(i + m) * n + j] = x;
        h[(size_t)(i + m) * n + (j + m)] = -x;
      }
    }
  }
  return KVQO_OK;
}

int kvqo_rotation_matrix(int kind, const int8_t *signs, const float *matrix, double *r) {
  const int d = KVQO_D;
  if (kind == KVQO_ROT_IDENTITY) {
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) r[i * d + j] = (i == j) ? 1.0 : 0.0;
    return KVQO_OK;
  }
  if (kind == KVQO_ROT_SIGNED_HADAMARD) {
    if (!signs) return KVQO_ERR_ARG;
    double *h = (double *)malloc(sizeof(double) * d * d);
    if (!h) return KVQO_ERR_ARG;
    kvqo_sylvester(d, h);
    double inv_sqrt = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) {
      if (signs[i] != 1 && signs[i] != -1) {
        free(h);
        return KVQO_ERR_ARG;
      }
      for (int j = 0; j < d; ++j) r[i * d + j] = (double)signs[i] * h[i * d + j] * inv_sqrt;
    }
    free(h);
    return KVQO_OK;
  }
  if (kind == KVQO_ROT_DENSE) {
    if (!matrix) return KVQO_ERR_ARG;
    for (int i = 0; i < d * d; ++i) r[i] = (double)matrix[i];
    return KVQO_OK;
  }
  return KVQO_ERR_ARG;
}

/* ------------------------------------------------------------------------ */
/* INT2 group quantizer Q2(.; c, G) [OptR, §3.1; Appendix Table A: group-wise
 * affine INT2, group size 128, clipping ratio].  READING of the unstated
 * arithmetic, in exactly this fp32 order:
 *   mn, mx = min, max of the group; lo = c*mn; hi = c*mx;
 *   s = fp16(((hi - lo) / 3)); z = fp16(lo);
 *   if s == 0 every code is 0; else inv = 1/s, t = (x - z) * inv,
 *   code = clamp(round-half-even(t), 0, 3).
 * Values outside [lo, hi] saturate to codes 0 and 3.                        */

int kvqo_quantize_group(const float *x, int n, float clip, uint8_t *codes, uint16_t *scale_bits,
                        uint16_t *zero_bits) {
  if (n < 1 || !x || !codes || !scale_bits || !zero_bits) return KVQO_ERR_ARG;
  if (!(clip > 0.0f && clip <= 1.0f)) return KVQO_ERR_ARG;
  for (int i = 0; i < n; ++i)
    if (!isfinite(x[i])) return KVQO_ERR_NONFINITE;
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  float lo = clip * mn;
  float hi = clip * mx;
  float span = hi - lo;
  float s32 = span / 3.0f;
  uint16_t sb, zb;
  int rc = kvqo_f32_to_f16(s32, &sb);
  if (rc) return rc;
  rc = kvqo_f32_to_f16(lo, &zb);
  if (rc) return rc;
  float s = kvqo_f16_to_f32(sb);
  float z = kvqo_f16_to_f32(zb);
  *scale_bits = sb;
  *zero_bits = zb;
  if (s == 0.0f) {
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return KVQO_OK;
  }
  float inv = 1.0f / s;
  for (int i = 0; i < n; ++i) {
    float diff = x[i] - z;
    float t = diff * inv;
    float r = nearbyintf(t);  /* default rounding mode: ties to even */
    if (r < 0.0f) r = 0.0f;
    if (r > 3.0f) r = 3.0f;
    codes[i] = (uint8_t)r;
  }
  return KVQO_OK;
}

/* Dequantized value: code * s + z, one fp32 rounding (code * s is exact). */
static float dequant(uint8_t code, uint16_t sb, uint16_t zb) {
  float s = kvqo_f16_to_f32(sb), z = kvqo_f16_to_f32(zb);
  float prod = (float)code * s;
  return prod + z;
}

/* Q2 then dequantization of n consecutive groups of 128 (x [n][128]), with
 * the straight-through estimator's pass-through flags of the OptR
 * calibration [OptR, §4.5 Eq. (18)]: x_hat = code * s + z of the group's Q2
 * (the values the cache would hold), in_range = 1 where lo <= x <= hi, the
 * group's clipping range.  READING: Eq. (18)'s |Z| <= tau_c, with tau_c
 * "determined by the clip ratio", is the range [c*min, c*max] that Q2 clips
 * to (R2): the gradient passes where the value is not clipped. */
int kvqo_quantize_dequant_groups(const float *x, int64_t n, float clip, float *x_hat, uint8_t *in_range) {
  if (!x || !x_hat || !in_range || n < 0) return KVQO_ERR_ARG;
  const int d = KVQO_D;
  uint8_t codes[KVQO_D];
  for (int64_t g = 0; g < n; ++g) {
    const float *xg = x + (size_t)g * d;
    uint16_t sb, zb;
    int rc = kvqo_quantize_group(xg, d, clip, codes, &sb, &zb);
    if (rc) return rc;
    float mn = xg[0], mx = xg[0];
    for (int i = 1; i < d; ++i) {
      if (xg[i] < mn) mn = xg[i];
      if (xg[i] > mx) mx = xg[i];
    }
    float lo = clip * mn, hi = clip * mx;
    for (int i = 0; i < d; ++i) {
      x_hat[(size_t)g * d + i] = dequant(codes[i], sb, zb);
      in_range[(size_t)g * d + i] = (uint8_t)(xg[i] >= lo && xg[i] <= hi);
    }
  }
  return KVQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed paged cache [OptR, §1 and §6: rotation keeps the cache shape and the
 * paged layout; the cache-write step quantizes, packs and writes].  Layout
 * (one block per (page, KV head), P tokens, 72*P bytes):
 *   K codes  at 32*p + m               (byte m of token p holds dims 4m..4m+3)
 *   V codes  at 32*P + 128*(p/4) + 4*m + (p%4)   (bytes of 4 tokens interleaved)
 *   K meta   at 64*P + 4*p: fp16 scale, then fp16 zero (little-endian)
 *   V meta   at 68*P + 4*p
 * Dim 4m+e of a code byte sits in bits 2e..2e+1.                             */

static uint8_t *block_ptr(const kvqo_cache *c, int64_t page, int32_t head) {
  return c->pages + ((size_t)page * (size_t)c->num_kv_heads + (size_t)head) * (size_t)(72 * c->page_size);
}

static size_t code_byte_offset(int P, int p, int dim, int kv) {
  int m = dim / 4;
  if (kv == 0) return (size_t)(32 * p + m);
  return (size_t)(32 * P + 128 * (p / 4) + 4 * m + (p % 4));
}

static size_t meta_offset(int P, int p, int kv) { return (size_t)((kv == 0 ? 64 : 68) * P + 4 * p); }

static void write_group(kvqo_cache *c, int64_t slot, int32_t head, int kv, const uint8_t *codes,
                        uint16_t sb, uint16_t zb) {
  int P = c->page_size;
  int64_t page = slot / P;
  int p = (int)(slot % P);
  uint8_t *blk = block_ptr(c, page, head);
  for (int i = 0; i < KVQO_D; ++i) {
    size_t off = code_byte_offset(P, p, i, kv);
    int sh = 2 * (i % 4);
    blk[off] = (uint8_t)((blk[off] & ~(3u << sh)) | ((unsigned)codes[i] << sh));
  }
  size_t mo = meta_offset(P, p, kv);
  blk[mo + 0] = (uint8_t)(sb & 0xff);
  blk[mo + 1] = (uint8_t)(sb >> 8);
  blk[mo + 2] = (uint8_t)(zb & 0xff);
  blk[mo + 3] = (uint8_t)(zb >> 8);
}

int kvqo_read_group(const kvqo_cache *c, int64_t slot, int32_t head, int kv, uint8_t *codes,
                    uint16_t *sb, uint16_t *zb) {
  if (!c || !c->pages || c->page_size < 4 || c->page_size % 4) return KVQO_ERR_ARG;
  int P = c->page_size;
  if (slot < 0 || slot >= c->num_pages * P || head < 0 || head >= c->num_kv_heads) return KVQO_ERR_ARG;
  int64_t page = slot / P;
  int p = (int)(slot % P);
  const uint8_t *blk = block_ptr(c, page, head);
  for (int i = 0; i < KVQO_D; ++i) {
    size_t off = code_byte_offset(P, p, i, kv);
    codes[i] = (uint8_t)((blk[off] >> (2 * (i % 4))) & 3u);
  }
  size_t mo = meta_offset(P, p, kv);
  *sb = (uint16_t)(blk[mo] | (blk[mo + 1] << 8));
  *zb = (uint16_t)(blk[mo + 2] | (blk[mo + 3] << 8));
  return KVQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Rotation of cached vectors with optional key centering.
 * [OptR, §4.1]: keys are centered by the per-channel calibration mean before
 * rotation and quantization (values are never shifted); [OptR, Appendix
 * Eq. (21)]: the stored key is Q2((k - mu) R_K).  Computed here in the
 * definition's form (k - mu) R, in fp64, then rounded to fp32.             */

int kvqo_rotate(const float *x, int64_t num_tokens, int32_t num_heads, const kvqo_rotation *rot,
                const float *mean, float *out) {
  const int d = KVQO_D;
  if (!x || !rot || !out || num_tokens < 0 || num_heads < 1) return KVQO_ERR_ARG;
  double *r = (double *)malloc(sizeof(double) * d * d);
  double *zc = (double *)malloc(sizeof(double) * d);
  if (!r || !zc) {
    free(r);
    free(zc);
    return KVQO_ERR_ARG;
  }
  int rc = KVQO_OK;
  for (int32_t h = 0; h < num_heads && rc == KVQO_OK; ++h) {
    rc = kvqo_rotation_matrix(rot->kind, rot->signs ? rot->signs + (size_t)h * d : NULL,
                              rot->matrix ? rot->matrix + (size_t)h * d * d : NULL, r);
    if (rc) break;
    for (int64_t t = 0; t < num_tokens; ++t) {
      const float *z = x + ((size_t)t * num_heads + h) * d;
      for (int i = 0; i < d; ++i) zc[i] = (double)z[i] - (mean ? (double)mean[(size_t)h * d + i] : 0.0);
      float *o = out + ((size_t)t * num_heads + h) * d;
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += zc[i] * r[i * d + j];
        o[j] = (float)acc;
      }
    }
  }
  free(r);
  free(zc);
  return rc;
}

static int quantize_rotated(const float *kr, const float *vr, int64_t num_tokens, int32_t H,
                            const int64_t *slot_mapping, float clip_k, float clip_v, kvqo_cache *cache) {
  uint8_t codes[KVQO_D];
  uint16_t sb, zb;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping ? slot_mapping[t] : t;
    if (slot < 0) continue; /* negative slot: token is not written */
    if (slot >= cache->num_pages * cache->page_size) return KVQO_ERR_ARG;
    for (int32_t h = 0; h < H; ++h) {
      const float *xk = kr + ((size_t)t * H + h) * KVQO_D;
      int rc = kvqo_quantize_group(xk, KVQO_D, clip_k, codes, &sb, &zb);
      if (rc) return rc;
      write_group(cache, slot, h, 0, codes, sb, zb);
      const float *xv = vr + ((size_t)t * H + h) * KVQO_D;
      rc = kvqo_quantize_group(xv, KVQO_D, clip_v, codes, &sb, &zb);
      if (rc) return rc;
      write_group(cache, slot, h, 1, codes, sb, zb);
    }
  }
  return KVQO_OK;
}

/* Cache write [OptR, §6 Efficiency Analysis and Appendix Eq. (20)-(21)]:
 * rotate the (centered) key, rotate the value, clip, quantize, pack, write. */
int kvqo_quantize(const float *k, const float *v, int64_t num_tokens, const int64_t *slot_mapping,
                  const kvqo_rotation *rot_k, const kvqo_rotation *rot_v, const float *key_mean,
                  float clip_k, float clip_v, kvqo_cache *cache) {
  if (!k || !v || !rot_k || !rot_v || !cache || !cache->pages || num_tokens < 0) return KVQO_ERR_ARG;
  if (cache->page_size < 4 || cache->page_size % 4 || cache->num_kv_heads < 1) return KVQO_ERR_ARG;
  int32_t H = cache->num_kv_heads;
  size_t n = (size_t)num_tokens * H * KVQO_D;
  float *kr = (float *)malloc(sizeof(float) * (n ? n : 1));
  float *vr = (float *)malloc(sizeof(float) * (n ? n : 1));
  int rc = (kr && vr) ? KVQO_OK : KVQO_ERR_ARG;
  if (!rc) rc = kvqo_rotate(k, num_tokens, H, rot_k, key_mean, kr);
  if (!rc) rc = kvqo_rotate(v, num_tokens, H, rot_v, NULL, vr);
  if (!rc) rc = quantize_rotated(kr, vr, num_tokens, H, slot_mapping, clip_k, clip_v, cache);
  free(kr);
  free(vr);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Decode attention.
 * [OptR, Appendix Eq. (21)-(22), (26)]: the cache stores the rotated key and
 * the query is rotated by its KV head's R_K, so logit = (q R_K) . k_R / sqrt(d)
 * (READING: the garbled "<q,k> d" of Eq. (1) is <q,k>/sqrt(d)).
 * [OptR, §3 Eq. (1)-(2)]: p = softmax over cached tokens, o = sum_s p_s v_s;
 * query head j uses KV head floor(j / (Hq/H)) (the set G_h of §3).
 * [OptR, Appendix Eq. (27)-(28)]: values were stored rotated, o' = o R_V, and
 * the inverse o = o' R_V^T recovers the original basis.
 * [OptR, §3 Eq. (3)]: y = sum_j o_j W_{O,j}^T, stored here as W_O rows
 * j*128 .. j*128+127 of a [Hq*128][d_model] matrix.                        */

int kvqo_decode_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                    const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                    const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                    double *out_o) {
  const int d = KVQO_D;
  if (!q || !cache || !cache->pages || !seq_lens || !rot_k || !rot_v || !out_o) return KVQO_ERR_ARG;
  if (num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1) return KVQO_ERR_ARG;
  int32_t H = cache->num_kv_heads, P = cache->page_size;
  if (H < 1 || num_q_heads % H) return KVQO_ERR_ARG;
  int32_t G = num_q_heads / H;
  double *rk = (double *)malloc(sizeof(double) * d * d);
  double *rv = (double *)malloc(sizeof(double) * d * d);
  double *qr = (double *)malloc(sizeof(double) * d);
  double *op = (double *)malloc(sizeof(double) * d);
  uint8_t codes[KVQO_D];
  uint16_t sb, zb;
  int rc = (rk && rv && qr && op) ? KVQO_OK : KVQO_ERR_ARG;
  for (int32_t b = 0; b < num_seqs && !rc; ++b) {
    int32_t L = seq_lens[b];
    if (L < 0 || L > max_pages * P) {
      rc = KVQO_ERR_ARG;
      break;
    }
    double *logit = (double *)malloc(sizeof(double) * (L ? L : 1));
    double *kh = (double *)malloc(sizeof(double) * (size_t)(L ? L : 1) * d);
    double *vh = (double *)malloc(sizeof(double) * (size_t)(L ? L : 1) * d);
    if (!logit || !kh || !vh) rc = KVQO_ERR_ARG;
    for (int32_t h = 0; h < H && !rc; ++h) {
      /* dequantize this head's cached keys and values (fp32 values) */
      for (int32_t t = 0; t < L && !rc; ++t) {
        int64_t page = page_table ? page_table[(size_t)b * max_pages + t / P] : (int64_t)b * max_pages + t / P;
        if (page < 0 || page >= cache->num_pages) {
          rc = KVQO_ERR_ARG;
          break;
        }
        int64_t slot = page * P + t % P;
        rc = kvqo_read_group(cache, slot, h, 0, codes, &sb, &zb);
        for (int i = 0; i < d && !rc; ++i) kh[(size_t)t * d + i] = (double)dequant(codes[i], sb, zb);
        if (!rc) rc = kvqo_read_group(cache, slot, h, 1, codes, &sb, &zb);
        for (int i = 0; i < d && !rc; ++i) vh[(size_t)t * d + i] = (double)dequant(codes[i], sb, zb);
      }
      if (rc) break;
      rc = kvqo_rotation_matrix(rot_k->kind, rot_k->signs ? rot_k->signs + (size_t)h * d : NULL,
                                rot_k->matrix ? rot_k->matrix + (size_t)h * d * d : NULL, rk);
      if (!rc)
        rc = kvqo_rotation_matrix(rot_v->kind, rot_v->signs ? rot_v->signs + (size_t)h * d : NULL,
                                  rot_v->matrix ? rot_v->matrix + (size_t)h * d * d : NULL, rv);
      if (rc) break;
      for (int32_t qi = 0; qi < queries_per_seq; ++qi) {
        int64_t row = (int64_t)b * queries_per_seq + qi;
        for (int32_t g = 0; g < G; ++g) {
          int32_t j = h * G + g;
          const float *qv = q + ((size_t)row * num_q_heads + j) * d;
          double *o = out_o + ((size_t)row * num_q_heads + j) * d;
          /* rotated query q' = q R_K */
          for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += (double)qv[i] * rk[i * d + c];
            qr[c] = acc;
          }
          if (L == 0) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            continue;
          }
          double mx = -INFINITY;
          for (int32_t t = 0; t < L; ++t) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += qr[i] * kh[(size_t)t * d + i];
            logit[t] = acc / sqrt((double)d);
            if (logit[t] > mx) mx = logit[t];
          }
          double zsum = 0.0;
          for (int c = 0; c < d; ++c) op[c] = 0.0;
          for (int32_t t = 0; t < L; ++t) {
            double p = exp(logit[t] - mx);
            zsum += p;
            for (int c = 0; c < d; ++c) op[c] += p * vh[(size_t)t * d + c];
          }
          for (int c = 0; c < d; ++c) op[c] /= zsum;
          /* inverse value rotation o = o' R_V^T */
          for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += op[c] * rv[i * d + c];
            o[i] = acc;
          }
        }
      }
    }
    free(logit);
    free(kh);
    free(vh);
  }
  free(rk);
  free(rv);
  free(qr);
  free(op);
  return rc;
}

static void project(const double *o, int32_t num_q_heads, const float *w_o, int32_t d_model, double *y) {
  for (int32_t n = 0; n < d_model; ++n) y[n] = 0.0;
  for (int32_t kk = 0; kk < num_q_heads * KVQO_D; ++kk) {
    const float *wr = w_o + (size_t)kk * d_model;
    for (int32_t n = 0; n < d_model; ++n) y[n] += o[kk] * (double)wr[n];
  }
}

int kvqo_decode(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                const float *w_o, int32_t d_model, float *out_o, float *out_y) {
  if (!out_o || num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1) return KVQO_ERR_ARG;
  size_t rows = (size_t)num_seqs * queries_per_seq;
  size_t n = rows * num_q_heads * KVQO_D;
  double *o = (double *)malloc(sizeof(double) * (n ? n : 1));
  if (!o) return KVQO_ERR_ARG;
  int rc = kvqo_decode_f64(q, num_seqs, queries_per_seq, num_q_heads, cache, page_table, max_pages, seq_lens,
                           rot_k, rot_v, o);
  if (!rc) {
    for (size_t i = 0; i < n; ++i) out_o[i] = (float)o[i];
    if (w_o && out_y && d_model > 0) {
      double *y = (double *)malloc(sizeof(double) * d_model);
      if (!y) rc = KVQO_ERR_ARG;
      for (size_t r = 0; r < rows && !rc; ++r) {
        project(o + r * num_q_heads * KVQO_D, num_q_heads, w_o, d_model, y);
        for (int32_t c = 0; c < d_model; ++c) out_y[r * d_model + c] = (float)y[c];
      }
      free(y);
    }
  }
  free(o);
  return rc;
}

/* Full-precision reference readout [OptR, §3 Eq. (1)-(2)] over raw,
 * unrotated, uncentered K and V. */
int kvqo_attention_ref(const float *q, int32_t rows, int32_t num_q_heads, const float *k,
                       const float *v, int64_t num_tokens, int32_t num_kv_heads, double *out_o) {
  const int d = KVQO_D;
  if (!q || !k || !v || !out_o || rows < 0 || num_q_heads < 1 || num_kv_heads < 1) return KVQO_ERR_ARG;
  if (num_q_heads % num_kv_heads || num_tokens < 1) return KVQO_ERR_ARG;
  int32_t G = num_q_heads / num_kv_heads;
  double *logit = (double *)malloc(sizeof(double) * num_tokens);
  if (!logit) return KVQO_ERR_ARG;
  for (int32_t r = 0; r < rows; ++r) {
    for (int32_t j = 0; j < num_q_heads; ++j) {
      int32_t h = j / G;
      const float *qv = q + ((size_t)r * num_q_heads + j) * d;
      double *o = out_o + ((size_t)r * num_q_heads + j) * d;
      double mx = -INFINITY;
      for (int64_t t = 0; t < num_tokens; ++t) {
        const float *kv = k + ((size_t)t * num_kv_heads + h) * d;
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += (double)qv[i] * (double)kv[i];
        logit[t] = acc / sqrt((double)d);
        if (logit[t] > mx) mx = logit[t];
      }
      double zsum = 0.0;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t t = 0; t < num_tokens; ++t) {
        double p = exp(logit[t] - mx);
        zsum += p;
        const float *vv = v + ((size_t)t * num_kv_heads + h) * d;
        for (int c = 0; c < d; ++c) o[c] += p * (double)vv[c];
      }
      for (int c = 0; c < d; ++c) o[c] /= zsum;
    }
  }
  free(logit);
  return KVQO_OK;
}

/* ------------------------------------------------------------------------ */
/* Candidate search [Eval, observed envelope]: every candidate rotation is
 * tried with every clip ratio; the objective is the post-W_O NMSE of the
 * layer output against the full-precision output, averaged over the
 * calibration queries; the first minimum is selected.  The error is the
 * post-W_O attention-output error of [OptR, §3.2 Eq. (7) and (10)].
 * READING: NMSE = ||y_hat - y||^2 / ||y||^2 per query, then the mean over
 * queries; per-head mode restricts y to the query heads of one KV head
 * (y_j = o_j W_{O,j}^T, Eq. (3)); K and V share the candidate and the clip. */

int kvqo_candidate_nmse(const float *k, const float *v, const float *q, int64_t num_tokens,
                        int32_t num_kv_heads, int32_t num_q_heads, int32_t num_queries,
                        const kvqo_rotation *candidates, int32_t num_candidates, const float *clips,
                        int32_t num_clips, const float *key_mean, const float *w_o, int32_t d_model,
                        int32_t mode, double *out_nmse, double *out_nmse_q, int32_t *out_best) {
  const int d = KVQO_D;
  if (!k || !v || !q || !candidates || !clips || !w_o || !out_nmse || !out_best) return KVQO_ERR_ARG;
  if (num_tokens < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads || num_queries < 1) return KVQO_ERR_ARG;
  if (num_candidates < 1 || num_clips < 1 || d_model < 1) return KVQO_ERR_ARG;
  if (mode != KVQO_SELECT_JOINT && mode != KVQO_SELECT_PER_HEAD) return KVQO_ERR_ARG;
  const int32_t H = num_kv_heads, Hq = num_q_heads, G = Hq / H, Nq = num_queries;
  const int32_t U = (mode == KVQO_SELECT_JOINT) ? 1 : H;
  const int32_t P = 16;
  const int64_t pages = (num_tokens + P - 1) / P;
  size_t nrot = (size_t)num_tokens * H * d;
  size_t no = (size_t)Nq * Hq * d;
  float *kr = (float *)malloc(sizeof(float) * nrot);
  float *vr = (float *)malloc(sizeof(float) * nrot);
  uint8_t *buf = (uint8_t *)calloc((size_t)pages * H * 72 * P, 1);
  double *o_ref = (double *)malloc(sizeof(double) * no);
  double *o_hat = (double *)malloc(sizeof(double) * no);
  double *y_ref = (double *)malloc(sizeof(double) * (size_t)Nq * Hq * d_model); /* per-head contributions */
  double *y_hat = (double *)malloc(sizeof(double) * (size_t)Hq * d_model);
  double *dy = (double *)malloc(sizeof(double) * d_model);
  double *yr = (double *)malloc(sizeof(double) * d_model);
  double *mean = (double *)malloc(sizeof(double) * U);
  int rc = (kr && vr && buf && o_ref && o_hat && y_ref && y_hat && dy && yr && mean) ? KVQO_OK : KVQO_ERR_ARG;
  kvqo_cache cache = {buf, pages, P, H};
  int32_t seq_len = (int32_t)num_tokens;
  /* reference outputs and per-head contributions y_{q,j} = o_{q,j} W_{O,j}^T */
  if (!rc) rc = kvqo_attention_ref(q, Nq, Hq, k, v, num_tokens, H, o_ref);
  for (int32_t qi = 0; qi < Nq && !rc; ++qi)
    for (int32_t j = 0; j < Hq; ++j) {
      double *y = y_ref + ((size_t)qi * Hq + j) * d_model;
      for (int32_t n = 0; n < d_model; ++n) y[n] = 0.0;
      for (int i = 0; i < d; ++i) {
        double oi = o_ref[((size_t)qi * Hq + j) * d + i];
        const float *wr = w_o + ((size_t)j * d + i) * d_model;
        for (int32_t n = 0; n < d_model; ++n) y[n] += oi * (double)wr[n];
      }
    }
  for (int32_t r = 0; r < num_candidates && !rc; ++r) {
    /* rotate once per candidate (keys centered first), then quantize per clip */
    rc = kvqo_rotate(k, num_tokens, H, &candidates[r], key_mean, kr);
    if (!rc) rc = kvqo_rotate(v, num_tokens, H, &candidates[r], NULL, vr);
    for (int32_t ci = 0; ci < num_clips && !rc; ++ci) {
      rc = quantize_rotated(kr, vr, num_tokens, H, NULL, clips[ci], clips[ci], &cache);
      if (!rc)
        rc = kvqo_decode_f64(q, 1, Nq, Hq, &cache, NULL, (int32_t)pages, &seq_len, &candidates[r],
                             &candidates[r], o_hat);
      if (rc) break;
      for (int32_t u = 0; u < U; ++u) mean[u] = 0.0;
      for (int32_t qi = 0; qi < Nq; ++qi) {
        for (int32_t j = 0; j < Hq; ++j) {
          double *y = y_hat + (size_t)j * d_model;
          for (int32_t n = 0; n < d_model; ++n) y[n] = 0.0;
          for (int i = 0; i < d; ++i) {
            double oi = o_hat[((size_t)qi * Hq + j) * d + i];
            const float *wr = w_o + ((size_t)j * d + i) * d_model;
            for (int32_t n = 0; n < d_model; ++n) y[n] += oi * (double)wr[n];
          }
        }
        for (int32_t u = 0; u < U; ++u) {
          int32_t j0 = (mode == KVQO_SELECT_JOINT) ? 0 : u * G;
          int32_t j1 = (mode == KVQO_SELECT_JOINT) ? Hq : (u + 1) * G;
          double num = 0.0, den = 0.0;
          if (mode == KVQO_SELECT_JOINT) {
            for (int32_t n = 0; n < d_model; ++n) {
              dy[n] = 0.0;
              yr[n] = 0.0;
            }
            for (int32_t j = j0; j < j1; ++j) {
              const double *yh = y_hat + (size_t)j * d_model;
              const double *y0 = y_ref + ((size_t)qi * Hq + j) * d_model;
              for (int32_t n = 0; n < d_model; ++n) {
                dy[n] += yh[n] - y0[n];
                yr[n] += y0[n];
              }
            }
            for (int32_t n = 0; n < d_model; ++n) {
              num += dy[n] * dy[n];
              den += yr[n] * yr[n];
            }
          } else {
            for (int32_t j = j0; j < j1; ++j) {
              const double *yh = y_hat + (size_t)j * d_model;
              const double *y0 = y_ref + ((size_t)qi * Hq + j) * d_model;
              for (int32_t n = 0; n < d_model; ++n) {
                double e = yh[n] - y0[n];
                num += e * e;
                den += y0[n] * y0[n];
              }
            }
          }
          double nm = num / den;
          if (out_nmse_q) out_nmse_q[(((size_t)u * num_candidates + r) * num_clips + ci) * Nq + qi] = nm;
          mean[u] += nm;
        }
      }
      for (int32_t u = 0; u < U; ++u)
        out_nmse[((size_t)u * num_candidates + r) * num_clips + ci] = mean[u] / (double)Nq;
    }
  }
  if (!rc) {
    for (int32_t u = 0; u < U; ++u) {
      int32_t best = 0;
      double bv = out_nmse[(size_t)u * num_candidates * num_clips];
      for (int32_t idx = 1; idx < num_candidates * num_clips; ++idx) {
        double x = out_nmse[(size_t)u * num_candidates * num_clips + idx];
        if (x < bv) {
          bv = x;
          best = idx;
        }
      }
      out_best[u] = best;
    }
  }
  free(kr);
  free(vr);
  free(buf);
  free(o_ref);
  free(o_hat);
  free(y_ref);
  free(y_hat);
  free(dy);
  free(yr);
  free(mean);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* BF16 sink and recent windows (the header states the passages). */

uint16_t kvqo_f32_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof(u));
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof(f));
  return (double)f;
}

int kvqo_window_write(const float *k, const float *v, int64_t num_tokens, int32_t num_kv_heads,
                      const int32_t *seq_idx, const int32_t *positions, const int32_t *seq_lens, int32_t num_seqs,
                      uint16_t *sink_k,
                      uint16_t *sink_v, uint16_t *recent_k, uint16_t *recent_v, int32_t num_sink,
                      int32_t num_recent) {
  const int d = KVQO_D;
  if (num_tokens < 0 || num_kv_heads < 1 || num_seqs < 0 || num_sink < 0 || num_recent < 0) return KVQO_ERR_ARG;
  if (num_tokens > 0 && (!k || !v || !seq_idx || !positions)) return KVQO_ERR_ARG;
  if ((num_sink > 0 && (!sink_k || !sink_v)) || (num_recent > 0 && (!recent_k || !recent_v))) return KVQO_ERR_ARG;
  for (int64_t i = 0; i < num_tokens; ++i) {
    const int32_t b = seq_idx[i], p = positions[i];
    if (b < 0 || b >= num_seqs || p < 0 || (seq_lens && p >= seq_lens[b])) continue;
    uint16_t *dk, *dv;
    if (p < num_sink) {
      dk = sink_k + ((size_t)b * num_sink + p) * num_kv_heads * d;
      dv = sink_v + ((size_t)b * num_sink + p) * num_kv_heads * d;
    } else if (num_recent > 0 && (!seq_lens || p >= seq_lens[b] - num_recent)) {
      dk = recent_k + ((size_t)b * num_recent + p % num_recent) * num_kv_heads * d;
      dv = recent_v + ((size_t)b * num_recent + p % num_recent) * num_kv_heads * d;
    } else {
      continue;
    }
    for (size_t e = 0; e < (size_t)num_kv_heads * d; ++e) {
      dk[e] = kvqo_f32_to_bf16(k[(size_t)i * num_kv_heads * d + e]);
      dv[e] = kvqo_f32_to_bf16(v[(size_t)i * num_kv_heads * d + e]);
    }
  }
  return KVQO_OK;
}

int kvqo_decode_windows_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                            const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                            const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                            const kvqo_windows *win, double *out_o) {
  const int d = KVQO_D;
  if (!q || !cache || !cache->pages || !seq_lens || !rot_k || !rot_v || !win || !out_o) return KVQO_ERR_ARG;
  if (num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1 || win->num_sink < 0 || win->num_recent < 0)
    return KVQO_ERR_ARG;
  if ((win->num_sink > 0 && (!win->sink_k || !win->sink_v)) ||
      (win->num_recent > 0 && (!win->recent_k || !win->recent_v)))
    return KVQO_ERR_ARG;
  const int32_t H = cache->num_kv_heads, P = cache->page_size, S = win->num_sink, W = win->num_recent;
  if (H < 1 || num_q_heads % H) return KVQO_ERR_ARG;
  const int32_t G = num_q_heads / H;
  double *rk = (double *)malloc(sizeof(double) * d * d);
  double *rv = (double *)malloc(sizeof(double) * d * d);
  double *qr = (double *)malloc(sizeof(double) * d);
  double *o_int = (double *)malloc(sizeof(double) * d);
  double *o_win = (double *)malloc(sizeof(double) * d);
  uint8_t codes[KVQO_D];
  uint16_t sb, zb;
  int rc = (rk && rv && qr && o_int && o_win) ? KVQO_OK : KVQO_ERR_ARG;
  for (int32_t b = 0; b < num_seqs && !rc; ++b) {
    const int32_t L = seq_lens[b];
    if (L < 0 || L > max_pages * P) {
      rc = KVQO_ERR_ARG;
      break;
    }
    const int32_t lo = L < S ? L : S;                /* sink: [0, lo)      */
    const int32_t hi = L - W > lo ? L - W : lo;      /* INT2: [lo, hi)     */
    const size_t n = (size_t)(L ? L : 1);            /* recent: [hi, L)    */
    double *logit = (double *)malloc(sizeof(double) * n);
    double *kt = (double *)malloc(sizeof(double) * n * d); /* INT2: rotated domain; window: k - mu */
    double *vt = (double *)malloc(sizeof(double) * n * d); /* INT2: rotated domain; window: v      */
    if (!logit || !kt || !vt) rc = KVQO_ERR_ARG;
    for (int32_t h = 0; h < H && !rc; ++h) {
      for (int32_t t = 0; t < L && !rc; ++t) {
        double *kr = kt + (size_t)t * d, *vr = vt + (size_t)t * d;
        if (t >= lo && t < hi) {
          int64_t page = page_table ? page_table[(size_t)b * max_pages + t / P] : (int64_t)b * max_pages + t / P;
          if (page < 0 || page >= cache->num_pages) {
            rc = KVQO_ERR_ARG;
            break;
          }
          const int64_t slot = page * P + t % P;
          rc = kvqo_read_group(cache, slot, h, 0, codes, &sb, &zb);
          for (int i = 0; i < d && !rc; ++i) kr[i] = (double)dequant(codes[i], sb, zb);
          if (!rc) rc = kvqo_read_group(cache, slot, h, 1, codes, &sb, &zb);
          for (int i = 0; i < d && !rc; ++i) vr[i] = (double)dequant(codes[i], sb, zb);
        } else {
          const uint16_t *ks, *vs;
          if (t < lo) {
            ks = win->sink_k + (((size_t)b * S + t) * H + h) * d;
            vs = win->sink_v + (((size_t)b * S + t) * H + h) * d;
          } else {
            ks = win->recent_k + (((size_t)b * W + t % W) * H + h) * d;
            vs = win->recent_v + (((size_t)b * W + t % W) * H + h) * d;
          }
          for (int i = 0; i < d; ++i) {
            const double mu = win->key_mean ? (double)win->key_mean[(size_t)h * d + i] : 0.0;
            kr[i] = bf16_to_f64(ks[i]) - mu;
            vr[i] = bf16_to_f64(vs[i]);
          }
        }
      }
      if (rc) break;
      rc = kvqo_rotation_matrix(rot_k->kind, rot_k->signs ? rot_k->signs + (size_t)h * d : NULL,
                                rot_k->matrix ? rot_k->matrix + (size_t)h * d * d : NULL, rk);
      if (!rc)
        rc = kvqo_rotation_matrix(rot_v->kind, rot_v->signs ? rot_v->signs + (size_t)h * d : NULL,
                                  rot_v->matrix ? rot_v->matrix + (size_t)h * d * d : NULL, rv);
      if (rc) break;
      for (int32_t qi = 0; qi < queries_per_seq; ++qi) {
        const int64_t row = (int64_t)b * queries_per_seq + qi;
        for (int32_t g = 0; g < G; ++g) {
          const int32_t j = h * G + g;
          const float *qv = q + ((size_t)row * num_q_heads + j) * d;
          double *o = out_o + ((size_t)row * num_q_heads + j) * d;
          for (int c = 0; c < d; ++c) { /* q' = q R_K for the INT2 keys */
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += (double)qv[i] * rk[i * d + c];
            qr[c] = acc;
          }
          if (L == 0) {
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            continue;
          }
          double mx = -INFINITY;
          for (int32_t t = 0; t < L; ++t) {
            const double *kr = kt + (size_t)t * d;
            const int in_int2 = t >= lo && t < hi;
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += (in_int2 ? qr[i] : (double)qv[i]) * kr[i];
            logit[t] = acc / sqrt((double)d);
            if (logit[t] > mx) mx = logit[t];
          }
          double zsum = 0.0;
          for (int c = 0; c < d; ++c) o_int[c] = o_win[c] = 0.0;
          for (int32_t t = 0; t < L; ++t) {
            const double p = exp(logit[t] - mx);
            const double *vr = vt + (size_t)t * d;
            double *acc = (t >= lo && t < hi) ? o_int : o_win;
            zsum += p;
            for (int c = 0; c < d; ++c) acc[c] += p * vr[c];
          }
          /* o = (o_int R_V^T + o_win) / zsum: the INT2 values are in the rotated domain */
          for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += o_int[c] * rv[i * d + c];
            o[i] = (acc + o_win[i]) / zsum;
          }
        }
      }
    }
    free(logit);
    free(kt);
    free(vt);
  }
  free(rk);
  free(rv);
  free(qr);
  free(o_int);
  free(o_win);
  return rc;
}

double kvqo_bits_per_element(int64_t L, int32_t num_sink, int32_t num_recent) {
  if (L <= 0) return 0.0;
  const int64_t sink = L < num_sink ? L : num_sink;
  const int64_t rest = L - sink;
  const int64_t recent = rest < num_recent ? rest : num_recent;
  const int64_t int2 = rest - recent;
  /* per head and side: an INT2 token stores 128 2-bit codes and two fp16 words, a window token 128 bf16 */
  return ((double)int2 * (128.0 * 2.0 + 32.0) + (double)(sink + recent) * 128.0 * 16.0) / ((double)L * 128.0);
}

/* ------------------------------------------------------------------------ */
/* Value-rotation folding (the header states the passage). */
int kvqo_fold_value_rotation(const float *w, int32_t num_blocks, int32_t blocks_per_head, int32_t cols,
                             const kvqo_rotation *rot_v, float *out) {
  const int d = KVQO_D;
  if (!w || !out || !rot_v || num_blocks < 1 || blocks_per_head < 1 || cols < 1 || num_blocks % blocks_per_head)
    return KVQO_ERR_ARG;
  double *r = (double *)malloc(sizeof(double) * d * d);
  if (!r) return KVQO_ERR_ARG;
  int rc = KVQO_OK;
  for (int32_t blk = 0; blk < num_blocks && !rc; ++blk) {
    const int32_t h = blk / blocks_per_head;
    rc = kvqo_rotation_matrix(rot_v->kind, rot_v->signs ? rot_v->signs + (size_t)h * d : NULL,
                              rot_v->matrix ? rot_v->matrix + (size_t)h * d * d : NULL, r);
    const float *wb = w + (size_t)blk * d * cols;
    float *ob = out + (size_t)blk * d * cols;
    for (int i = 0; i < d && !rc; ++i)
      for (int32_t n = 0; n < cols; ++n) {
        double acc = 0.0;  /* (R^T)[i][c] = R[c][i] */
        for (int c = 0; c < d; ++c) acc += r[c * d + i] * (double)wb[(size_t)c * cols + n];
        ob[(size_t)i * cols + n] = (float)acc;
      }
  }
  free(r);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Causal queries (the header states the passage). */
int kvqo_decode_causal_f64(const float *q, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                           const kvqo_cache *cache, const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, const kvqo_rotation *rot_k, const kvqo_rotation *rot_v,
                           double *out_o) {
  if (!q || !seq_lens || !out_o || num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1) return KVQO_ERR_ARG;
  const size_t row_elems = (size_t)num_q_heads * KVQO_D;
  for (int32_t b = 0; b < num_seqs; ++b) {
    for (int32_t qi = 0; qi < queries_per_seq; ++qi) {
      int32_t len = seq_lens[b] - (queries_per_seq - 1 - qi);
      if (len < 0) len = 0;
      const size_t row = (size_t)b * queries_per_seq + qi;
      const int rc = kvqo_decode_f64(q + row * row_elems, 1, 1, num_q_heads, cache,
                                     page_table ? page_table + (size_t)b * max_pages : NULL, max_pages, &len, rot_k,
                                     rot_v, out_o + row * row_elems);
      if (rc) return rc;
    }
  }
  return KVQO_OK;
}
