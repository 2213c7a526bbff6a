// kvq_internal.h -- device helpers and launcher declarations shared by the
// kernel translation units of libkvq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int D = 128;         // head dimension == quantization group size
constexpr int kMaxRows = 64;   // query rows sharing one (sequence, KV head)
constexpr int kChunk = 256;    // tokens per inner iteration of a decode split
constexpr int kMaxMfmaSplitTokens = 16384;  // tokens per split (page ids of a split fit in LDS)
constexpr int kMaxSplits = 4096;            // split partials merged per (row, head)
constexpr int64_t kMaxSeqLen = static_cast<int64_t>(kMaxSplits) * kMaxMfmaSplitTokens;

// Rotation descriptor passed by value to kernels.
struct RotDev {
  int32_t kind;
  const int8_t *signs;   // [H][128]
  const float *matrix;   // [H][128][128]
};

inline RotDev to_dev(const kvq_rotation &r) { return RotDev{r.kind, r.signs, r.matrix}; }

template <int DT>
__device__ __forceinline__ float load_elem(const void *p, size_t idx) {
  if constexpr (DT == KVQ_F32) {
    return static_cast<const float *>(p)[idx];
  } else {
    uint32_t b = static_cast<const uint16_t *>(p)[idx];
    return __uint_as_float(b << 16);
  }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  _Float16 h;
  uint16_t b = static_cast<uint16_t>(bits16);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// Entry of the Sylvester Hadamard matrix H[i][j] = (-1)^popcount(i & j).
__device__ __forceinline__ float hadamard_sign(int i, int j) {
  return (__popc(static_cast<unsigned>(i & j)) & 1) ? -1.0f : 1.0f;
}

// R[i][j] of one head as fp32 (used off the hot path: query rotation, inverse
// value rotation).  inv_sqrt_d = 1/sqrt(128).
__device__ __forceinline__ float rot_entry(const RotDev &r, int h, int i, int j, float inv_sqrt_d) {
  if (r.kind == KVQ_ROT_IDENTITY) return i == j ? 1.0f : 0.0f;
  if (r.kind == KVQ_ROT_SIGNED_HADAMARD)
    return static_cast<float>(r.signs[h * D + i]) * hadamard_sign(i, j) * inv_sqrt_d;
  return r.matrix[(static_cast<size_t>(h) * D + i) * D + j];
}

// One wave holds a 128-vector as x0 = x[lane], x1 = x[lane + 64].
// In-place fast Walsh-Hadamard transform: x <- x H, H[i][j] = (-1)^popcount(i & j)
// (Sylvester order, unnormalized): one butterfly stage per index bit.
__device__ __forceinline__ void fwht128(float &x0, float &x1, int lane) {
  const float a = x0 + x1, b = x0 - x1;  // bit 6: pairs (lane, lane + 64)
  x0 = a;
  x1 = b;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float p0 = __shfl_xor(x0, d), p1 = __shfl_xor(x1, d);
    const bool upper = (lane & d) != 0;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// q' = q R_K * log2(e)/sqrt(128) of one 128-vector held by a wave (row-vector
// convention z' = z R; signed Hadamard by the transform above).
__device__ __forceinline__ void rotate_query_wave(float &x0, float &x1, const RotDev &rk, int h, int lane) {
  float y0 = x0, y1 = x1;
  if (rk.kind == KVQ_ROT_SIGNED_HADAMARD) {
    x0 *= static_cast<float>(rk.signs[h * D + lane]);
    x1 *= static_cast<float>(rk.signs[h * D + lane + 64]);
    fwht128(x0, x1, lane);
    y0 = x0 * kInvSqrtD;
    y1 = x1 * kInvSqrtD;
  } else if (rk.kind == KVQ_ROT_DENSE) {
    const float *m = rk.matrix + static_cast<size_t>(h) * D * D;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll 8
    for (int i = 0; i < D; ++i) {
      const float zi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(i < 64 ? x0 : x1), i & 63));
      a0 += zi * m[i * D + lane];
      a1 += zi * m[i * D + lane + 64];
    }
    y0 = a0;
    y1 = a1;
  }
  x0 = y0 * (kLog2eF * kInvSqrtD);
  x1 = y1 * (kLog2eF * kInvSqrtD);
}

// ----------------------------------------------------------------- launchers
hipError_t launch_quantize(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                           const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean, float clip_k,
                           float clip_v, uint8_t *pages, int64_t num_pages, int page_size, hipStream_t stream);

struct DecodePlan {
  int num_seqs, queries_per_seq, Hq, H, G, rows_per_head;  // rows_per_head = queries_per_seq * G
  int max_seq_len, splits, split_tokens;                   // split_tokens % kChunk == 0
  int d_model, wo_ksplit, wo_kslice;
  size_t off_qrot, off_qsum, off_part, off_ypart;          // workspace layout (bytes)
  size_t off_qdig, off_qexp;                               // key-side query digits (matrix-core kernel)
  size_t off_ot;                                           // o laid out for the W_O projection
  int tiles_per_seq;                                       // 16-token tiles per sequence
  size_t off_tiles, total;                                 // tile address table (matrix-core kernel)
};
DecodePlan make_decode_plan(int num_seqs, int queries_per_seq, int Hq, int H, int max_seq_len, int d_model,
                            int num_splits);

// Rotated, pre-scaled queries and their sums (prologue of the decode step).
hipError_t launch_query_rotation(const void *q, int dtype, const DecodePlan &pl, RotDev rk, float *qrot,
                                 float *qsum, hipStream_t stream);
// Split-K partial attention over the packed cache.
hipError_t launch_decode_split(const DecodePlan &pl, const uint8_t *pages, int64_t num_pages, int page_size,
                               const int32_t *page_table, int max_pages, const int32_t *seq_lens,
                               const float *qrot, const float *qsum, float *part, hipStream_t stream);
// Same partials from the matrix-core kernel (rows_per_head <= 4).
bool decode_mfma_supported(const DecodePlan &pl, int page_size);
// Prologue of the matrix-core kernel (one launch): rotated queries and their
// sums, their fixed-point int8 digits (one 64-lane operand set per (sequence,
// KV head)) and the absolute code / metadata addresses of every 16-token tile
// (page indices validated here).
hipError_t launch_decode_prologue(const DecodePlan &pl, const void *q, int dtype, RotDev rk, const uint8_t *pages,
                                  int64_t num_pages, int page_size, const int32_t *page_table, int max_pages,
                                  float *qrot, float *qsum, int32_t *qdig, int32_t *qexp, uint64_t *tiles,
                                  hipStream_t stream);
hipError_t launch_decode_split_mfma(const DecodePlan &pl, int page_size, const int32_t *seq_lens,
                                    const int32_t *qdig, const int32_t *qexp, const float *qsum,
                                    const uint64_t *tiles, float *part, hipStream_t stream);
// Split-K partial attention over raw (unquantized, unrotated) K and V that
// every query row attends in full (reference readout of the candidate search).
hipError_t launch_reference_split(const DecodePlan &pl, const void *k, const void *v, int dtype,
                                  int64_t num_tokens, const float *qrot, float *part, hipStream_t stream);
// Merge splits, inverse value rotation, write out_o (and the W_O operand
// copy `ot` when not null).
hipError_t launch_combine(const DecodePlan &pl, const float *part, RotDev rv, float *out_o, float *ot,
                          hipStream_t stream);
// out_y = concat(out_o) W_O, from the copy written by launch_combine.
hipError_t launch_wo_projection(const DecodePlan &pl, const float *ot, const void *w_o, int dtype, float *ypart,
                                float *out_y, hipStream_t stream);

// Candidate search helpers.
hipError_t launch_fill_i32(int32_t *p, int32_t value, int n, hipStream_t stream);
hipError_t launch_nmse_terms(const float *o_hat, const float *o_ref, const void *w_o, int dtype, int Nq, int Hq,
                             int H, int d_model, int mode, float *nmse_q_out, size_t stride_u, hipStream_t stream);
hipError_t launch_select(const float *nmse_q, int U, int C, int n_clip, int Nq, float *out_nmse, int32_t *out_best,
                         hipStream_t stream);

}  // namespace kvq
