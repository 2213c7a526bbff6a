// decode.hip -- decode attention straight from the packed INT2 cache.
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization".
//   Appendix Eq. (21)-(22), (26): keys are stored rotated, the query is
//   rotated by its KV head's R_K, logit = (q R_K) . k_R / sqrt(128).
//   §3 Eq. (1)-(3): softmax over cached tokens, o = sum_t p_t v_t, and the
//   per-head W_O blocks; GQA head j uses KV head j / (Hq / H) (the set G_h).
//   Appendix Eq. (27)-(28): values are stored rotated; o = o' R_V^T.
//
// Dequantization is factored out of the dot products: with a group's scale
// s and zero z, q . (c s + z) = s (q . c) + z sum(q), and
// sum_t w_t (c_t s_t + z_t) = sum_t (w_t s_t) c_t + sum_t w_t z_t.
// Softmax runs in base 2: queries are pre-scaled by log2(e) / sqrt(128).
#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr float kLog2e = 1.4426950408889634f;


// ------------------------------------------------------------ rotations of one head vector
// One wave holds a 128-vector as two registers per lane: x0 = x[lane],
// x1 = x[lane + 64].

// ------------------------------------------------------------ query rotation
// q'[row][j] = q[row][j] R_K[h(j)] * log2(e)/sqrt(128); qsum = sum_c q'_c.
// One wave per (query row, query head).
template <int DT>
__global__ __launch_bounds__(256) void query_rotation_kernel(const void *q, int n_items, int Hq, int G, RotDev rk,
                                                             float *qrot, float *qsum) {
  const int lane = threadIdx.x & 63;
  const int rj = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rj >= n_items) return;
  const int h = (rj % Hq) / G;
  float y0 = load_elem<DT>(q, static_cast<size_t>(rj) * D + lane);
  float y1 = load_elem<DT>(q, static_cast<size_t>(rj) * D + lane + 64);
  rotate_query_wave(y0, y1, rk, h, lane);
  qrot[static_cast<size_t>(rj) * D + lane] = y0;
  qrot[static_cast<size_t>(rj) * D + lane + 64] = y1;
  const float sum = wave_sum(y0 + y1);
  if (lane == 0) qsum[rj] = sum;
}

// ------------------------------------------------------------ split kernels
struct SplitArgs {
  int R;            // rows of this (sequence, KV head): queries_per_seq * G
  int G, Hq, H, Nq;
  int split_tokens, splits;
  int max_seq_len;
  // packed cache
  const uint8_t *pages;
  int64_t num_pages;
  int P;
  const int32_t *page_table;
  int max_pages;
  const int32_t *seq_lens;
  const float *qrot, *qsum;
  float *part;
};

// Shared-memory layout of one split workgroup (floats unless noted).
template <int RB>
struct Smem {
  static constexpr int kQ = 0;                       // [RB][128] rotated queries
  static constexpr int kQsum = kQ + RB * D;          // [RB]
  static constexpr int kW = kQsum + RB;              // [RB][256] logits, then weights
  static constexpr int kVs = kW + RB * kChunk;       // [256] value scales
  static constexpr int kVz = kVs + kChunk;           // [256] value zeros
  static constexpr int kM = kVz + kChunk;            // [RB] running max
  static constexpr int kL = kM + RB;                 // [RB] running sum
  static constexpr int kZ = kL + RB;                 // [RB] running sum of w z
  static constexpr int kAlpha = kZ + RB;             // [RB] rescale factor of this chunk
  static constexpr int kFlag = kAlpha + RB;          // [1] error flag (int)
  static constexpr int kVc = kFlag + 4;              // bytes [256][32] value codes (as floats: 2048)
  static constexpr int kFloats = kVc + kChunk * 32 / 4;
  static constexpr size_t bytes() { return sizeof(float) * kFloats; }
};

// Phase 3: online softmax over one chunk; wave w owns rows w, w+4, ...
template <int RB>
__device__ __forceinline__ void softmax_chunk(float *sm, int R) {
  using S = Smem<RB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = wave; r < R; r += 4) {
    float *w = sm + S::kW + r * kChunk;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = w[lane * 4 + e];
    float cm = wave_maxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_old = sm[S::kM + r];
    const float m_new = fmaxf(m_old, cm);
    float alpha = 1.0f, lsum = 0.0f, zs = 0.0f;
    if (m_new != -INFINITY) {
      alpha = exp2f(m_old - m_new);  // m_old = -inf gives 0
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = lane * 4 + e;
        const float p = exp2f(x[e] - m_new);  // -inf logits give 0
        lsum += p;
        zs += p * sm[S::kVz + t];
        w[t] = p * sm[S::kVs + t];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[lane * 4 + e] = 0.0f;
    }
    lsum = wave_sum(lsum);
    zs = wave_sum(zs);
    if (lane == 0) {
      sm[S::kM + r] = m_new;
      sm[S::kL + r] = sm[S::kL + r] * alpha + lsum;
      sm[S::kZ + r] = sm[S::kZ + r] * alpha + zs;
      sm[S::kAlpha + r] = alpha;
    }
  }
}

// Phase 5: merge the two token halves of the value accumulators and write
// this split's partial (m, l, z, acc[128]) for every row.
template <int RB>
__device__ __forceinline__ void write_partial(float *sm, const SplitArgs &a, int b, int h, int s, float (&acc)[RB],
                                              bool bad) {
  using S = Smem<RB>;
  const int tid = threadIdx.x, i = tid & 127, half = tid >> 7;
  __syncthreads();
  float *x = sm + S::kW;  // reuse [RB][128]
  if (half == 1) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < a.R) x[r * D + i] = acc[r];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r < a.R) {
        const int qi = r / a.G, g = r % a.G;
        const size_t row = static_cast<size_t>(b) * a.Nq + qi;
        const int j = h * a.G + g;
        float *dst = a.part + ((row * a.Hq + j) * a.splits + s) * (D + 4);
        dst[4 + i] = acc[r] + x[r * D + i];
        if (i == 0) {
          dst[0] = sm[S::kM + r];
          dst[1] = bad ? __builtin_nanf("") : sm[S::kL + r];
          dst[2] = sm[S::kZ + r];
          dst[3] = 0.0f;
        }
      }
    }
  }
}

template <int RB>
__device__ __forceinline__ void init_split(float *sm, const SplitArgs &a, int b, int h) {
  using S = Smem<RB>;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < a.R * D; idx += 256) {
    const int r = idx / D, c = idx % D;
    const int qi = r / a.G, g = r % a.G;
    const size_t rj = (static_cast<size_t>(b) * a.Nq + qi) * a.Hq + h * a.G + g;
    sm[S::kQ + idx] = a.qrot[rj * D + c];
  }
  for (int r = tid; r < a.R; r += 256) {
    const int qi = r / a.G, g = r % a.G;
    const size_t rj = (static_cast<size_t>(b) * a.Nq + qi) * a.Hq + h * a.G + g;
    sm[S::kQsum + r] = a.qsum[rj];
    sm[S::kM + r] = -INFINITY;
    sm[S::kL + r] = 0.0f;
    sm[S::kZ + r] = 0.0f;
  }
  if (tid == 0) reinterpret_cast<int *>(sm)[S::kFlag] = 0;
}

// Partial attention over the packed cache: one workgroup per
// (split, KV head, sequence); 256 threads.
template <int RB>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitArgs a) {
  extern __shared__ float sm[];
  using S = Smem<RB>;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  init_split<RB>(sm, a, b, h);
  int L = a.seq_lens[b];
  bool bad = L < 0 || L > a.max_seq_len;
  if (bad) L = 0;
  const int t_begin = s * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, L);
  float acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = 0.0f;
  uint8_t *vc = reinterpret_cast<uint8_t *>(sm + S::kVc);
  const size_t block_bytes = static_cast<size_t>(72) * a.P;
  __syncthreads();

  for (int tok0 = t_begin; tok0 < t_end; tok0 += kChunk) {
    // ---- phase 1: this thread's token: K codes + metadata; stage V codes/meta
    const int tt = tok0 + tid;
    const bool valid = tt < t_end;
    const bool group_live = (tok0 + (tid & ~3)) < t_end;  // some token of this 4-group is valid
    uint32_t kw[8];
    float ks = 0.0f, kz = 0.0f, vsc = 0.0f, vze = 0.0f;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
    bool page_ok = true;
    if (group_live) {
      const int64_t page = a.page_table ? static_cast<int64_t>(a.page_table[static_cast<size_t>(b) * a.max_pages + tt / a.P])
                                        : static_cast<int64_t>(b) * a.max_pages + tt / a.P;
      page_ok = page >= 0 && page < a.num_pages;
      if (page_ok) {
        const int p = tt % a.P;
        const uint8_t *blk = a.pages + (static_cast<size_t>(page) * a.H + h) * block_bytes;
        v0 = *reinterpret_cast<const uint4 *>(blk + 32 * a.P + 32 * p);
        v1 = *reinterpret_cast<const uint4 *>(blk + 32 * a.P + 32 * p + 16);
        if (valid) {
          const uint4 k0 = *reinterpret_cast<const uint4 *>(blk + 32 * p);
          const uint4 k1 = *reinterpret_cast<const uint4 *>(blk + 32 * p + 16);
          kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
          kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
          const uint32_t km = *reinterpret_cast<const uint32_t *>(blk + 64 * a.P + 4 * p);
          const uint32_t vm = *reinterpret_cast<const uint32_t *>(blk + 68 * a.P + 4 * p);
          ks = half_bits_to_float(km & 0xffffu);
          kz = half_bits_to_float(km >> 16);
          vsc = half_bits_to_float(vm & 0xffffu);
          vze = half_bits_to_float(vm >> 16);
        }
      } else {
        reinterpret_cast<int *>(sm)[S::kFlag] = 1;
      }
    }
    const bool live = valid && page_ok;
    *reinterpret_cast<uint4 *>(vc + 32 * tid) = v0;
    *reinterpret_cast<uint4 *>(vc + 32 * tid + 16) = v1;
    sm[S::kVs + tid] = live ? vsc : 0.0f;
    sm[S::kVz + tid] = live ? vze : 0.0f;

    // ---- phase 2: logits of every row against this token
    float dot[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) dot[r] = 0.0f;
    if (live) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float cf[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) cf[e] = static_cast<float>((kw[w] >> (2 * e)) & 3u);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (r < a.R) {
            const float4 *qv = reinterpret_cast<const float4 *>(sm + S::kQ + r * D + 16 * w);
            float d = dot[r];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const float4 qq = qv[e4];
              d += qq.x * cf[4 * e4] + qq.y * cf[4 * e4 + 1] + qq.z * cf[4 * e4 + 2] + qq.w * cf[4 * e4 + 3];
            }
            dot[r] = d;
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (r < a.R) sm[S::kW + r * kChunk + tid] = live ? ks * dot[r] + kz * sm[S::kQsum + r] : -INFINITY;
    __syncthreads();

    // ---- phase 3: online softmax, weights w = p * s_v
    softmax_chunk<RB>(sm, a.R);
    __syncthreads();

    // ---- phase 4: value accumulation, thread = (dim i, token half)
    {
      const int i = tid & 127, half = tid >> 7;
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < a.R) acc[r] *= sm[S::kAlpha + r];
      const int n_tok = t_end - tok0;
      const int t_lo = half * (kChunk / 2);
      const int t_hi = min(t_lo + kChunk / 2, (n_tok + 3) & ~3);
      const int sh = 2 * (i & 3);
      for (int t = t_lo; t < t_hi; t += 4) {
        const uint32_t word = *reinterpret_cast<const uint32_t *>(vc + 128 * (t >> 2) + 4 * (i >> 2));
        const float c0 = static_cast<float>((word >> sh) & 3u);
        const float c1 = static_cast<float>((word >> (8 + sh)) & 3u);
        const float c2 = static_cast<float>((word >> (16 + sh)) & 3u);
        const float c3 = static_cast<float>((word >> (24 + sh)) & 3u);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          if (r < a.R) {
            const float4 wv = *reinterpret_cast<const float4 *>(sm + S::kW + r * kChunk + t);
            acc[r] += wv.x * c0 + wv.y * c1 + wv.z * c2 + wv.w * c3;
          }
        }
      }
    }
    __syncthreads();
  }
  if (reinterpret_cast<int *>(sm)[S::kFlag]) bad = true;
  write_partial<RB>(sm, a, b, h, s, acc, bad);
}

// ------------------------------------------------------------ combine
// Merge split partials (base-2 log-sum-exp), apply R_V^T, write out_o (and,
// for the W_O projection, a copy of o laid out [row group][K][16 rows]).
// One wave per (query row, query head).
constexpr int kMaxCombineSplits = kMaxSplits;

__global__ __launch_bounds__(256) void combine_kernel(const float *part, int n_items, int splits, int Hq, int G,
                                                      RotDev rv, float *out_o, float *ot, float *y_zero, int d_model) {
  const int lane = threadIdx.x & 63;
  const int rj = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rj >= n_items) return;
  const int row = rj / Hq, j = rj % Hq;
  float o0, o1;
  merge_partials(part + static_cast<size_t>(rj) * splits * (D + 4), splits, lane, o0, o1);
  unrotate_value_wave(o0, o1, rv, j / G, lane);
  store_output_wave(out_o, ot, row, j, Hq, lane, o0, o1);
  if (y_zero && j == 0)  // the row's W_O output starts at zero (the projection adds into it)
    for (int i = lane; i < d_model; i += 64) y_zero[static_cast<size_t>(row) * d_model + i] = 0.0f;
}


template <int RB>
hipError_t launch_split_rb(const DecodePlan &pl, const SplitArgs &a, hipStream_t stream) {
  const size_t smem = Smem<RB>::bytes();
  dim3 grid(pl.splits, pl.H, pl.num_seqs);
  if (smem > 65536) {
    // above the default dynamic shared-memory limit: opt in (gfx950 has 160 KB of LDS per workgroup)
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_split_kernel<RB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(decode_split_kernel<RB>, grid, dim3(256), smem, stream, a);
  return hipGetLastError();
}

hipError_t launch_split(const DecodePlan &pl, const SplitArgs &a, hipStream_t stream) {
  if (pl.rows_per_head <= 4) return launch_split_rb<4>(pl, a, stream);
  if (pl.rows_per_head <= 16) return launch_split_rb<16>(pl, a, stream);
  return launch_split_rb<64>(pl, a, stream);
}

}  // namespace

DecodePlan make_decode_plan(int num_seqs, int queries_per_seq, int Hq, int H, int max_seq_len, int d_model,
                            int num_splits, int page_size, bool windows) {
  DecodePlan pl{};
  pl.num_seqs = num_seqs;
  pl.queries_per_seq = queries_per_seq;
  pl.Hq = Hq;
  pl.H = H;
  pl.G = Hq / H;
  pl.rows_per_head = queries_per_seq * pl.G;
  pl.max_seq_len = max_seq_len;
  const int max_chunks = max_seq_len > 0 ? (max_seq_len + kChunk - 1) / kChunk : 1;
  int splits = num_splits;
  if (splits <= 0) {
    // at most one workgroup (8 waves) of the matrix-core kernel per CU, all
    // resident at once: two workgroups sharing a CU run at unequal speed (the
    // older one's waves win the issue arbitration), so the younger one's tail
    // runs at half occupancy, and workgroups past one per CU run as a second
    // round.  At most 64 splits (the last split merges up to 64 partials in
    // one pass; past 8 splits each workgroup merges its waves' partials
    // first); splits of at least 1024 tokens.  A workgroup takes one or two
    // groups of 4 query rows.
    const int n_rg = (queries_per_seq * (Hq / H) + 3) / 4;
    const int per_wg = mfma_row_groups_per_workgroup(n_rg, page_size, windows);
    const int n_wy = (n_rg + per_wg - 1) / per_wg;
    const int units = num_seqs * H * n_wy > 0 ? num_seqs * H * n_wy : 1;
    splits = device_cu_count() / units;
    if (splits > 64) splits = 64;
    const int max_by_len = max_chunks / 4 > 0 ? max_chunks / 4 : 1;  // >= 4 chunks of 256 tokens
    if (splits > max_by_len) splits = max_by_len;
  }
  if (splits > max_chunks) splits = max_chunks;
  if (splits > kMaxCombineSplits) splits = kMaxCombineSplits;
  if (splits < 1) splits = 1;
  int chunks_per_split = (max_chunks + splits - 1) / splits;
  if (chunks_per_split * kChunk > kMaxMfmaSplitTokens) chunks_per_split = kMaxMfmaSplitTokens / kChunk;
  pl.split_tokens = chunks_per_split * kChunk;
  pl.splits = (max_chunks + chunks_per_split - 1) / chunks_per_split;
  pl.d_model = d_model;
  // W_O: K slices so that column blocks x slices x row groups fill the chip
  const int K = Hq * D;
  const size_t rows_w = static_cast<size_t>(num_seqs) * queries_per_seq;
  const int row_groups = static_cast<int>((rows_w + kWoRows - 1) / kWoRows);
  const size_t rows = static_cast<size_t>(num_seqs) * queries_per_seq;
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  pl.off_qrot = off;
  off = align(off + rows * Hq * D * sizeof(float));
  pl.off_qsum = off;
  off = align(off + rows * Hq * sizeof(float));
  pl.off_part = off;
  // (the matrix-core kernel writes one partial per (split, wave), and one per split for the BF16 windows)
  off = align(off + rows * Hq * static_cast<size_t>(pl.splits) * (kMfmaWaves + 1) * (D + 4) * sizeof(float));
  pl.off_ot = off;  // [row groups][K][16] copy of o for the W_O projection
  off = align(off + (d_model > 0 ? static_cast<size_t>(row_groups) * K * kWoRows * sizeof(float) : 0));
  const size_t n_rg_all = static_cast<size_t>(num_seqs) * H * ((queries_per_seq * (Hq / H) + 3) / 4);
  pl.off_cnt = off;  // [num_seqs][H][row groups][kArrivalWords] uint64
  off = align(off + n_rg_all * kArrivalWords * sizeof(uint64_t));
  pl.total = off;
  return pl;
}

hipError_t launch_query_rotation(const void *q, int dtype, const DecodePlan &pl, RotDev rk, float *qrot,
                                 float *qsum, hipStream_t stream) {
  const int n = pl.num_seqs * pl.queries_per_seq * pl.Hq;
  if (n == 0) return hipSuccess;
  const dim3 grid((n + 3) / 4);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(query_rotation_kernel<KVQ_F32>, grid, dim3(256), 0, stream, q, n, pl.Hq, pl.G, rk, qrot,
                       qsum);
  else
    hipLaunchKernelGGL(query_rotation_kernel<KVQ_BF16>, grid, dim3(256), 0, stream, q, n, pl.Hq, pl.G, rk, qrot,
                       qsum);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodePlan &pl, const uint8_t *pages, int64_t num_pages, int page_size,
                               const int32_t *page_table, int max_pages, const int32_t *seq_lens,
                               const float *qrot, const float *qsum, float *part, hipStream_t stream) {
  if (pl.num_seqs == 0) return hipSuccess;
  SplitArgs a{};
  a.R = pl.rows_per_head;
  a.G = pl.G;
  a.Hq = pl.Hq;
  a.H = pl.H;
  a.Nq = pl.queries_per_seq;
  a.split_tokens = pl.split_tokens;
  a.splits = pl.splits;
  a.max_seq_len = pl.max_seq_len;
  a.pages = pages;
  a.num_pages = num_pages;
  a.P = page_size;
  a.page_table = page_table;
  a.max_pages = max_pages;
  a.seq_lens = seq_lens;
  a.qrot = qrot;
  a.qsum = qsum;
  a.part = part;
  return launch_split(pl, a, stream);
}

hipError_t launch_combine(const DecodePlan &pl, const float *part, RotDev rv, float *out_o, float *ot,
                          hipStream_t stream, float *y_zero) {
  const int n = pl.num_seqs * pl.queries_per_seq * pl.Hq;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, part, n, pl.splits, pl.Hq, pl.G, rv,
                     out_o, ot, y_zero, pl.d_model);
  return hipGetLastError();
}


}  // namespace kvq
