// reference_mfma.hip -- full-precision attention readout of the raw
// (unquantized, unrotated) K and V on the fp32 matrix cores: the reference
// output of the candidate search.
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization", §3
// Eq. (1)-(2): softmax over every token of the calibration window, o = sum_t
// p_t v_t; GQA query head j reads KV head j / (Hq / H).  Softmax runs in base
// 2 on queries pre-scaled by log2(e) / sqrt(128).
//
// One workgroup per (split of the tokens, KV head); wave w owns rows
// 16w .. 16w+15 of the head (row r = query qi * G + g) and runs its own online
// softmax over the split, 16 tokens per step, with v_mfma_f32_16x16x4_f32:
//   S^T = K Q^T:  A = K (16 tokens x 4 dims), B = Q^T (4 dims x 16 rows);
//                 lane (c, kg) supplies K[t0 + c][32 kg + st] and
//                 Q[row c][32 kg + st] at step st = 0..31, so each lane reads
//                 32 consecutive dims of one token and of one query row; lane
//                 (c, kg) ends with S[row c][t0 + 4 kg + i], i = 0..3.
//   O^T += V^T P^T: A = V^T (16 dims x 4 tokens), B = P^T (4 tokens x 16
//                 rows); at step st lane (c, kg) supplies V[t0 + 4 kg + st]
//                 [8 c + dt] for output tile dt (8 consecutive dims per load)
//                 and P[row c][t0 + 4 kg + st] -- its own softmax value, no
//                 lane exchange.  Lane (c, kg) ends with O[row c][32 kg + 8 i
//                 + dt]: 32 consecutive dims of its row, so the running max,
//                 sum and rescale of a row stay inside the 4 lanes of column c.
// Products and sums are fp32 (bf16 inputs widen exactly).  Each wave writes
// the (m, l, 0, o[128]) partial of its rows for its split; the combine kernel
// merges the splits.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

struct RefArgs {
  const void *k, *v;  // [T][H][128]
  int T, H, Hq, G, R;
  int split_tokens, splits;
  const float *qrot;  // [Nq][Hq][128], pre-scaled by log2(e) / sqrt(128)
  float *part;        // [Nq][Hq][splits][4 + 128]
};

// 8 consecutive elements of one token row
template <int DT>
struct Raw8;
template <>
struct Raw8<KVQ_BF16> {
  uint4 w;
};
template <>
struct Raw8<KVQ_F32> {
  float4 a, b;
};

template <int DT>
__device__ __forceinline__ Raw8<DT> load8(const void *base, size_t idx, bool ok) {
  Raw8<DT> r;
  if constexpr (DT == KVQ_BF16) {
    r.w = ok ? *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + idx) : uint4{0u, 0u, 0u, 0u};
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    r.a = ok ? p[0] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    r.b = ok ? p[1] : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  return r;
}

template <int DT>
__device__ __forceinline__ float elem8(const Raw8<DT> &r, int e) {
  if constexpr (DT == KVQ_BF16) {
    const uint32_t x = e < 2 ? r.w.x : e < 4 ? r.w.y : e < 6 ? r.w.z : r.w.w;
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  } else {
    const float4 &h = e < 4 ? r.a : r.b;
    const int f = e & 3;
    return f == 0 ? h.x : f == 1 ? h.y : f == 2 ? h.z : h.w;
  }
}

// K: 32 dims of token t0 + c; V: 8 dims of tokens t0 + 4 kg + st (zero past t_end)
template <int DT>
__device__ __forceinline__ void load_tile(const RefArgs &a, int h, int t0, int t_end, int c, int kg, Raw8<DT> (&kr)[4],
                                          Raw8<DT> (&vr)[4]) {
  const size_t tstride = static_cast<size_t>(a.H) * D;
  const int tk = t0 + c;
  const bool okk = tk < t_end;
  const size_t kb = static_cast<size_t>(okk ? tk : 0) * tstride + static_cast<size_t>(h) * D + 32 * kg;
#pragma unroll
  for (int u = 0; u < 4; ++u) kr[u] = load8<DT>(a.k, kb + 8 * u, okk);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int tv = t0 + 4 * kg + st;
    const bool okv = tv < t_end;
    vr[st] = load8<DT>(a.v, static_cast<size_t>(okv ? tv : 0) * tstride + static_cast<size_t>(h) * D + 8 * c, okv);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void reference_mfma_kernel(RefArgs a) {
  const int s = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, kg = lane >> 4;
  const int r = wave * 16 + c;  // this lane's row of the head
  const bool row_ok = r < a.R;
  const int qi = row_ok ? r / a.G : 0, j = h * a.G + (row_ok ? r % a.G : 0);

  float qv[32];  // Q[row][32 kg .. 32 kg + 31] (zero for rows past R)
  {
    const float4 *qp = reinterpret_cast<const float4 *>(a.qrot + (static_cast<size_t>(qi) * a.Hq + j) * D + 32 * kg);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 x = row_ok ? qp[u] : float4{0.0f, 0.0f, 0.0f, 0.0f};
      qv[4 * u] = x.x;
      qv[4 * u + 1] = x.y;
      qv[4 * u + 2] = x.z;
      qv[4 * u + 3] = x.w;
    }
  }
  const int t_begin = s * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, a.T);
  float m = -INFINITY, l = 0.0f;
  v4f o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  Raw8<DT> kn[4], vn[4];
  if (t_begin < t_end) load_tile<DT>(a, h, t_begin, t_end, c, kg, kn, vn);
  for (int t0 = t_begin; t0 < t_end; t0 += 16) {
    Raw8<DT> kc[4], vc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kc[u] = kn[u];
      vc[u] = vn[u];
    }
    if (t0 + 16 < t_end) load_tile<DT>(a, h, t0 + 16, t_end, c, kg, kn, vn);

    // logits of 16 tokens x 16 rows (four independent accumulation chains)
    v4f sa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sa[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < 32; ++st)
      sa[st & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(elem8<DT>(kc[st >> 3], st & 7), qv[st], sa[st & 3], 0, 0, 0);
    const v4f sv = (sa[0] + sa[1]) + (sa[2] + sa[3]);

    // online softmax of row c over tokens t0 + 4 kg + i
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (t0 + 4 * kg + i < t_end) ? sv[i] : -INFINITY;
    float tm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tm = fmaxf(tm, lane_xor(tm, 16));
    tm = fmaxf(tm, lane_xor(tm, 32));
    const float mn = fmaxf(m, tm);  // finite: token t0 is in range
    const float alpha = exp2f(m - mn);
    float p[4], ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(x[i] - mn);
      ps += p[i];
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(elem8<DT>(vc[st], dt), p[st], o[dt], 0, 0, 0);
  }
  // the row's sum over its 4 lanes (same running max in all of them)
  l += lane_xor(l, 16);
  l += lane_xor(l, 32);
  if (!row_ok) return;
  float *dst = a.part + ((static_cast<size_t>(qi) * a.Hq + j) * a.splits + s) * (D + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 *d4 = reinterpret_cast<float4 *>(dst + 4 + 32 * kg + 8 * i);
    d4[0] = float4{o[0][i], o[1][i], o[2][i], o[3][i]};
    d4[1] = float4{o[4][i], o[5][i], o[6][i], o[7][i]};
  }
  if (kg == 0) *reinterpret_cast<float4 *>(dst) = float4{m, l, 0.0f, 0.0f};
}

}  // namespace

hipError_t launch_reference_split(const DecodePlan &pl, const void *k, const void *v, int dtype,
                                  int64_t num_tokens, const float *qrot, float *part, hipStream_t stream) {
  if (pl.num_seqs != 1 || num_tokens < 1 || num_tokens > INT32_MAX) return hipErrorInvalidValue;
  const int R = pl.rows_per_head;
  if (R < 1 || R > 64) return hipErrorInvalidValue;
  RefArgs a{};
  a.k = k;
  a.v = v;
  a.T = static_cast<int>(num_tokens);
  a.H = pl.H;
  a.Hq = pl.Hq;
  a.G = pl.G;
  a.R = R;
  a.split_tokens = pl.split_tokens;
  a.splits = pl.splits;
  a.qrot = qrot;
  a.part = part;
  const dim3 grid(pl.splits, pl.H);
  const dim3 block(64 * ((R + 15) / 16));
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(reference_mfma_kernel<KVQ_F32>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(reference_mfma_kernel<KVQ_BF16>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
