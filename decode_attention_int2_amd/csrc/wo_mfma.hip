// wo_mfma.hip -- output projection y = concat_j(o_j) W_O on the gfx950 matrix
// cores ([OptR] §3 Eq. (3): the attention output of query head j meets its
// own 128-row block of W_O; concatenating the heads makes it one product).
//
// o is the fp32 operand copy written by the decode kernel, laid out
// [row group of 16][K = Hq * 128][16]; W_O is [K][d_model] row-major, bf16 or
// fp32.  v_mfma_f32_16x16x4_f32 with A = o (16 rows x 4 k) and B = W_O
// (4 k x 16 columns): lane (c, kg) supplies o[row c][k + kg] and
// W_O[k + kg][n0 + 4c + j] for the 4 column tiles j, so each lane loads 4
// consecutive columns of one W_O row (64 lanes: 4 rows x 128 contiguous
// bytes for bf16) and tile j's output column c is n0 + 4c + j.  bf16
// weights are widened exactly; products and sums are fp32.
//
// One workgroup of 8 waves per (64 columns, K slice of 512 rows, row
// group); each wave takes 64 rows of the slice and issues all of its loads
// before the first product.  (Slices of 512 rows give two workgroups per CU
// at d_model = 4096, whose load round trips overlap: 2.7 us less per call
// than slices of 1,024 rows at 16 rows x [4096, 4096].)  The 8 waves are summed in LDS in a fixed order;
// with several K slices each workgroup adds its slice sum into y with fp32
// atomics (y cleared by the launch that wrote the o copy), so the order of
// the slice additions, and the last bits of y, vary from run to run.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kCols = 64;                 // columns per workgroup
constexpr int kWaves = 8;
constexpr int kWaveRows = 64;             // K rows per wave
constexpr int kSteps = kWaveRows / 4;     // matrix-core steps per wave

template <int DT>
struct WRaw;
template <>
struct WRaw<KVQ_BF16> {
  typedef uint2 type;  // 4 bf16
};
template <>
struct WRaw<KVQ_F32> {
  typedef float4 type;
};

// 4 consecutive W_O elements of row k from column n (columns past d_model read as 0)
template <int DT>
__device__ __forceinline__ typename WRaw<DT>::type load_w(const void *w, int k, int n, int d_model, bool vec) {
  const size_t idx = static_cast<size_t>(k) * d_model + n;
  if constexpr (DT == KVQ_BF16) {
    const uint16_t *p = static_cast<const uint16_t *>(w) + idx;
    if (vec) return *reinterpret_cast<const uint2 *>(p);
    uint32_t e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = n + j < d_model ? p[j] : 0u;
    return uint2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
  } else {
    const float *p = static_cast<const float *>(w) + idx;
    if (vec) return *reinterpret_cast<const float4 *>(p);
    float e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = n + j < d_model ? p[j] : 0.0f;
    return float4{e[0], e[1], e[2], e[3]};
  }
}

template <int DT>
__device__ __forceinline__ float w_elem(const typename WRaw<DT>::type &r, int j) {
  if constexpr (DT == KVQ_BF16) {
    const uint32_t x = j < 2 ? r.x : r.y;
    return __uint_as_float((j & 1) ? (x & 0xFFFF0000u) : (x << 16));
  } else {
    return j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
  }
}

struct WoArgs {
  const float *ot;     // [row groups][K][16]
  const void *w;       // [K][d_model]
  int rows, K, d_model, kslices;
  float *y;            // [rows][d_model]
};

template <int DT>
__global__ __launch_bounds__(64 * kWaves) void wo_mfma_kernel(WoArgs a) {
  __shared__ float red[kWaves][16][kCols + 4];  // per wave: 16 rows x 64 columns (padded)
  const int cb = blockIdx.x, ks = blockIdx.y, rg = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c = lane & 15, kg = lane >> 4;
  const int n0 = cb * kCols;
  const int ncol = n0 + 4 * c;
  // (workgroup-uniform: the whole 64-column block in range with 4-aligned rows)
  const bool vec = (a.d_model & 3) == 0 && n0 + kCols <= a.d_model;
  const int kw0 = ks * (kWaves * kWaveRows) + wave * kWaveRows;
  const int nk = min(max(a.K - kw0, 0), kWaveRows);  // rows of this wave
  const float *o = a.ot + static_cast<size_t>(rg) * a.K * 16;

  // all loads of the wave first (rows past the wave's share read as zero)
  typename WRaw<DT>::type wv[kSteps];
  float ov[kSteps];
  if (vec && nk == kWaveRows) {
    // (the common case: unconditional vector loads, all in flight together)
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int k = kw0 + 4 * st + kg;
      wv[st] = load_w<DT>(a.w, k, ncol, a.d_model, true);
      ov[st] = o[static_cast<size_t>(k) * 16 + c];
    }
  } else {
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int kr = 4 * st + kg;
      if (kr < nk) {
        wv[st] = load_w<DT>(a.w, kw0 + kr, ncol, a.d_model, vec);
        ov[st] = o[static_cast<size_t>(kw0 + kr) * 16 + c];
      } else {
        wv[st] = typename WRaw<DT>::type{};
        ov[st] = 0.0f;
      }
    }
  }
  v4f acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < kSteps; ++st)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ov[st], w_elem<DT>(wv[st], j), acc[j], 0, 0, 0);

  // lane (c, kg) holds rows 4 kg + i, columns n0 + 4c + j
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<float4 *>(&red[wave][4 * kg + i][4 * c]) = float4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
  __syncthreads();
  // fixed-order sum over the 8 waves: thread t takes outputs t and t + 512
  const int nrows = min(16, a.rows - rg * 16);
  float sums[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = threadIdx.x + 512 * u, r = idx >> 6, col = idx & 63;
    float v = red[0][r][col];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) v += red[w2][r][col];
    sums[u] = v;
  }
  if (a.kslices == 1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = threadIdx.x + 512 * u, r = idx >> 6, col = idx & 63;
      if (r < nrows && n0 + col < a.d_model) a.y[static_cast<size_t>(rg * 16 + r) * a.d_model + n0 + col] = sums[u];
    }
    return;
  }
  // several K slices: each adds its sums into y (cleared by the launch that
  // wrote ot), fp32 atomics at the device's memory, no reply awaited
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int idx = threadIdx.x + 512 * u, r = idx >> 6, col = idx & 63;
    if (r < nrows && n0 + col < a.d_model)
      unsafeAtomicAdd(a.y + static_cast<size_t>(rg * 16 + r) * a.d_model + n0 + col, sums[u]);
  }
}

}  // namespace

int wo_kslices(int K) { return (K + kWaves * kWaveRows - 1) / (kWaves * kWaveRows); }
int wo_col_blocks(int d_model) { return (d_model + kCols - 1) / kCols; }

hipError_t launch_wo_projection(const DecodePlan &pl, const float *ot, const void *w_o, int dtype, float *out_y,
                                hipStream_t stream) {
  const int rows = pl.num_seqs * pl.queries_per_seq;
  if (rows == 0 || pl.d_model <= 0) return hipSuccess;
  WoArgs a{};
  a.ot = ot;
  a.w = w_o;
  a.rows = rows;
  a.K = pl.Hq * D;
  a.d_model = pl.d_model;
  a.kslices = wo_kslices(a.K);
  a.y = out_y;
  const dim3 grid(wo_col_blocks(pl.d_model), a.kslices, (rows + 15) / 16);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(wo_mfma_kernel<KVQ_F32>, grid, dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(wo_mfma_kernel<KVQ_BF16>, grid, dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
