// fold.hip -- value-rotation folding of the projection weights.
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization", Appendix,
// equivalent inference implementation, Eq. (29)-(31): the value rotation
// and its inverse become part of W_V and W_O.  w holds blocks of 128 rows,
// block b belonging to KV head b / blocks_per_head; out block b =
// R_V[h]^T w block b.  With W_O [Hq*128][d_model] (blocks_per_head = Hq / H)
// the decode can then skip R_V^T (out_o stays in the rotated domain, y is
// unchanged); with W_V in [H*128][d_in] rows (blocks_per_head = 1) the
// projected values arrive rotated.  One-time weight preparation: fp32 sums
// over c in order, the result rounded to the weights' dtype.
#include "kvq_internal.h"

namespace kvq {
namespace {

struct FoldArgs {
  const void *w;
  void *out;
  int num_blocks, blocks_per_head, cols;
  RotDev rv;
};

constexpr int kFoldCols = 64;

template <int DT>
__global__ __launch_bounds__(256) void fold_kernel(FoldArgs a) {
  __shared__ float r_s[D][D + 1];        // R[c][i] of the block's head
  __shared__ float w_s[D][kFoldCols];    // the block's rows, 64 columns
  const int blk = blockIdx.y, n0 = blockIdx.x * kFoldCols;
  const int h = blk / a.blocks_per_head;
  for (int idx = threadIdx.x; idx < D * D; idx += 256) {
    const int c = idx >> 7, i = idx & 127;
    float r;
    if (a.rv.kind == KVQ_ROT_DENSE) {
      r = a.rv.matrix[static_cast<size_t>(h) * D * D + idx];
    } else if (a.rv.kind == KVQ_ROT_SIGNED_HADAMARD) {
      // diag(s) H / sqrt(128), H[c][i] = (-1)^popcount(c & i)
      const float hci = (__popc(c & i) & 1) ? -1.0f : 1.0f;
      r = static_cast<float>(a.rv.signs[h * D + c]) * hci * kInvSqrtD;
    } else {
      r = c == i ? 1.0f : 0.0f;
    }
    r_s[c][i] = r;
  }
  for (int idx = threadIdx.x; idx < D * kFoldCols; idx += 256) {
    const int c = idx / kFoldCols, n = idx % kFoldCols;
    w_s[c][n] = n0 + n < a.cols ? load_elem<DT>(a.w, (static_cast<size_t>(blk) * D + c) * a.cols + n0 + n) : 0.0f;
  }
  __syncthreads();
  const int n = threadIdx.x & 63, i0 = threadIdx.x >> 6;  // rows i0, i0 + 4, ..., i0 + 124
  float acc[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) acc[m] = 0.0f;
  for (int c = 0; c < D; ++c) {
    const float wv = w_s[c][n];
#pragma unroll
    for (int m = 0; m < 32; ++m) acc[m] += r_s[c][i0 + 4 * m] * wv;
  }
  if (n0 + n >= a.cols) return;
#pragma unroll
  for (int m = 0; m < 32; ++m) {
    const size_t o = (static_cast<size_t>(blk) * D + i0 + 4 * m) * a.cols + n0 + n;
    if constexpr (DT == KVQ_F32) {
      static_cast<float *>(a.out)[o] = acc[m];
    } else {
      uint32_t u = __float_as_uint(acc[m]);  // round to nearest even (NaN stays NaN)
      u = (u & 0x7FFFFFFFu) > 0x7F800000u ? (u | 0x400000u) : u + 0x7FFFu + ((u >> 16) & 1u);
      static_cast<uint16_t *>(a.out)[o] = static_cast<uint16_t>(u >> 16);
    }
  }
}

}  // namespace

hipError_t launch_fold_value_rotation(const void *w, int dtype, int num_blocks, int blocks_per_head, int cols,
                                      RotDev rv, void *out, hipStream_t stream) {
  FoldArgs a{w, out, num_blocks, blocks_per_head, cols, rv};
  const dim3 grid((cols + kFoldCols - 1) / kFoldCols, num_blocks);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(fold_kernel<KVQ_F32>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fold_kernel<KVQ_BF16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
