// candidate.hip -- post-W_O NMSE terms and candidate selection.
//
// [Eval] = "Output-aware INT2 KV-cache rotation evaluation", observed
// envelope: every candidate rotation is searched over the clip grid and the
// one with the lowest calibration post-W_O NMSE is selected.
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization", §3.2
// Eq. (7) and (10): the error is measured after W_O; §3 Eq. (3): head j
// contributes y_j = o_j W_{O,j}^T, here rows j*128..j*128+127 of W_O.
#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ void fill_i32_kernel(int32_t *p, int32_t value, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

// One workgroup per (query q, unit u).  JOINT: unit = all query heads, the
// per-head contributions are summed before squaring.  PER_HEAD: unit = the
// query heads of KV head u, each contribution squared separately.
template <int DT>
__global__ __launch_bounds__(256) void nmse_terms_kernel(const float *o_hat, const float *o_ref, const void *w_o,
                                                         int Hq, int G, int d_model, int mode, float *nmse_q,
                                                         size_t stride_u, int Nq) {
  extern __shared__ float sh[];  // [2][nh][128]: delta o, reference o
  __shared__ double red[2][4];
  const int q = blockIdx.x, u = blockIdx.y;
  const int j0 = (mode == KVQ_SELECT_JOINT) ? 0 : u * G;
  const int nh = (mode == KVQ_SELECT_JOINT) ? Hq : G;
  float *dob = sh, *orb = sh + nh * D;
  for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
    const size_t g = (static_cast<size_t>(q) * Hq + j0) * D + idx;
    dob[idx] = o_hat[g] - o_ref[g];
    orb[idx] = o_ref[g];
  }
  __syncthreads();
  double num = 0.0, den = 0.0;
  for (int n = threadIdx.x; n < d_model; n += 256) {
    float dy_sum = 0.0f, y_sum = 0.0f;
    for (int jj = 0; jj < nh; ++jj) {
      float dy = 0.0f, y = 0.0f;
      const size_t krow = static_cast<size_t>(j0 + jj) * D;
      for (int k = 0; k < D; ++k) {
        const float w = load_elem<DT>(w_o, (krow + k) * d_model + n);
        dy += dob[jj * D + k] * w;
        y += orb[jj * D + k] * w;
      }
      if (mode == KVQ_SELECT_JOINT) {
        dy_sum += dy;
        y_sum += y;
      } else {
        num += static_cast<double>(dy) * dy;
        den += static_cast<double>(y) * y;
      }
    }
    if (mode == KVQ_SELECT_JOINT) {
      num += static_cast<double>(dy_sum) * dy_sum;
      den += static_cast<double>(y_sum) * y_sum;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    num += __shfl_xor(num, o);
    den += __shfl_xor(den, o);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    red[0][wave] = num;
    red[1][wave] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double a = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const double b = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    nmse_q[static_cast<size_t>(u) * stride_u + q] = static_cast<float>(a / b);
  }
}

// Mean over queries and first argmin in (candidate, clip) order, per unit.
__global__ void select_kernel(const float *nmse_q, int C, int n_clip, int Nq, float *out_nmse, int32_t *out_best) {
  const int u = blockIdx.x;
  const int V = C * n_clip;
  const float *src = nmse_q + static_cast<size_t>(u) * V * Nq;
  for (int idx = threadIdx.x; idx < V; idx += blockDim.x) {
    double s = 0.0;
    for (int q = 0; q < Nq; ++q) s += src[static_cast<size_t>(idx) * Nq + q];
    out_nmse[static_cast<size_t>(u) * V + idx] = static_cast<float>(s / Nq);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int best = 0;
    float bv = out_nmse[static_cast<size_t>(u) * V];
    for (int idx = 1; idx < V; ++idx) {
      const float x = out_nmse[static_cast<size_t>(u) * V + idx];
      if (x < bv) {
        bv = x;
        best = idx;
      }
    }
    out_best[u] = best;
  }
}

}  // namespace

hipError_t launch_fill_i32(int32_t *p, int32_t value, int n, hipStream_t stream) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, value, n);
  return hipGetLastError();
}

hipError_t launch_nmse_terms(const float *o_hat, const float *o_ref, const void *w_o, int dtype, int Nq, int Hq,
                             int H, int d_model, int mode, float *nmse_q_out, size_t stride_u, hipStream_t stream) {
  const int G = Hq / H;
  const int U = (mode == KVQ_SELECT_JOINT) ? 1 : H;
  const int nh = (mode == KVQ_SELECT_JOINT) ? Hq : G;
  const size_t smem = sizeof(float) * 2 * nh * D;
  dim3 grid(Nq, U);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(nmse_terms_kernel<KVQ_F32>, grid, dim3(256), smem, stream, o_hat, o_ref, w_o, Hq, G, d_model,
                       mode, nmse_q_out, stride_u, Nq);
  else
    hipLaunchKernelGGL(nmse_terms_kernel<KVQ_BF16>, grid, dim3(256), smem, stream, o_hat, o_ref, w_o, Hq, G,
                       d_model, mode, nmse_q_out, stride_u, Nq);
  return hipGetLastError();
}

hipError_t launch_select(const float *nmse_q, int U, int C, int n_clip, int Nq, float *out_nmse, int32_t *out_best,
                         hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(U), dim3(256), 0, stream, nmse_q, C, n_clip, Nq, out_nmse, out_best);
  return hipGetLastError();
}

}  // namespace kvq
