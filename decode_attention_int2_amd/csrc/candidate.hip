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

// The post-W_O error of a unit through the Gram matrix of its W_O rows:
// ||sum_j x_j W_j||^2 = x G x^T with G = W W^T over the unit's rows of W_O
// (W_j = rows j*128 .. j*128+127).  PER_HEAD: each query head j of the unit
// is squared separately, so only the diagonal blocks G_jj = W_j W_j^T are
// needed (blocks of 128); JOINT: the unit is the whole layer output, one
// block of K = Hq * 128.  G is computed once per search; the reference
// output's square norms once per search; each variant then needs x G x^T of
// its output error x = o_hat - o_ref only.

// G[a][b] = sum_n W[a][n] W[b][n] for a, b in one block (fp32 products and
// sums): one workgroup per 64 x 64 tile of a block, W staged 64 columns at a
// time.  grid = (tiles per block, blocks).
template <int DT>
__global__ __launch_bounds__(256) void gram_kernel(const void *w_o, int d_model, int bdim, float *g) {
  __shared__ float wa[64][65], wb[64][65];
  const int blk = blockIdx.y, tpr = bdim / 64;
  const int ta = blockIdx.x / tpr, tb = blockIdx.x % tpr;
  const int a0 = blk * bdim + 64 * ta, b0 = blk * bdim + 64 * tb;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // 4 x 4 entries: rows ty + 16 i, cols tx + 16 j
  float acc[4][4] = {};
  for (int n0 = 0; n0 < d_model; n0 += 64) {
    for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
      const int r = idx >> 6, cc = idx & 63;
      const bool in = n0 + cc < d_model;
      wa[r][cc] = in ? load_elem<DT>(w_o, static_cast<size_t>(a0 + r) * d_model + n0 + cc) : 0.0f;
      wb[r][cc] = in ? load_elem<DT>(w_o, static_cast<size_t>(b0 + r) * d_model + n0 + cc) : 0.0f;
    }
    __syncthreads();
    for (int cc = 0; cc < 64; ++cc) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = wa[ty + 16 * i][cc];
        bv[i] = wb[tx + 16 * i][cc];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
    }
    __syncthreads();
  }
  float *gb = g + static_cast<size_t>(blk) * bdim * bdim;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) gb[static_cast<size_t>(64 * ta + ty + 16 * i) * bdim + 64 * tb + tx + 16 * j] = acc[i][j];
}

// One workgroup per (unit u, QW queries): e_q = sum over the unit's blocks
// of x_q G x_q^T, x = x1 - x0 (x0 may be null).  Thread t owns row
// r = t % 128 (+ 128 i) of a block for the QW / 2 queries of half t / 128:
// t_q(r) = sum_c G[c][r] x_q[c] (G is symmetric bit for bit -- its two
// triangles are the same products summed in the same order -- so the reads
// of column r are coalesced and each G value serves QW / 2 queries), then
// e_q = sum_r x_q[r] t_q(r).  kDen: store e as the unit's reference norm
// den[u][q]; otherwise write the NMSE e / den[u][q].  x is staged in LDS as
// [QW][bdim] fp32 (at most 64 KiB: QW is picked from bdim).
template <bool kDen, int QW>
__global__ __launch_bounds__(256) void quadform_kernel(const float *x1_all, const float *x0, const float *g, int Hq,
                                                       int blocks_per_unit, int bdim, double *den, float *nmse_q_all,
                                                       size_t stride_u, int Nq, int nvar) {
  constexpr int kHalf = QW / 2;
  extern __shared__ float xs[];  // [QW][bdim]
  __shared__ double red[4][kHalf];
  const int u = blockIdx.y, q0 = blockIdx.x * QW;
  const int nq = min(QW, Nq - q0);
  const int r0 = threadIdx.x & 127, qh = threadIdx.x >> 7;
  const size_t x_stride = static_cast<size_t>(Nq) * Hq * D;
  for (int var = blockIdx.z; var < nvar; var += gridDim.z) {
  const float *x1 = x1_all + var * x_stride;
  float *nmse_q = kDen ? nullptr : nmse_q_all + static_cast<size_t>(var) * Nq;
  double e[kHalf] = {};
  for (int bi = 0; bi < blocks_per_unit; ++bi) {
    const int blk = u * blocks_per_unit + bi;
    __syncthreads();
    for (int idx = threadIdx.x; idx < QW * bdim; idx += 256) {
      const int qq = idx / bdim, i = idx - qq * bdim;
      float v = 0.0f;
      if (qq < nq) {
        const size_t xo = static_cast<size_t>(q0 + qq) * Hq * D + static_cast<size_t>(blk) * bdim + i;
        v = x0 ? x1[xo] - x0[xo] : x1[xo];
      }
      xs[idx] = v;
    }
    __syncthreads();
    const float *gb = g + static_cast<size_t>(blk) * bdim * bdim;
    const float *xq = xs + kHalf * qh * bdim;
    for (int r = r0; r < bdim; r += 128) {
      float t[kHalf] = {};
#pragma unroll 8
      for (int cc = 0; cc < bdim; ++cc) {
        const float gv = gb[static_cast<size_t>(cc) * bdim + r];
#pragma unroll
        for (int j = 0; j < kHalf; ++j) t[j] += gv * xq[j * bdim + cc];
      }
#pragma unroll
      for (int j = 0; j < kHalf; ++j) e[j] += static_cast<double>(xq[j * bdim + r]) * t[j];
    }
  }
  // sum over the 128 threads of each half (two waves each)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kHalf; ++j) {
    double v = e[j];
    for (int o = 32; o > 0; o >>= 1) v += lane_xor(v, o);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (threadIdx.x < nq) {
    const int h2 = threadIdx.x / kHalf, j = threadIdx.x % kHalf;
    const double tot = red[2 * h2][j] + red[2 * h2 + 1][j];
    const int q = q0 + threadIdx.x;
    if constexpr (kDen)
      den[static_cast<size_t>(u) * Nq + q] = tot;
    else
      nmse_q[static_cast<size_t>(u) * stride_u + q] = static_cast<float>(tot / den[static_cast<size_t>(u) * Nq + q]);
  }
  }
}

// x1 holds nvar variants [nvar][Nq][Hq][128]; variant v writes nmse_q + v * Nq.
template <bool kDen>
hipError_t launch_quadform(const float *x1, const float *x0, const float *g, int Hq, int pu, int bdim, int U,
                           double *den, float *nmse_q, size_t stride_u, int Nq, int nvar, hipStream_t stream) {
  constexpr size_t kLds = 64 * 1024;
  const size_t row = sizeof(float) * bdim;
  const unsigned gz = static_cast<unsigned>(nvar < 65535 ? nvar : 65535);
  if (16 * row <= kLds)
    hipLaunchKernelGGL((quadform_kernel<kDen, 16>), dim3((Nq + 15) / 16, U, gz), dim3(256), 16 * row, stream, x1, x0,
                       g, Hq, pu, bdim, den, nmse_q, stride_u, Nq, nvar);
  else if (4 * row <= kLds)
    hipLaunchKernelGGL((quadform_kernel<kDen, 4>), dim3((Nq + 3) / 4, U, gz), dim3(256), 4 * row, stream, x1, x0, g,
                       Hq, pu, bdim, den, nmse_q, stride_u, Nq, nvar);
  else if (2 * row <= kLds)
    hipLaunchKernelGGL((quadform_kernel<kDen, 2>), dim3((Nq + 1) / 2, U, gz), dim3(256), 2 * row, stream, x1, x0, g,
                       Hq, pu, bdim, den, nmse_q, stride_u, Nq, nvar);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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

// Block geometry of the NMSE unit: PER_HEAD blocks of 128 (one per query
// head, G per unit), JOINT one block of Hq * 128.
static void nmse_blocks(int Hq, int H, int mode, int &bdim, int &nblocks, int &per_unit) {
  if (mode == KVQ_SELECT_JOINT) {
    bdim = Hq * D;
    nblocks = 1;
    per_unit = 1;
  } else {
    bdim = D;
    nblocks = Hq;
    per_unit = Hq / H;
  }
}

size_t nmse_gram_floats(int Hq, int H, int mode) {
  int bdim, nb, pu;
  nmse_blocks(Hq, H, mode, bdim, nb, pu);
  return static_cast<size_t>(nb) * bdim * bdim;
}

hipError_t launch_nmse_prepare(const float *o_ref, const void *w_o, int dtype, int Nq, int Hq, int H, int d_model,
                               int mode, float *gram, double *den, hipStream_t stream) {
  int bdim, nb, pu;
  nmse_blocks(Hq, H, mode, bdim, nb, pu);
  const dim3 ggrid((bdim / 64) * (bdim / 64), nb);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(gram_kernel<KVQ_F32>, ggrid, dim3(256), 0, stream, w_o, d_model, bdim, gram);
  else
    hipLaunchKernelGGL(gram_kernel<KVQ_BF16>, ggrid, dim3(256), 0, stream, w_o, d_model, bdim, gram);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int U = (mode == KVQ_SELECT_JOINT) ? 1 : H;
  return launch_quadform<true>(o_ref, nullptr, gram, Hq, pu, bdim, U, den, nullptr, size_t{0}, Nq, 1, stream);
}

hipError_t launch_nmse_terms(const float *o_hat, const float *o_ref, const float *gram, const double *den, int Nq,
                             int Hq, int H, int mode, int nvar, float *nmse_q_out, size_t stride_u,
                             hipStream_t stream) {
  int bdim, nb, pu;
  nmse_blocks(Hq, H, mode, bdim, nb, pu);
  const int U = (mode == KVQ_SELECT_JOINT) ? 1 : H;
  return launch_quadform<false>(o_hat, o_ref, gram, Hq, pu, bdim, U, const_cast<double *>(den), nmse_q_out, stride_u,
                                Nq, nvar, stream);
}

hipError_t launch_select(const float *nmse_q, int U, int C, int n_clip, int Nq, float *out_nmse, int32_t *out_best,
                         hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(U), dim3(256), 0, stream, nmse_q, C, n_clip, Nq, out_nmse, out_best);
  return hipGetLastError();
}

}  // namespace kvq
