// optr.hip -- OptR offline calibration on the GPU ("Output-Aware Rotation for
// INT2 KV-Cache Quantization": §4.1-§4.5, Eq. (11)-(18); Appendix "OptR
// Algorithm", Algorithm 1; Appendix calibration details and Table A).
//
// For every KV head: the key mean of the calibration traces; then the key
// rotation R_K = R0_K exp(A - A^T) learned by Adam on
//   L_K = mean_(t,j) KL(p_t || p_t^K) + lambda_K ||e_K(t,j)||^2 / d_model
// (Eq. (12)-(14)) with the held-out objective checked every eval_every steps
// (the first minimum is kept); then the value rotation under the selected key
// attention, on L_V = mean ||e_V||^2 / d_model (Eq. (15)-(16)).  Gradients pass
// the INT2 quantizer by the straight-through estimator of Eq. (18): identity
// where a value lies inside its group's clipping range [c min, c max], zero
// outside.  Sink and recent window tokens stay unquantized (keys centered).
//
// Arithmetic: fp64 throughout (the calibration is a one-time, small
// contraction workload, and MI355X runs fp64 at the same peak on its vector
// units as on its matrix cores), except the INT2 quantizer, which follows the
// library's fp32 step sequence on the rotated values rounded to fp32.
//
// Layout (workspace, per trace set): keys centered and values widened to
// fp64, head-major [H][num_seqs][max_len][128] (zero past each length);
// queries [H][num_seqs][G][nq][128] (row r = g nq + t: query head h G + g at
// the t-th of the final nq positions); logits and probabilities
// [H][num_seqs][G nq][max_len].  Generators, Adam moments and rotations are
// [H][128][128].
#include <algorithm>
#include <cmath>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxTraceSeqs = 64;
constexpr int kTaylor = 13;       // Taylor degree of exp on ||X||_1 <= 1/2: remainder < 1e-15
constexpr double kTheta = 0.5;

// ---------------------------------------------------------------- batched fp64 GEMM
// C(i,j) = alpha sum_k A(i,k) B(k,j) + beta C(i,j) for every batch index z,
// with A(i,k) = A[i ars + k acs], B(k,j) = B[k brs + j bcs], C(i,j) = C[i crs + j]
// and operand offsets (z / div) s1 + (z % mod) s2.  beta == 0 never reads C.
struct G64 {
  const double *A, *B;
  double *C;
  int M, N, K;
  int64_t ars, acs, brs, bcs, crs;
  int64_t as1, as2, bs1, bs2, cs1, cs2;
  int adiv, amod, bdiv, bmod, cdiv, cmod;
  double alpha, beta;
};

G64 gemm(const double *A, int64_t ars, int64_t acs, const double *B, int64_t brs, int64_t bcs, double *C,
         int64_t crs, int M, int N, int K, double alpha = 1.0, double beta = 0.0) {
  G64 g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ars = ars;
  g.acs = acs;
  g.brs = brs;
  g.bcs = bcs;
  g.crs = crs;
  g.adiv = g.bdiv = g.cdiv = 1;
  g.amod = g.bmod = g.cmod = 1;
  g.alpha = alpha;
  g.beta = beta;
  return g;
}

constexpr int kGT = 64, kGK = 16;

__global__ __launch_bounds__(256) void gemm64_kernel(G64 g) {
  __shared__ double as[kGK][kGT + 1];
  __shared__ double bs[kGK][kGT + 1];
  const int z = blockIdx.z;
  const double *A = g.A + static_cast<int64_t>(z / g.adiv) * g.as1 + static_cast<int64_t>(z % g.amod) * g.as2;
  const double *B = g.B + static_cast<int64_t>(z / g.bdiv) * g.bs1 + static_cast<int64_t>(z % g.bmod) * g.bs2;
  double *C = g.C + static_cast<int64_t>(z / g.cdiv) * g.cs1 + static_cast<int64_t>(z % g.cmod) * g.cs2;
  const int m0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  const bool a_kfast = g.acs == 1, b_jfast = g.bcs == 1;
  for (int k0 = 0; k0 < g.K; k0 += kGK) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = tid + 256 * p;
      const int ia = a_kfast ? e >> 4 : e & 63, ka = a_kfast ? e & 15 : e >> 6;
      const int gi = m0 + ia, gk = k0 + ka;
      as[ka][ia] = (gi < g.M && gk < g.K) ? A[gi * g.ars + gk * g.acs] : 0.0;
      const int kb = b_jfast ? e >> 6 : e & 15, jb = b_jfast ? e & 63 : e >> 4;
      const int gj = n0 + jb, gk2 = k0 + kb;
      bs[kb][jb] = (gj < g.N && gk2 < g.K) ? B[gk2 * g.brs + gj * g.bcs] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kGK; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = as[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = bs[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gi = m0 + ty + 16 * i, gj = n0 + tx + 16 * j;
      if (gi < g.M && gj < g.N) {
        double *c = C + gi * g.crs + gj;
        *c = g.beta != 0.0 ? g.alpha * acc[i][j] + g.beta * *c : g.alpha * acc[i][j];
      }
    }
}

hipError_t run_gemm(const G64 &g, int batch, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  const dim3 grid((g.N + kGT - 1) / kGT, (g.M + kGT - 1) / kGT, batch);
  hipLaunchKernelGGL(gemm64_kernel, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------- exp and its Frechet adjoint
// One workgroup (512 threads) per KV head; 128 x 128 fp64 matrices in global
// memory (L2-resident), K-slices staged in LDS.

constexpr int kExT = 512;  // threads of the exponential kernels

// C = alpha (A B [+ A2 B2]) [+ I]; C distinct from the inputs.  Thread
// (ty, tx) computes rows ty + 16 i (i < 8) and columns tx + 32 j (j < 4).
__device__ void wg_mm(const double *A, const double *B, const double *A2, const double *B2, double *C, double alpha,
                      bool add_identity, double (*sa)[D], double (*sb)[D]) {
  const int tid = threadIdx.x, tx = tid & 31, ty = tid >> 5;
  double acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int pass = 0; pass < (A2 ? 2 : 1); ++pass) {
    const double *a = pass ? A2 : A, *b = pass ? B2 : B;
    for (int k0 = 0; k0 < D; k0 += kGK) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e = tid + kExT * p;
        sa[e & 15][e >> 4] = a[(e >> 4) * D + k0 + (e & 15)];
        sb[e >> 7][e & 127] = b[(k0 + (e >> 7)) * D + (e & 127)];
      }
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < kGK; ++k) {
        double x[8], y[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sa[k][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = sb[k][tx + 32 * j];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fma(x[i], y[j], acc[i][j]);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty + 16 * i, c = tx + 32 * j;
      C[r * D + c] = alpha * acc[i][j] + ((add_identity && r == c) ? 1.0 : 0.0);
    }
  __syncthreads();
}

// max over columns of sum_i |X[i][j]| (the matrix 1-norm), every thread gets it
__device__ double wg_norm1(const double *X, double *red) {
  const int tid = threadIdx.x;
  double s = 0.0;
  if (tid < D)
    for (int i = 0; i < D; ++i) s += fabs(X[i * D + tid]);
  red[tid] = tid < D ? s : 0.0;
  __syncthreads();
  for (int w = kExT / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmax(red[tid], red[tid + w]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ int squarings(double norm) {
  int s = 0;
  while (norm > kTheta && s < 60) {
    norm *= 0.5;
    ++s;
  }
  return s;
}

// S = A - A^T and E = exp(S) by scaling and squaring with a degree-13
// Taylor polynomial (Horner); scratch: 3 matrices per head.
__global__ __launch_bounds__(kExT) void expm_kernel(const double *A_all, double *S_all, double *E_all,
                                                   double *scratch) {
  __shared__ double sa[kGK][D];
  __shared__ double sb[kGK][D];
  __shared__ double red[kExT];
  if (blockDim.x != kExT) return;   // (the thread mapping below assumes kExT threads)
  const int h = blockIdx.x;
  const double *A = A_all + static_cast<size_t>(h) * D * D;
  double *S = S_all + static_cast<size_t>(h) * D * D;
  double *X = scratch + static_cast<size_t>(h) * 3 * D * D, *P = X + D * D, *T = P + D * D;
  for (int e = threadIdx.x; e < D * D; e += kExT) S[e] = A[e] - A[(e % D) * D + e / D];
  __syncthreads();
  const int s = squarings(wg_norm1(S, red));
  const double sc = ldexp(1.0, -s);
  for (int e = threadIdx.x; e < D * D; e += kExT) {
    X[e] = S[e] * sc;
    P[e] = (e % D == e / D) ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int k = kTaylor; k >= 1; --k) {   // P <- I + X P / k
    wg_mm(X, P, nullptr, nullptr, T, 1.0 / k, true, sa, sb);
    double *t = P;
    P = T;
    T = t;
  }
  for (int i = 0; i < s; ++i) {
    wg_mm(P, P, nullptr, nullptr, T, 1.0, false, sa, sb);
    double *t = P;
    P = T;
    T = t;
  }
  double *E = E_all + static_cast<size_t>(h) * D * D;
  for (int e = threadIdx.x; e < D * D; e += kExT) E[e] = P[e];
}

// out = L(S^T, G): the Frechet derivative of exp at S^T in the direction G,
// which is the adjoint of the Frechet derivative at S (the chain rule of
// exp(S) for a scalar loss: dL/dS = L(S^T, dL/dE)).  exp of the block matrix
// [[X, G], [0, X]] is [[exp X, L(X, G)], [0, exp X]]; the pair (P, Q) stands
// for [[P, Q], [0, P]].  G is scaled to unit 1-norm first (L is linear in G).
__global__ __launch_bounds__(kExT) void expm_frechet_kernel(const double *S_all, const double *G_all, double *out_all,
                                                           double *scratch) {
  __shared__ double sa[kGK][D];
  __shared__ double sb[kGK][D];
  __shared__ double red[kExT];
  if (blockDim.x != kExT) return;   // (the thread mapping below assumes kExT threads)
  const int h = blockIdx.x;
  const double *S = S_all + static_cast<size_t>(h) * D * D;
  const double *Gin = G_all + static_cast<size_t>(h) * D * D;
  double *out = out_all + static_cast<size_t>(h) * D * D;
  double *X = scratch + static_cast<size_t>(h) * 7 * D * D;
  double *Gs = X + D * D, *P = Gs + D * D, *Q = P + D * D, *P2 = Q + D * D, *Q2 = P2 + D * D, *Xt = Q2 + D * D;
  for (int e = threadIdx.x; e < D * D; e += kExT) Xt[e] = S[(e % D) * D + e / D];   // S^T
  __syncthreads();
  const double gn = wg_norm1(Gin, red);
  if (gn == 0.0) {
    for (int e = threadIdx.x; e < D * D; e += kExT) out[e] = 0.0;
    return;
  }
  const int s = squarings(wg_norm1(Xt, red) + 1.0);
  const double sc = ldexp(1.0, -s);
  for (int e = threadIdx.x; e < D * D; e += kExT) {
    X[e] = Xt[e] * sc;
    Gs[e] = Gin[e] / gn * sc;
    P[e] = (e % D == e / D) ? 1.0 : 0.0;
    Q[e] = 0.0;
  }
  __syncthreads();
  for (int k = kTaylor; k >= 1; --k) {   // (P, Q) <- (I + X P / k, (X Q + G P) / k)
    wg_mm(X, Q, Gs, P, Q2, 1.0 / k, false, sa, sb);
    wg_mm(X, P, nullptr, nullptr, P2, 1.0 / k, true, sa, sb);
    double *t = P;
    P = P2;
    P2 = t;
    t = Q;
    Q = Q2;
    Q2 = t;
  }
  for (int i = 0; i < s; ++i) {           // (P, Q) <- (P P, P Q + Q P)
    wg_mm(P, Q, Q, P, Q2, 1.0, false, sa, sb);
    wg_mm(P, P, nullptr, nullptr, P2, 1.0, false, sa, sb);
    double *t = P;
    P = P2;
    P2 = t;
    t = Q;
    Q = Q2;
    Q2 = t;
  }
  for (int e = threadIdx.x; e < D * D; e += kExT) out[e] = Q[e] * gn;
}

// ---------------------------------------------------------------- trace preparation
struct SeqLens {
  int n;
  int lens[kMaxTraceSeqs];
};

template <int DT>
__device__ __forceinline__ double ld64(const void *p, size_t i) {
  return static_cast<double>(load_elem<DT>(p, i));
}

// Per-KV-head mean of every cached key of the set, fp64 sums in (sequence,
// position) order, rounded to fp32 (out) and kept in fp64 (mu64).
template <int DT>
__global__ __launch_bounds__(D) void key_mean_kernel(const void *k, int Lm, int H, SeqLens sl, float *out,
                                                     double *mu64) {
  const int h = blockIdx.x, i = threadIdx.x;
  double s = 0.0;
  int64_t n = 0;
  for (int b = 0; b < sl.n; ++b) {
    for (int t = 0; t < sl.lens[b]; ++t) s += ld64<DT>(k, ((static_cast<size_t>(b) * Lm + t) * H + h) * D + i);
    n += sl.lens[b];
  }
  const float m = static_cast<float>(s / static_cast<double>(n));
  if (out) out[h * D + i] = m;
  mu64[h * D + i] = static_cast<double>(m);
}

// Keys centered (mu64 may be null) and values widened to fp64, head-major,
// zero past each length; queries reordered to [H][num_seqs][G][nq][128].
template <int DT>
__global__ __launch_bounds__(256) void prep_kernel(const void *k, const void *v, const void *q, int Lm, int H, int G,
                                                   int nq, SeqLens sl, const double *mu64, double *Kc, double *V,
                                                   double *Q) {
  const int b = blockIdx.y, h = blockIdx.z;
  const int Hq = H * G;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < Lm * D; e += gridDim.x * 256) {
    const int t = e / D, i = e % D;
    const size_t dst = ((static_cast<size_t>(h) * sl.n + b) * Lm + t) * D + i;
    if (t < sl.lens[b]) {
      const size_t src = ((static_cast<size_t>(b) * Lm + t) * H + h) * D + i;
      Kc[dst] = ld64<DT>(k, src) - (mu64 ? mu64[h * D + i] : 0.0);
      V[dst] = ld64<DT>(v, src);
    } else {
      Kc[dst] = 0.0;
      V[dst] = 0.0;
    }
  }
  for (int e = blockIdx.x * 256 + threadIdx.x; e < G * nq * D; e += gridDim.x * 256) {
    const int g = e / (nq * D), t = (e / D) % nq, i = e % D;
    Q[((static_cast<size_t>(h) * sl.n + b) * G * nq + g * nq + t) * D + i] =
        ld64<DT>(q, ((static_cast<size_t>(b) * nq + t) * Hq + h * G + g) * D + i);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void widen_kernel(const void *x, size_t n, double *y) {
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256)
    y[e] = ld64<DT>(x, e);
}

__global__ __launch_bounds__(256) void widen_f32_kernel(const float *x, size_t n, double *y) {
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256)
    y[e] = static_cast<double>(x[e]);
}

__global__ __launch_bounds__(256) void narrow_kernel(const double *x, size_t n, float *y) {
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256)
    y[e] = static_cast<float>(x[e]);
}

// ---------------------------------------------------------------- quantizer with straight-through flags
__device__ __forceinline__ float wmin(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, lane_xor(x, o));
  return x;
}
__device__ __forceinline__ float wmax(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, lane_xor(x, o));
  return x;
}

// One wave per token row (h, b, t).  INT2 positions [lo, hi): the fp32
// rotated value is quantized in the library's fp32 order and dequantized
// (code s + z), flag = 1 inside the group's clipping range [c min, c max].
// Window positions: keys pass through (flag 1), values give 0 (flag 0: the
// window values are kept exactly, so they carry no error).  Past the length: 0.
__global__ __launch_bounds__(256) void quant_ste_kernel(const double *Z, double *out, uint8_t *flag, int H, int Lm,
                                                        SeqLens sl, int num_sink, int num_recent, float clip,
                                                        int keys) {
#pragma clang fp contract(off)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  const int64_t rows = static_cast<int64_t>(H) * sl.n * Lm;
  if (row >= rows) return;
  const int t = static_cast<int>(row % Lm), b = static_cast<int>((row / Lm) % sl.n);
  const int L = sl.lens[b];
  const int lo_w = min(num_sink, L), hi_w = max(lo_w, L - num_recent);
  const double *z = Z + row * D;
  double *o = out + row * D;
  uint8_t *f = flag + row * D;
  if (t >= L) {
    o[lane] = o[lane + 64] = 0.0;
    f[lane] = f[lane + 64] = 0;
    return;
  }
  if (t < lo_w || t >= hi_w) {
    o[lane] = keys ? z[lane] : 0.0;
    o[lane + 64] = keys ? z[lane + 64] : 0.0;
    f[lane] = f[lane + 64] = keys ? 1 : 0;
    return;
  }
  const float x0 = static_cast<float>(z[lane]), x1 = static_cast<float>(z[lane + 64]);
  const float mn = wmin(fminf(x0, x1)), mx = wmax(fmaxf(x0, x1));
  float lo = clip * mn;
  const float hi = clip * mx;
  const float span = hi - lo;
  float s32 = span / 3.0f;
  asm volatile("" : "+v"(lo));   // (each rounded to fp32 before the fp16 conversion)
  asm volatile("" : "+v"(s32));
  const float s = static_cast<float>(static_cast<_Float16>(s32));
  const float zz = static_cast<float>(static_cast<_Float16>(lo));
  float c0 = 0.0f, c1 = 0.0f;
  if (s != 0.0f) {
    const float inv = 1.0f / s;
    const float d0 = x0 - zz, d1 = x1 - zz;
    const float t0 = d0 * inv, t1 = d1 * inv;
    c0 = fminf(fmaxf(__builtin_rintf(t0), 0.0f), 3.0f);
    c1 = fminf(fmaxf(__builtin_rintf(t1), 0.0f), 3.0f);
  }
  const float p0 = c0 * s, p1 = c1 * s;   // exact
  o[lane] = static_cast<double>(p0 + zz);
  o[lane + 64] = static_cast<double>(p1 + zz);
  f[lane] = (x0 >= lo && x0 <= hi) ? 1 : 0;
  f[lane + 64] = (x1 >= lo && x1 <= hi) ? 1 : 0;
}

__global__ __launch_bounds__(256) void mask_mul_kernel(double *x, const uint8_t *flag, size_t n) {
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256)
    if (!flag[e]) x[e] = 0.0;
}

// ---------------------------------------------------------------- softmax rows
// Row r of (h, b): query position t = r % nq of the final nq attends
// positions s < n = len - nq + t + 1.
__device__ __forceinline__ int row_len(int r, int nq, int L) { return L - nq + (r % nq) + 1; }

__device__ __forceinline__ double block_reduce(double x, double *red, bool is_max) {
  const int tid = threadIdx.x;
  red[tid] = x;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = is_max ? fmax(red[tid], red[tid + w]) : red[tid] + red[tid + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// logits -> p^K in place; delta = p^K - p (reference p from ref_logits);
// kl[row] = sum_s p (log p - log p^K).  With ref_logits null only p^K.
__global__ __launch_bounds__(256) void softmax_fwd_kernel(double *logits, const double *ref_logits, double *delta,
                                                          double *kl, int RQ, int Lm, int nq, SeqLens sl) {
  __shared__ double red[256];
  const int64_t row = blockIdx.x;
  const int r = static_cast<int>(row % RQ), b = static_cast<int>((row / RQ) % sl.n);
  const int n = row_len(r, nq, sl.lens[b]);
  double *a = logits + row * Lm;
  const double *ar = ref_logits ? ref_logits + row * Lm : nullptr;
  double m = -INFINITY, mr = -INFINITY;
  for (int s = threadIdx.x; s < n; s += 256) {
    m = fmax(m, a[s]);
    if (ar) mr = fmax(mr, ar[s]);
  }
  m = block_reduce(m, red, true);
  if (ar) mr = block_reduce(mr, red, true);
  double z = 0.0, zr = 0.0;
  for (int s = threadIdx.x; s < n; s += 256) {
    z += exp(a[s] - m);
    if (ar) zr += exp(ar[s] - mr);
  }
  const double lse = m + log(block_reduce(z, red, false));
  const double lser = ar ? mr + log(block_reduce(zr, red, false)) : 0.0;
  double k = 0.0;
  for (int s = threadIdx.x; s < Lm; s += 256) {
    if (s < n) {
      const double lp = a[s] - lse;
      const double pk = exp(lp);
      a[s] = pk;
      if (ar) {
        const double lq = ar[s] - lser;
        const double p = exp(lq);
        delta[row * Lm + s] = pk - p;
        k += p * (lq - lp);
      }
    } else {
      a[s] = 0.0;
      if (ar) delta[row * Lm + s] = 0.0;
    }
  }
  if (ar) {
    k = block_reduce(k, red, false);
    if (threadIdx.x == 0) kl[row] = k;
  }
}

// g -> dL/dlogits in place: p^K (g - sum_s p^K g) + kl_coef (p^K - p)
__global__ __launch_bounds__(256) void softmax_bwd_kernel(double *g, const double *pk, const double *delta,
                                                          double kl_coef, int RQ, int Lm, int nq, SeqLens sl) {
  __shared__ double red[256];
  const int64_t row = blockIdx.x;
  const int r = static_cast<int>(row % RQ), b = static_cast<int>((row / RQ) % sl.n);
  const int n = row_len(r, nq, sl.lens[b]);
  double *gr = g + row * Lm;
  const double *p = pk + row * Lm, *d = delta + row * Lm;
  double s0 = 0.0;
  for (int s = threadIdx.x; s < n; s += 256) s0 += p[s] * gr[s];
  s0 = block_reduce(s0, red, false);
  for (int s = threadIdx.x; s < Lm; s += 256) gr[s] = s < n ? p[s] * (gr[s] - s0) + kl_coef * d[s] : 0.0;
}

// p_hat restricted to the INT2 positions of each sequence (value phase)
__global__ __launch_bounds__(256) void int2_restrict_kernel(double *p, int RQ, int Lm, SeqLens sl, int num_sink,
                                                            int num_recent) {
  const int64_t row = blockIdx.x;
  const int b = static_cast<int>((row / RQ) % sl.n);
  const int L = sl.lens[b];
  const int lo = min(num_sink, L), hi = max(lo, L - num_recent);
  for (int s = threadIdx.x; s < Lm; s += 256)
    if (s < lo || s >= hi) p[row * Lm + s] = 0.0;
}

// e2[row] = x . xg / d_model; xg <- coef xg (= dL/dx)
__global__ __launch_bounds__(256) void err_rows_kernel(const double *x, double *xg, double *e2, int64_t rows,
                                                       double inv_dm, double coef) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  const double *a = x + row * D;
  double *c = xg + row * D;
  double s = a[lane] * c[lane] + a[lane + 64] * c[lane + 64];
  for (int o = 32; o > 0; o >>= 1) s += lane_xor(s, o);
  if (lane == 0) e2[row] = s * inv_dm;
  c[lane] *= coef;
  c[lane + 64] *= coef;
}

// loss[h] = (sum kl + lambda sum e2) / rows_per_head, fixed summation order;
// written to log_out[h * log_stride] too when given
__global__ __launch_bounds__(256) void loss_kernel(const double *kl, const double *e2, int64_t rows_per_head,
                                                   double lambda, double *loss, double *log_out, int64_t log_stride) {
  __shared__ double red[256];
  const int h = blockIdx.x;
  double s = 0.0;
  for (int64_t r = threadIdx.x; r < rows_per_head; r += 256) {
    const int64_t i = h * rows_per_head + r;
    s += (kl ? kl[i] : 0.0) + lambda * e2[i];
  }
  s = block_reduce(s, red, false) / static_cast<double>(rows_per_head);
  if (threadIdx.x == 0) {
    loss[h] = s;
    if (log_out) log_out[h * log_stride] = s;
  }
}

// Adam (Kingma and Ba) on A with the gradient g = dS - dS^T, in the form
// m <- m + (1 - b1) (g - m); v <- b2 v + (1 - b2) g g;
// A <- A - (lr / bc1) m / (sqrt(v) / sqrt(bc2) + eps)
__global__ __launch_bounds__(256) void adam_kernel(double *A, double *m, double *v, const double *dS, double lr,
                                                   double bc1, double bc2_sqrt, int H) {
  const double b1 = 0.9, b2 = 0.999, eps = 1e-8;
  const size_t n = static_cast<size_t>(H) * D * D;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256) {
    const size_t h = e / (D * D), ij = e % (D * D), i = ij / D, j = ij % D;
    const double g = dS[e] - dS[h * D * D + j * D + i];
    const double mm = m[e] + (1.0 - b1) * (g - m[e]);
    const double vv = v[e] * b2 + (1.0 - b2) * g * g;
    m[e] = mm;
    v[e] = vv;
    A[e] = A[e] - (lr / bc1) * (mm / (sqrt(vv) / bc2_sqrt + eps));
  }
}

// held-out checkpoint: keep the first minimum
__global__ __launch_bounds__(256) void checkpoint_kernel(const double *loss, double *best, const double *A, double *Abest,
                                                         int step, double *log_held, int64_t log_stride,
                                                         double *log_sel) {
  const int h = blockIdx.x;
  const double l = loss[h];
  const bool take = !(best[h] <= l);   // (best starts at NaN: the first checkpoint is taken)
  __syncthreads();
  if (take)
    for (int e = threadIdx.x; e < D * D; e += 256) Abest[static_cast<size_t>(h) * D * D + e] = A[static_cast<size_t>(h) * D * D + e];
  if (threadIdx.x == 0) {
    if (take) {
      best[h] = l;
      if (log_sel) log_sel[h * log_stride] = step;
    }
    if (log_held) log_held[h * log_stride] = l;
  }
}

// out = dS - dS^T per head (the gradient in A of a loss of S = A - A^T)
__global__ __launch_bounds__(256) void antisym_kernel(const double *dS, double *out, int H) {
  const size_t n = static_cast<size_t>(H) * D * D;
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256) {
    const size_t h = e / (D * D), ij = e % (D * D), i = ij / D, j = ij % D;
    out[e] = dS[e] - dS[h * D * D + j * D + i];
  }
}

__global__ __launch_bounds__(256) void fill_kernel(double *x, size_t n, double value) {
  for (size_t e = blockIdx.x * 256 + threadIdx.x; e < n; e += static_cast<size_t>(gridDim.x) * 256) x[e] = value;
}

int blocks_for(size_t n) {
  const size_t b = (n + 255) / 256;
  return static_cast<int>(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

// ---------------------------------------------------------------- host side
struct SetDev {
  SeqLens sl;
  int Lm;
  double *Kc, *V, *Q, *Lref, *Phat, *Cv;
};

struct Layout {
  size_t total;
  size_t set_off[2][6];  // Kc, V, Q, Lref, Phat, Cv
  size_t Z, Xt, flag, Qr, P, Dl, Gm, X, XG, dQ, dK, kl, e2;
  size_t A, Am, Av, Ab, S, E, R, R0k, R0v, Rk_hat, dR, dE, dS, ex, fr, gamma, w64, mu64, loss, best;
};

struct Shape {
  int H, G, nq, d_model;
  int ns[2], lm[2];
};

Layout layout(const Shape &s) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  const size_t RQ = static_cast<size_t>(s.G) * s.nq;
  size_t tok_max = 0, row_max = 0, lg_max = 0;
  for (int i = 0; i < 2; ++i) {
    const size_t tok = static_cast<size_t>(s.H) * s.ns[i] * s.lm[i];
    const size_t rows = static_cast<size_t>(s.H) * s.ns[i] * RQ;
    L.set_off[i][0] = take(tok * D * 8);
    L.set_off[i][1] = take(tok * D * 8);
    L.set_off[i][2] = take(rows * D * 8);
    L.set_off[i][3] = take(rows * s.lm[i] * 8);
    L.set_off[i][4] = take(rows * s.lm[i] * 8);
    L.set_off[i][5] = take(rows * D * 8);
    tok_max = std::max(tok_max, tok);
    row_max = std::max(row_max, rows);
    lg_max = std::max(lg_max, rows * s.lm[i]);
  }
  L.Z = take(tok_max * D * 8);
  L.Xt = take(tok_max * D * 8);
  L.flag = take(tok_max * D);
  L.dK = take(tok_max * D * 8);
  L.Qr = take(row_max * D * 8);
  L.X = take(row_max * D * 8);
  L.XG = take(row_max * D * 8);
  L.dQ = take(row_max * D * 8);
  L.kl = take(row_max * 8);
  L.e2 = take(row_max * 8);
  L.P = take(lg_max * 8);
  L.Dl = take(lg_max * 8);
  L.Gm = take(lg_max * 8);
  const size_t mat = static_cast<size_t>(s.H) * D * D * 8;
  L.A = take(mat);
  L.Am = take(mat);
  L.Av = take(mat);
  L.Ab = take(mat);
  L.S = take(mat);
  L.E = take(mat);
  L.R = take(mat);
  L.R0k = take(mat);
  L.R0v = take(mat);
  L.Rk_hat = take(mat);
  L.dR = take(mat);
  L.dE = take(mat);
  L.dS = take(mat);
  L.ex = take(3 * mat);
  L.fr = take(7 * mat);
  L.gamma = take(static_cast<size_t>(s.H) * s.G * D * D * 8);
  L.w64 = take(static_cast<size_t>(s.H) * s.G * D * s.d_model * 8);
  L.mu64 = take(static_cast<size_t>(s.H) * D * 8);
  L.loss = take(static_cast<size_t>(s.H) * 8);
  L.best = take(static_cast<size_t>(s.H) * 8);
  L.total = off;
  return L;
}

#define OPTR_TRY(expr)                        \
  do {                                        \
    const hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return e_;          \
  } while (0)

struct Ctx {
  Shape sh;
  Layout L;
  uint8_t *ws;
  const kvq_optr_config *cfg;
  hipStream_t st;
  SetDev set[2];
  double *p(size_t off) const { return reinterpret_cast<double *>(ws + off); }
};

// R = R0 exp(A - A^T) of every head (S and E kept)
hipError_t rotation_of(Ctx &c, const double *A, const double *R0, double *R) {
  const int H = c.sh.H;
  hipLaunchKernelGGL(expm_kernel, dim3(H), dim3(kExT), 0, c.st, A, c.p(c.L.S), c.p(c.L.E), c.p(c.L.ex));
  OPTR_TRY(hipGetLastError());
  G64 g = gemm(R0, D, 1, c.p(c.L.E), D, 1, R, D, D, D, D);
  g.as1 = g.bs1 = g.cs1 = D * D;
  return run_gemm(g, H, c.st);
}

// Forward of the key objective on set si at rotation R: p^K (in P), delta,
// kl, x, e2 and dx (in XG); loss per head into loss (and log_out).
hipError_t key_forward(Ctx &c, int si, const double *R, double *log_out, int64_t log_stride, bool only_pk = false) {
  const SetDev &sd = c.set[si];
  const int H = c.sh.H, NS = sd.sl.n, Lm = sd.Lm, G = c.sh.G, nq = c.sh.nq, RQ = G * nq;
  const int64_t toks = static_cast<int64_t>(NS) * Lm;
  // Z = Kc R (per head: NS Lm rows)
  G64 g = gemm(sd.Kc, D, 1, R, D, 1, c.p(c.L.Z), D, static_cast<int>(toks), D, D);
  g.as1 = g.cs1 = toks * D;
  g.bs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  const int64_t rows_tok = H * toks;
  hipLaunchKernelGGL(quant_ste_kernel, dim3(static_cast<unsigned>((rows_tok + 3) / 4)), dim3(256), 0, c.st,
                     c.p(c.L.Z), c.p(c.L.Xt), c.ws + c.L.flag, H, Lm, sd.sl, c.cfg->num_sink, c.cfg->num_recent,
                     c.cfg->clip_k, 1);
  OPTR_TRY(hipGetLastError());
  // Qr = Q R
  g = gemm(sd.Q, D, 1, R, D, 1, c.p(c.L.Qr), D, NS * RQ, D, D);
  g.as1 = g.cs1 = static_cast<int64_t>(NS) * RQ * D;
  g.bs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  // logits = Qr Kt^T / sqrt(d), batch (h, b)
  g = gemm(c.p(c.L.Qr), D, 1, c.p(c.L.Xt), 1, D, c.p(c.L.P), Lm, RQ, Lm, D, 1.0 / std::sqrt(static_cast<double>(D)));
  g.as1 = static_cast<int64_t>(RQ) * D;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * Lm;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  const int64_t rows = static_cast<int64_t>(H) * NS * RQ;
  hipLaunchKernelGGL(softmax_fwd_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, c.st, c.p(c.L.P),
                     only_pk ? nullptr : sd.Lref, c.p(c.L.Dl), c.p(c.L.kl), RQ, Lm, nq, sd.sl);
  OPTR_TRY(hipGetLastError());
  if (only_pk) return hipSuccess;
  // x = delta V, batch (h, b)
  g = gemm(c.p(c.L.Dl), Lm, 1, sd.V, D, 1, c.p(c.L.X), D, RQ, D, Lm);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * D;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  // XG = x_g Gamma_{hG+g}, batch ((h, b), g)
  g = gemm(c.p(c.L.X), D, 1, c.p(c.L.gamma), D, 1, c.p(c.L.XG), D, nq, D, D);
  g.as1 = g.cs1 = static_cast<int64_t>(nq) * D;
  g.bdiv = NS * G;
  g.bs1 = static_cast<int64_t>(G) * D * D;
  g.bmod = G;
  g.bs2 = D * D;
  OPTR_TRY(run_gemm(g, H * NS * G, c.st));
  const double N = static_cast<double>(NS) * RQ;
  const double lam = c.cfg->lambda_k;
  hipLaunchKernelGGL(err_rows_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, c.st, c.p(c.L.X),
                     c.p(c.L.XG), c.p(c.L.e2), rows, 1.0 / c.sh.d_model, 2.0 * lam / (N * c.sh.d_model));
  OPTR_TRY(hipGetLastError());
  hipLaunchKernelGGL(loss_kernel, dim3(H), dim3(256), 0, c.st, c.p(c.L.kl), c.p(c.L.e2),
                     static_cast<int64_t>(NS) * RQ, lam, c.p(c.L.loss), log_out, log_stride);
  return hipGetLastError();
}

// dR of the key objective (after key_forward on set 0)
hipError_t key_backward(Ctx &c) {
  const SetDev &sd = c.set[0];
  const int H = c.sh.H, NS = sd.sl.n, Lm = sd.Lm, RQ = c.sh.G * c.sh.nq;
  const int64_t toks = static_cast<int64_t>(NS) * Lm;
  const double N = static_cast<double>(NS) * RQ, isd = 1.0 / std::sqrt(static_cast<double>(D));
  // g = dx V^T, batch (h, b)
  G64 g = gemm(c.p(c.L.XG), D, 1, sd.V, 1, D, c.p(c.L.Gm), Lm, RQ, Lm, D);
  g.as1 = static_cast<int64_t>(RQ) * D;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * Lm;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  const int64_t rows = static_cast<int64_t>(H) * NS * RQ;
  hipLaunchKernelGGL(softmax_bwd_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, c.st, c.p(c.L.Gm),
                     c.p(c.L.P), c.p(c.L.Dl), 1.0 / N, RQ, Lm, c.sh.nq, sd.sl);
  OPTR_TRY(hipGetLastError());
  // dQr = da Kt / sqrt(d), batch (h, b)
  g = gemm(c.p(c.L.Gm), Lm, 1, c.p(c.L.Xt), D, 1, c.p(c.L.dQ), D, RQ, D, Lm, isd);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * D;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  // dKt = da^T Qr / sqrt(d), batch (h, b); then the straight-through flags
  g = gemm(c.p(c.L.Gm), 1, Lm, c.p(c.L.Qr), D, 1, c.p(c.L.dK), D, Lm, D, RQ, isd);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(RQ) * D;
  g.cs1 = static_cast<int64_t>(Lm) * D;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  const size_t n = static_cast<size_t>(H) * toks * D;
  hipLaunchKernelGGL(mask_mul_kernel, dim3(blocks_for(n)), dim3(256), 0, c.st, c.p(c.L.dK), c.ws + c.L.flag, n);
  OPTR_TRY(hipGetLastError());
  // dR = Kc^T dZ + Q^T dQr, batch h
  g = gemm(sd.Kc, 1, D, c.p(c.L.dK), D, 1, c.p(c.L.dR), D, D, D, static_cast<int>(toks));
  g.as1 = g.bs1 = toks * D;
  g.cs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  g = gemm(sd.Q, 1, D, c.p(c.L.dQ), D, 1, c.p(c.L.dR), D, D, D, NS * RQ, 1.0, 1.0);
  g.as1 = g.bs1 = static_cast<int64_t>(NS) * RQ * D;
  g.cs1 = D * D;
  return run_gemm(g, H, c.st);
}

// Forward of the value objective on set si at rotation R (p_hat restricted to
// the INT2 positions in Phat, c = Phat V in Cv): x = (Phat Q2(V R)) R^T - c.
hipError_t value_forward(Ctx &c, int si, const double *R, double *log_out, int64_t log_stride) {
  const SetDev &sd = c.set[si];
  const int H = c.sh.H, NS = sd.sl.n, Lm = sd.Lm, G = c.sh.G, nq = c.sh.nq, RQ = G * nq;
  const int64_t toks = static_cast<int64_t>(NS) * Lm;
  G64 g = gemm(sd.V, D, 1, R, D, 1, c.p(c.L.Z), D, static_cast<int>(toks), D, D);
  g.as1 = g.cs1 = toks * D;
  g.bs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  const int64_t rows_tok = H * toks;
  hipLaunchKernelGGL(quant_ste_kernel, dim3(static_cast<unsigned>((rows_tok + 3) / 4)), dim3(256), 0, c.st,
                     c.p(c.L.Z), c.p(c.L.Xt), c.ws + c.L.flag, H, Lm, sd.sl, c.cfg->num_sink, c.cfg->num_recent,
                     c.cfg->clip_v, 0);
  OPTR_TRY(hipGetLastError());
  // U = Phat Xt (into Qr), batch (h, b)
  g = gemm(sd.Phat, Lm, 1, c.p(c.L.Xt), D, 1, c.p(c.L.Qr), D, RQ, D, Lm);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * D;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  // x = U R^T - c, batch h
  const int64_t rows = static_cast<int64_t>(H) * NS * RQ;
  OPTR_TRY(hipMemcpyAsync(c.p(c.L.X), sd.Cv, static_cast<size_t>(rows) * D * 8, hipMemcpyDeviceToDevice, c.st));
  g = gemm(c.p(c.L.Qr), D, 1, R, 1, D, c.p(c.L.X), D, NS * RQ, D, D, 1.0, -1.0);
  g.as1 = g.cs1 = static_cast<int64_t>(NS) * RQ * D;
  g.bs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  g = gemm(c.p(c.L.X), D, 1, c.p(c.L.gamma), D, 1, c.p(c.L.XG), D, nq, D, D);
  g.as1 = g.cs1 = static_cast<int64_t>(nq) * D;
  g.bdiv = NS * G;
  g.bs1 = static_cast<int64_t>(G) * D * D;
  g.bmod = G;
  g.bs2 = D * D;
  OPTR_TRY(run_gemm(g, H * NS * G, c.st));
  const double N = static_cast<double>(NS) * RQ;
  hipLaunchKernelGGL(err_rows_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, c.st, c.p(c.L.X),
                     c.p(c.L.XG), c.p(c.L.e2), rows, 1.0 / c.sh.d_model, 2.0 / (N * c.sh.d_model));
  OPTR_TRY(hipGetLastError());
  hipLaunchKernelGGL(loss_kernel, dim3(H), dim3(256), 0, c.st, nullptr, c.p(c.L.e2), static_cast<int64_t>(NS) * RQ,
                     1.0, c.p(c.L.loss), log_out, log_stride);
  return hipGetLastError();
}

hipError_t value_backward(Ctx &c, const double *R) {
  const SetDev &sd = c.set[0];
  const int H = c.sh.H, NS = sd.sl.n, Lm = sd.Lm, RQ = c.sh.G * c.sh.nq;
  const int64_t toks = static_cast<int64_t>(NS) * Lm;
  // dU = dx R (into dQ); dR = dx^T U
  G64 g = gemm(c.p(c.L.XG), D, 1, R, D, 1, c.p(c.L.dQ), D, NS * RQ, D, D);
  g.as1 = g.cs1 = static_cast<int64_t>(NS) * RQ * D;
  g.bs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  g = gemm(c.p(c.L.XG), 1, D, c.p(c.L.Qr), D, 1, c.p(c.L.dR), D, D, D, NS * RQ);
  g.as1 = g.bs1 = static_cast<int64_t>(NS) * RQ * D;
  g.cs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  // dXt = Phat^T dU (into dK), batch (h, b); flags; dR += V^T dZ
  g = gemm(sd.Phat, 1, Lm, c.p(c.L.dQ), D, 1, c.p(c.L.dK), D, Lm, D, RQ);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(RQ) * D;
  g.cs1 = static_cast<int64_t>(Lm) * D;
  OPTR_TRY(run_gemm(g, H * NS, c.st));
  const size_t n = static_cast<size_t>(H) * toks * D;
  hipLaunchKernelGGL(mask_mul_kernel, dim3(blocks_for(n)), dim3(256), 0, c.st, c.p(c.L.dK), c.ws + c.L.flag, n);
  OPTR_TRY(hipGetLastError());
  g = gemm(sd.V, 1, D, c.p(c.L.dK), D, 1, c.p(c.L.dR), D, D, D, static_cast<int>(toks), 1.0, 1.0);
  g.as1 = g.bs1 = toks * D;
  g.cs1 = D * D;
  return run_gemm(g, H, c.st);
}

// dS from dR (S of the last rotation_of): dE = R0^T dR, dS = L(S^T, dE)
hipError_t generator_grad(Ctx &c, const double *R0) {
  const int H = c.sh.H;
  G64 g = gemm(R0, 1, D, c.p(c.L.dR), D, 1, c.p(c.L.dE), D, D, D, D);
  g.as1 = g.bs1 = g.cs1 = D * D;
  OPTR_TRY(run_gemm(g, H, c.st));
  hipLaunchKernelGGL(expm_frechet_kernel, dim3(H), dim3(kExT), 0, c.st, c.p(c.L.S), c.p(c.L.dE), c.p(c.L.dS),
                     c.p(c.L.fr));
  return hipGetLastError();
}

// the gradient, then the Adam step
hipError_t generator_step(Ctx &c, const double *R0, int step) {
  const int H = c.sh.H;
  OPTR_TRY(generator_grad(c, R0));
  const double bc1 = 1.0 - std::pow(0.9, step), bc2 = 1.0 - std::pow(0.999, step);
  const size_t n = static_cast<size_t>(H) * D * D;
  hipLaunchKernelGGL(adam_kernel, dim3(blocks_for(n)), dim3(256), 0, c.st, c.p(c.L.A), c.p(c.L.Am), c.p(c.L.Av),
                     c.p(c.L.dS), c.cfg->lr, bc1, std::sqrt(bc2), H);
  return hipGetLastError();
}

hipError_t fill(double *x, size_t n, double v, hipStream_t st) {
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(n)), dim3(256), 0, st, x, n, v);
  return hipGetLastError();
}

int num_checkpoints(const kvq_optr_config &cfg) {
  const int n = cfg.steps / cfg.eval_every;
  return n > 0 ? n : 1;
}
bool is_checkpoint(const kvq_optr_config &cfg, int i) {
  return cfg.steps < cfg.eval_every ? i == cfg.steps : i % cfg.eval_every == 0;
}

// One phase of Algorithm 1 (0: keys, 1: values): Adam from A = 0 with the
// held-out checkpoints; leaves the selected generator in Ab.
hipError_t run_phase(Ctx &c, int phase, const double *R0, double *log_base) {
  const int H = c.sh.H;
  const size_t mat = static_cast<size_t>(H) * D * D;
  const int steps = c.cfg->steps, nck = num_checkpoints(*c.cfg);
  const int64_t lstride = 2 * (static_cast<int64_t>(steps) + nck + 1);
  double *lg = log_base ? log_base + phase * (steps + nck + 1) : nullptr;
  OPTR_TRY(fill(c.p(c.L.A), mat, 0.0, c.st));
  OPTR_TRY(fill(c.p(c.L.Am), mat, 0.0, c.st));
  OPTR_TRY(fill(c.p(c.L.Av), mat, 0.0, c.st));
  OPTR_TRY(fill(c.p(c.L.best), H, NAN, c.st));
  int ck = 0;
  for (int i = 1; i <= steps; ++i) {
    OPTR_TRY(rotation_of(c, c.p(c.L.A), R0, c.p(c.L.R)));
    if (phase == 0) {
      OPTR_TRY(key_forward(c, 0, c.p(c.L.R), lg ? lg + (i - 1) : nullptr, lstride));
      OPTR_TRY(key_backward(c));
    } else {
      OPTR_TRY(value_forward(c, 0, c.p(c.L.R), lg ? lg + (i - 1) : nullptr, lstride));
      OPTR_TRY(value_backward(c, c.p(c.L.R)));
    }
    OPTR_TRY(generator_step(c, R0, i));
    if (is_checkpoint(*c.cfg, i)) {
      OPTR_TRY(rotation_of(c, c.p(c.L.A), R0, c.p(c.L.R)));
      if (phase == 0)
        OPTR_TRY(key_forward(c, 1, c.p(c.L.R), nullptr, 0));
      else
        OPTR_TRY(value_forward(c, 1, c.p(c.L.R), nullptr, 0));
      hipLaunchKernelGGL(checkpoint_kernel, dim3(H), dim3(256), 0, c.st, c.p(c.L.loss), c.p(c.L.best), c.p(c.L.A),
                         c.p(c.L.Ab), i, lg ? lg + steps + ck : nullptr, lstride, lg ? lg + steps + nck : nullptr);
      OPTR_TRY(hipGetLastError());
      ++ck;
    }
  }
  return hipSuccess;
}

// p_hat of the selected key rotation on set si, restricted to INT2 positions, and c = p_hat V
hipError_t value_attention(Ctx &c, int si, const double *Rk) {
  SetDev &sd = c.set[si];
  const int H = c.sh.H, NS = sd.sl.n, Lm = sd.Lm, RQ = c.sh.G * c.sh.nq;
  OPTR_TRY(key_forward(c, si, Rk, nullptr, 0, true));
  const int64_t rows = static_cast<int64_t>(H) * NS * RQ;
  OPTR_TRY(hipMemcpyAsync(sd.Phat, c.p(c.L.P), static_cast<size_t>(rows) * Lm * 8, hipMemcpyDeviceToDevice, c.st));
  hipLaunchKernelGGL(int2_restrict_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, c.st, sd.Phat, RQ, Lm,
                     sd.sl, c.cfg->num_sink, c.cfg->num_recent);
  OPTR_TRY(hipGetLastError());
  G64 g = gemm(sd.Phat, Lm, 1, sd.V, D, 1, sd.Cv, D, RQ, D, Lm);
  g.as1 = static_cast<int64_t>(RQ) * Lm;
  g.bs1 = static_cast<int64_t>(Lm) * D;
  g.cs1 = static_cast<int64_t>(RQ) * D;
  return run_gemm(g, H * NS, c.st);
}

// Set-up shared by the entry points: traces to fp64 head-major, reference
// logits, W_O Gram blocks Gamma_j = W_j W_j^T, base rotations.
hipError_t setup(Ctx &c, int dtype, const kvq_trace_set *sets[2], const void *w_o, const float *r0_k,
                 const float *r0_v, const float *key_mean_in, float *key_mean_out) {
  const int H = c.sh.H, G = c.sh.G, nq = c.sh.nq, RQ = G * nq, dm = c.sh.d_model;
  const bool f32 = dtype == KVQ_F32;
  double *mu64 = c.p(c.L.mu64);
  if (key_mean_in) {
    hipLaunchKernelGGL(widen_f32_kernel, dim3(blocks_for(H * D)), dim3(256), 0, c.st, key_mean_in,
                       static_cast<size_t>(H) * D, mu64);
    OPTR_TRY(hipGetLastError());
    if (key_mean_out)
      OPTR_TRY(hipMemcpyAsync(key_mean_out, key_mean_in, static_cast<size_t>(H) * D * 4, hipMemcpyDeviceToDevice,
                              c.st));
  } else {
    if (f32)
      hipLaunchKernelGGL(key_mean_kernel<KVQ_F32>, dim3(H), dim3(D), 0, c.st, sets[0]->k, sets[0]->max_len, H,
                         c.set[0].sl, key_mean_out, mu64);
    else
      hipLaunchKernelGGL(key_mean_kernel<KVQ_BF16>, dim3(H), dim3(D), 0, c.st, sets[0]->k, sets[0]->max_len, H,
                         c.set[0].sl, key_mean_out, mu64);
    OPTR_TRY(hipGetLastError());
  }
  for (int si = 0; si < 2; ++si) {
    if (!sets[si]) continue;
    SetDev &sd = c.set[si];
    const dim3 grid(16, sd.sl.n, H);
    if (f32)
      hipLaunchKernelGGL(prep_kernel<KVQ_F32>, grid, dim3(256), 0, c.st, sets[si]->k, sets[si]->v, sets[si]->q, sd.Lm,
                         H, G, nq, sd.sl, mu64, sd.Kc, sd.V, sd.Q);
    else
      hipLaunchKernelGGL(prep_kernel<KVQ_BF16>, grid, dim3(256), 0, c.st, sets[si]->k, sets[si]->v, sets[si]->q,
                         sd.Lm, H, G, nq, sd.sl, mu64, sd.Kc, sd.V, sd.Q);
    OPTR_TRY(hipGetLastError());
    // reference logits Q Kc^T / sqrt(d) (centering shifts every logit of a row equally)
    G64 g = gemm(sd.Q, D, 1, sd.Kc, 1, D, sd.Lref, sd.Lm, RQ, sd.Lm, D, 1.0 / std::sqrt(static_cast<double>(D)));
    g.as1 = static_cast<int64_t>(RQ) * D;
    g.bs1 = static_cast<int64_t>(sd.Lm) * D;
    g.cs1 = static_cast<int64_t>(RQ) * sd.Lm;
    OPTR_TRY(run_gemm(g, H * sd.sl.n, c.st));
  }
  const size_t nw = static_cast<size_t>(H) * G * D * dm;
  if (f32)
    hipLaunchKernelGGL(widen_kernel<KVQ_F32>, dim3(blocks_for(nw)), dim3(256), 0, c.st, w_o, nw, c.p(c.L.w64));
  else
    hipLaunchKernelGGL(widen_kernel<KVQ_BF16>, dim3(blocks_for(nw)), dim3(256), 0, c.st, w_o, nw, c.p(c.L.w64));
  OPTR_TRY(hipGetLastError());
  G64 g = gemm(c.p(c.L.w64), dm, 1, c.p(c.L.w64), 1, dm, c.p(c.L.gamma), D, D, D, dm);
  g.as1 = g.bs1 = static_cast<int64_t>(D) * dm;
  g.cs1 = D * D;
  OPTR_TRY(run_gemm(g, H * G, c.st));
  const size_t mat = static_cast<size_t>(H) * D * D;
  if (r0_k) {
    hipLaunchKernelGGL(widen_f32_kernel, dim3(blocks_for(mat)), dim3(256), 0, c.st, r0_k, mat, c.p(c.L.R0k));
    OPTR_TRY(hipGetLastError());
  }
  if (r0_v) {
    hipLaunchKernelGGL(widen_f32_kernel, dim3(blocks_for(mat)), dim3(256), 0, c.st, r0_v, mat, c.p(c.L.R0v));
    OPTR_TRY(hipGetLastError());
  }
  return hipSuccess;
}

// 0 = ok, else a kvq_status; fills the shape and the sets' lengths
int check_sets(const kvq_trace_set *calib, const kvq_trace_set *heldout, int H, int Hq, int nq, int d_model,
               Shape &sh, SeqLens sl[2]) {
  if (!calib || H < 1 || Hq < 1 || Hq % H || nq < 1 || d_model < 1) return KVQ_ERR_INVALID_ARGUMENT;
  sh.H = H;
  sh.G = Hq / H;
  sh.nq = nq;
  sh.d_model = d_model;
  const kvq_trace_set *s2[2] = {calib, heldout};
  for (int i = 0; i < 2; ++i) {
    const kvq_trace_set *s = s2[i] ? s2[i] : calib;
    if (s->num_seqs < 1 || s->max_len < 1 || !s->seq_lens) return KVQ_ERR_INVALID_ARGUMENT;
    if (s->num_seqs > kMaxTraceSeqs) return KVQ_ERR_UNSUPPORTED;
    if (!s->k || !s->v || !s->q) return KVQ_ERR_INVALID_ARGUMENT;
    for (const void *p : {s->k, s->v, s->q})
      if (reinterpret_cast<uintptr_t>(p) & 15u) return KVQ_ERR_INVALID_ARGUMENT;
    sl[i].n = s->num_seqs;
    for (int b = 0; b < s->num_seqs; ++b) {
      const int L = s->seq_lens[b];
      if (L < nq || L > s->max_len) return KVQ_ERR_INVALID_ARGUMENT;
      sl[i].lens[b] = L;
    }
    sh.ns[i] = s->num_seqs;
    sh.lm[i] = s->max_len;
  }
  return KVQ_OK;
}

int check_config(const kvq_optr_config *cfg) {
  if (!cfg) return KVQ_ERR_INVALID_ARGUMENT;
  if (!(cfg->clip_k > 0.0f && cfg->clip_k <= 1.0f) || !(cfg->clip_v > 0.0f && cfg->clip_v <= 1.0f))
    return KVQ_ERR_INVALID_ARGUMENT;
  if (cfg->num_sink < 0 || cfg->num_recent < 0 || cfg->steps < 1 || cfg->eval_every < 1) return KVQ_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(cfg->lr) || cfg->lr <= 0.0f || !std::isfinite(cfg->lambda_k) || cfg->lambda_k < 0.0f)
    return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

void bind_sets(Ctx &c, const SeqLens sl[2]) {
  for (int i = 0; i < 2; ++i) {
    SetDev &sd = c.set[i];
    sd.sl = sl[i];
    sd.Lm = c.sh.lm[i];
    sd.Kc = c.p(c.L.set_off[i][0]);
    sd.V = c.p(c.L.set_off[i][1]);
    sd.Q = c.p(c.L.set_off[i][2]);
    sd.Lref = c.p(c.L.set_off[i][3]);
    sd.Phat = c.p(c.L.set_off[i][4]);
    sd.Cv = c.p(c.L.set_off[i][5]);
  }
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" {

size_t kvq_optr_workspace_bytes(const kvq_trace_set *calib, const kvq_trace_set *heldout, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t num_queries, int32_t d_model) {
  Shape sh{};
  SeqLens sl[2];
  if (check_sets(calib, heldout, num_kv_heads, num_q_heads, num_queries, d_model, sh, sl)) return 0;
  return layout(sh).total;
}

int kvq_optr_calibrate(int32_t dtype, const kvq_trace_set *calib, const kvq_trace_set *heldout, int32_t num_kv_heads,
                       int32_t num_q_heads, int32_t num_queries, const void *w_o, int32_t d_model, const float *r0_k,
                       const float *r0_v, const float *key_mean, const kvq_optr_config *cfg, float *out_r_k,
                       float *out_r_v, float *out_key_mean, double *out_log, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (dtype != KVQ_F32 && dtype != KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  if (!heldout) return KVQ_ERR_INVALID_ARGUMENT;
  Shape sh{};
  SeqLens sl[2];
  int rc = check_sets(calib, heldout, num_kv_heads, num_q_heads, num_queries, d_model, sh, sl);
  if (rc) return rc;
  rc = check_config(cfg);
  if (rc) return rc;
  if (!w_o || !r0_k || !r0_v || !out_r_k || !out_r_v) return KVQ_ERR_INVALID_ARGUMENT;
  for (const void *p : {w_o, static_cast<const void *>(r0_k), static_cast<const void *>(r0_v)})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return KVQ_ERR_INVALID_ARGUMENT;
  Ctx c{};
  c.sh = sh;
  c.L = layout(sh);
  if (!workspace || workspace_bytes < c.L.total) return KVQ_ERR_WORKSPACE;
  c.ws = static_cast<uint8_t *>(workspace);
  c.cfg = cfg;
  c.st = stream;
  bind_sets(c, sl);
  const kvq_trace_set *sets[2] = {calib, heldout};
  if (setup(c, dtype, sets, w_o, r0_k, r0_v, key_mean, out_key_mean) != hipSuccess) return KVQ_ERR_HIP;
  const size_t mat = static_cast<size_t>(sh.H) * D * D;
  // keys: Adam on L_K with held-out selection, then the selected R_K
  if (run_phase(c, 0, c.p(c.L.R0k), out_log) != hipSuccess) return KVQ_ERR_HIP;
  if (rotation_of(c, c.p(c.L.Ab), c.p(c.L.R0k), c.p(c.L.Rk_hat)) != hipSuccess) return KVQ_ERR_HIP;
  hipLaunchKernelGGL(narrow_kernel, dim3(blocks_for(mat)), dim3(256), 0, stream, c.p(c.L.Rk_hat), mat, out_r_k);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  // values: under the selected key attention of each set
  for (int si = 0; si < 2; ++si)
    if (value_attention(c, si, c.p(c.L.Rk_hat)) != hipSuccess) return KVQ_ERR_HIP;
  if (run_phase(c, 1, c.p(c.L.R0v), out_log) != hipSuccess) return KVQ_ERR_HIP;
  if (rotation_of(c, c.p(c.L.Ab), c.p(c.L.R0v), c.p(c.L.R)) != hipSuccess) return KVQ_ERR_HIP;
  hipLaunchKernelGGL(narrow_kernel, dim3(blocks_for(mat)), dim3(256), 0, stream, c.p(c.L.R), mat, out_r_v);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  return KVQ_OK;
}

int kvq_optr_loss_grad(int32_t dtype, int32_t phase, const kvq_trace_set *set, int32_t num_kv_heads,
                       int32_t num_q_heads, int32_t num_queries, const void *w_o, int32_t d_model, const float *r0,
                       const double *a, const float *r_k_hat, const float *key_mean, const kvq_optr_config *cfg,
                       double *out_loss, double *out_grad, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (dtype != KVQ_F32 && dtype != KVQ_BF16) return KVQ_ERR_UNSUPPORTED;
  if (phase != 0 && phase != 1) return KVQ_ERR_UNSUPPORTED;
  Shape sh{};
  SeqLens sl[2];
  int rc = check_sets(set, nullptr, num_kv_heads, num_q_heads, num_queries, d_model, sh, sl);
  if (rc) return rc;
  rc = check_config(cfg);
  if (rc) return rc;
  if (!w_o || !r0 || !a || !key_mean || !out_loss || !out_grad || (phase == 1 && !r_k_hat))
    return KVQ_ERR_INVALID_ARGUMENT;
  Ctx c{};
  c.sh = sh;
  c.L = layout(sh);
  if (!workspace || workspace_bytes < c.L.total) return KVQ_ERR_WORKSPACE;
  c.ws = static_cast<uint8_t *>(workspace);
  c.cfg = cfg;
  c.st = stream;
  bind_sets(c, sl);
  const kvq_trace_set *sets[2] = {set, nullptr};
  if (setup(c, dtype, sets, w_o, r0, r_k_hat, key_mean, nullptr) != hipSuccess) return KVQ_ERR_HIP;
  const size_t mat = static_cast<size_t>(sh.H) * D * D;
  if (hipMemcpyAsync(c.p(c.L.A), a, mat * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess) return KVQ_ERR_HIP;
  if (phase == 1) {   // the key attention of the given key rotation (already a rotation: R0v slot holds it)
    if (hipMemcpyAsync(c.p(c.L.Rk_hat), c.p(c.L.R0v), mat * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return KVQ_ERR_HIP;
    if (value_attention(c, 0, c.p(c.L.Rk_hat)) != hipSuccess) return KVQ_ERR_HIP;
  }
  if (rotation_of(c, c.p(c.L.A), c.p(c.L.R0k), c.p(c.L.R)) != hipSuccess) return KVQ_ERR_HIP;
  if (phase == 0) {
    if (key_forward(c, 0, c.p(c.L.R), nullptr, 0) != hipSuccess || key_backward(c) != hipSuccess) return KVQ_ERR_HIP;
  } else {
    if (value_forward(c, 0, c.p(c.L.R), nullptr, 0) != hipSuccess || value_backward(c, c.p(c.L.R)) != hipSuccess)
      return KVQ_ERR_HIP;
  }
  // dA = dS - dS^T with dS = L(S^T, R0^T dR)
  if (generator_grad(c, c.p(c.L.R0k)) != hipSuccess) return KVQ_ERR_HIP;
  hipLaunchKernelGGL(antisym_kernel, dim3(blocks_for(mat)), dim3(256), 0, stream, c.p(c.L.dS), out_grad, sh.H);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  if (hipMemcpyAsync(out_loss, c.p(c.L.loss), static_cast<size_t>(sh.H) * 8, hipMemcpyDeviceToDevice, stream) !=
      hipSuccess)
    return KVQ_ERR_HIP;
  return KVQ_OK;
}

}  // extern "C"
