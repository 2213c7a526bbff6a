// quantize.hip -- cache-write kernel: rotation, optional key centering, INT2
// group quantization with clip ratio, 2-bit packing into the paged layout.
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization".
//   §6 Efficiency Analysis: one launch rotates the (centered) key, clips,
//   quantizes, packs and writes; §4.1 and Appendix Eq. (20)-(21): keys are
//   centered by the calibration mean before rotation; §3.1 Eq. (4): z' = z R.
//
// The fp32 quantizer step order is fixed (see kvq.h), so contraction of
// multiply-add pairs into FMAs is switched off for this translation unit.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

struct QuantArgs {
  const void *k, *v;
  int64_t num_tokens;
  int H;
  const int64_t *slot_mapping;
  RotDev rk, rv;
  const float *key_mean;
  float clip_k, clip_v;
  uint8_t *pages;
  int64_t num_pages;
  int P;
  double inv_sqrt_d;  // 1/sqrt(128) as a correctly rounded double
};

__device__ __forceinline__ float wave_min(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ uint32_t f16_bits(_Float16 h) {
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// One wave per (token, head) item; lane l holds group elements l and l + 64.
// All waves of a block run the same number of iterations, so the block-wide
// barriers below are uniform.
template <int DT>
__global__ __launch_bounds__(256) void quantize_exact_kernel(QuantArgs a) {
  __shared__ double zsh[4][D];
  __shared__ uint8_t csh[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n_items = a.num_tokens * a.H;
  const int64_t slots = a.num_pages * a.P;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 4; base < n_items;
       base += static_cast<int64_t>(gridDim.x) * 4) {
    const int64_t item = base + wave;
    bool active = item < n_items;
    int64_t t = 0, slot = -1;
    int h = 0;
    if (active) {
      t = item / a.H;
      h = static_cast<int>(item % a.H);
      slot = a.slot_mapping ? a.slot_mapping[t] : t;
      active = slot >= 0 && slot < slots;
    }
    const int64_t page = active ? slot / a.P : 0;
    const int p = active ? static_cast<int>(slot % a.P) : 0;
    uint8_t *blk = a.pages + (static_cast<size_t>(page) * a.H + h) * static_cast<size_t>(72 * a.P);
    const size_t gbase = (static_cast<size_t>(t) * a.H + h) * D;

    for (int kv = 0; kv < 2; ++kv) {
      const void *src = kv ? a.v : a.k;
      const RotDev rot = kv ? a.rv : a.rk;
      const float *mean = kv ? nullptr : a.key_mean;
      const float clip = kv ? a.clip_v : a.clip_k;
      float r0 = 0.0f, r1 = 0.0f;
      if (active) {
        const float x0 = load_elem<DT>(src, gbase + lane);
        const float x1 = load_elem<DT>(src, gbase + lane + 64);
        if (rot.kind == KVQ_ROT_IDENTITY) {
          r0 = mean ? x0 - mean[h * D + lane] : x0;
          r1 = mean ? x1 - mean[h * D + lane + 64] : x1;
        } else {
          zsh[wave][lane] = static_cast<double>(x0) - (mean ? static_cast<double>(mean[h * D + lane]) : 0.0);
          zsh[wave][lane + 64] =
              static_cast<double>(x1) - (mean ? static_cast<double>(mean[h * D + lane + 64]) : 0.0);
        }
      }
      __syncthreads();
      if (active && rot.kind != KVQ_ROT_IDENTITY) {
        // z' = z R in fp64, summed in index order: products and sums rounded
        // separately, then one rounding to fp32.
        double acc0 = 0.0, acc1 = 0.0;
        if (rot.kind == KVQ_ROT_DENSE) {
          const float *m = rot.matrix + static_cast<size_t>(h) * D * D;
          for (int i = 0; i < D; ++i) {
            const double zi = zsh[wave][i];
            acc0 = acc0 + zi * static_cast<double>(m[i * D + lane]);
            acc1 = acc1 + zi * static_cast<double>(m[i * D + lane + 64]);
          }
        } else {
          const int8_t *s = rot.signs + h * D;
          for (int i = 0; i < D; ++i) {
            const double zi = zsh[wave][i];
            const double si = static_cast<double>(s[i]);
            const double e0 = si * static_cast<double>(hadamard_sign(i, lane)) * a.inv_sqrt_d;
            const double e1 = si * static_cast<double>(hadamard_sign(i, lane + 64)) * a.inv_sqrt_d;
            acc0 = acc0 + zi * e0;
            acc1 = acc1 + zi * e1;
          }
        }
        r0 = static_cast<float>(acc0);
        r1 = static_cast<float>(acc1);
      }

      // INT2 group quantizer, fixed fp32 step order.
      const float mn = wave_min(fminf(r0, r1));
      const float mx = wave_max(fmaxf(r0, r1));
      float lo = clip * mn;
      const float hi = clip * mx;
      const float span = hi - lo;
      float s32 = span / 3.0f;
      // Round lo and s32 to fp32 before the fp16 conversion: without the
      // register barrier the backend fuses clip*mn and the conversion into one
      // mixed-precision FMA that rounds once, which is not the defined order.
      asm volatile("" : "+v"(lo));
      asm volatile("" : "+v"(s32));
      const _Float16 sh = static_cast<_Float16>(s32);
      const _Float16 zh = static_cast<_Float16>(lo);
      const float s = static_cast<float>(sh);
      const float z = static_cast<float>(zh);
      uint32_t c0 = 0, c1 = 0;
      if (s != 0.0f) {
        const float inv = 1.0f / s;
        const float d0 = r0 - z, d1 = r1 - z;
        const float t0 = d0 * inv, t1 = d1 * inv;
        const float q0 = fminf(fmaxf(__builtin_rintf(t0), 0.0f), 3.0f);
        const float q1 = fminf(fmaxf(__builtin_rintf(t1), 0.0f), 3.0f);
        c0 = static_cast<uint32_t>(q0);
        c1 = static_cast<uint32_t>(q1);
      }
      csh[wave][lane] = static_cast<uint8_t>(c0);
      csh[wave][lane + 64] = static_cast<uint8_t>(c1);
      __syncthreads();
      if (active && lane < 32) {
        const uint32_t b = csh[wave][4 * lane] | (csh[wave][4 * lane + 1] << 2) | (csh[wave][4 * lane + 2] << 4) |
                           (csh[wave][4 * lane + 3] << 6);
        if (kv == 0)
          blk[32 * p + lane] = static_cast<uint8_t>(b);
        else
          blk[32 * a.P + 128 * (p / 4) + 4 * lane + (p % 4)] = static_cast<uint8_t>(b);
      }
      if (active && lane == 0) {
        const uint32_t meta = f16_bits(sh) | (f16_bits(zh) << 16);
        *reinterpret_cast<uint32_t *>(blk + (kv ? 68 : 64) * a.P + 4 * p) = meta;
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                           const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean, float clip_k,
                           float clip_v, uint8_t *pages, int64_t num_pages, int page_size, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  QuantArgs a{k, v, num_tokens, H, slot_mapping, rk, rv, key_mean, clip_k, clip_v, pages, num_pages, page_size,
              1.0 / __builtin_sqrt(128.0)};
  const int64_t items = num_tokens * H;
  int64_t blocks = (items + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(quantize_exact_kernel<KVQ_F32>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_exact_kernel<KVQ_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace kvq
