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
  for (int o = 32; o > 0; o >>= 1) x = fminf(x, lane_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, lane_xor(x, o));
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
        } else if (rot.kind == KVQ_ROT_SIGNED_HADAMARD) {
          // z' = (s z) H / sqrt(128) in fp64 by the fast transform (the same
          // sums as the index-order product, in butterfly order: they differ
          // in fp64 rounding only), then one rounding to fp32
          const int8_t *sg = rot.signs + h * D;
          double y0 = (static_cast<double>(x0) - (mean ? static_cast<double>(mean[h * D + lane]) : 0.0)) *
                      static_cast<double>(sg[lane]);
          double y1 = (static_cast<double>(x1) - (mean ? static_cast<double>(mean[h * D + lane + 64]) : 0.0)) *
                      static_cast<double>(sg[lane + 64]);
          fwht128(y0, y1, lane);
          r0 = static_cast<float>(y0 * a.inv_sqrt_d);
          r1 = static_cast<float>(y1 * a.inv_sqrt_d);
        } else {
          zsh[wave][lane] = static_cast<double>(x0) - (mean ? static_cast<double>(mean[h * D + lane]) : 0.0);
          zsh[wave][lane + 64] =
              static_cast<double>(x1) - (mean ? static_cast<double>(mean[h * D + lane + 64]) : 0.0);
        }
      }
      __syncthreads();
      if (active && rot.kind == KVQ_ROT_DENSE) {
        // z' = z R in fp64, summed in index order: products and sums rounded
        // separately, then one rounding to fp32.
        double acc0 = 0.0, acc1 = 0.0;
        const float *m = rot.matrix + static_cast<size_t>(h) * D * D;
        for (int i = 0; i < D; ++i) {
          const double zi = zsh[wave][i];
          acc0 = acc0 + zi * static_cast<double>(m[i * D + lane]);
          acc1 = acc1 + zi * static_cast<double>(m[i * D + lane + 64]);
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


// ------------------------------------------------------------------------
// bf16 inputs: rotation on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// One workgroup takes one KV head of one side (keys or values) over a run
// of 16-token tiles; the head's rotation is staged once in LDS as the A
// operand.  For a tile, D = R'^T X^T: A rows are output dims, B columns are
// the 16 tokens (the bf16 input rows, exact), k runs over input dims.  The A
// rows are permuted so that lane (token tk = l%16, g = l/16) ends up with the
// 32 consecutive output dims 32g..32g+31 of token tk: dim 32g + 4nt + i sits
// in accumulator nt, element i, i.e. the codes of byte 8g + nt.
//   signed Hadamard: R' = diag(s) H (entries +-1, exact in bf16) and the
//                    1/sqrt(128) is applied to the fp32 result;
//   dense:           R = R_hi + R_mid + R_lo, three bf16 parts (24 bits);
//   identity:        no product, the lane loads its 32 dims directly.
// Key centering subtracts mu R (fp64 dot products, one per dim) after the
// product: (k - mu) R = k R - mu R.
// The quantizer is the same fp32 sequence as the exact kernel; with the
// identity rotation the codes are therefore identical to it.  With a
// rotation the rotated values differ from an fp64 product by fp32 rounding.
// ------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kQTiles = 64;       // 16-token tiles per workgroup
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: x + kMagic rounds x to an integer (ties to even)
constexpr uint32_t kMagicBits = 0x4B400000u;

// sum_{j<16} kMagicBits * 4^j (mod 2^32): the offset left by packing 16
// magic-biased codes with shift-add.
__host__ __device__ constexpr uint32_t magic_pack_offset() {
  uint32_t acc = 0;
  for (int j = 15; j >= 0; --j) acc = (acc << 2) + kMagicBits;
  return acc;
}

constexpr int kMaxClips = 8;  // clip ratios written by one launch (one cache each)

// One side (keys or values) of a cache write.
struct FastSide {
  const uint16_t *x;    // [T][H][128] bf16 bits
  const int8_t *signs;  // [H][128]
  const float *matrix;  // [H][128][128]
  float clip[kMaxClips];  // clip ratio of cache c (c < nclip)
  int side;             // 0 keys, 1 values
};

struct FastArgs {
  FastSide sd[2];       // the sides of the launch (sd[1] unused for one side)
  int64_t T;
  int H;
  const int64_t *slot_mapping;
  const float *mean;    // [H][128] or null (keys only; the keys are sd[0])
  uint8_t *pages;
  int64_t num_pages;
  int P;
  int p_shift;          // log2(P) if P is a power of two, else -1
  int nclip;            // caches written (one per clip ratio), at pages + c * clip_stride
  size_t clip_stride;   // bytes between the caches of consecutive clip ratios
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ int qdpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int qdpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }

// Output dim of A row r of accumulator tile nt.
__device__ __forceinline__ int a_row_dim(int nt, int r) { return 32 * (r >> 2) + 4 * nt + (r & 3); }

constexpr int kQWavesF = 8;  // waves per workgroup of the cache-write kernel

// kSides = 2: keys and values of each tile in one pass, so that every
// (page, head) block of the cache is written whole within a few
// instructions (writing its halves in two launches costs ~10% more time);
// kStaged = number of staged rotations (1 when both sides use the same one).
// (at most 128 VGPRs: two workgroups of 8 waves per CU)
// kClips: false = one clip ratio (clip[0], cache at pages), true = a.nclip.
template <int KIND, bool kCenter, bool kWide, int kSides, int kStaged, bool kClips>
__global__ __launch_bounds__(64 * kQWavesF, 4) void quantize_fast_kernel(FastArgs a) {
  constexpr int kParts = KIND == KVQ_ROT_DENSE ? 3 : (KIND == KVQ_ROT_SIGNED_HADAMARD ? 1 : 0);
  extern __shared__ __attribute__((aligned(16))) uint4 ash[];  // [kStaged][kParts][4 ks][8 nt][64 lanes]
  __shared__ float mrot[D];
  // the H heads of a run of tokens are read together, on one XCD: workgroup
  // i runs on XCD i mod 8 (workgroups are dealt to the 8 XCDs in turn), so
  // with a multiple of 8 runs, workgroup i = 8 (H q + h) + x takes head h of
  // run 8 q + x (16 x 32K cache write 553-559 -> 545-548 us); otherwise head
  // i mod H of run i / H
  const int64_t n_runs = ((a.T + 15) / 16 + kQTiles - 1) / kQTiles;
  const unsigned wid = blockIdx.x, H_u = static_cast<unsigned>(a.H);
  const bool xcd_local = n_runs % 8 == 0;
  const int h = static_cast<int>(xcd_local ? (wid >> 3) % H_u : wid % H_u);
  const int64_t run = xcd_local ? 8 * static_cast<int64_t>((wid >> 3) / H_u) + (wid & 7u) : wid / H_u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tk = lane & 15, g = lane >> 4;

  // ---- stage the rotations (A operands) and mu R
  if constexpr (kParts > 0) {
    for (int e2 = threadIdx.x; e2 < kStaged * 4 * 8 * 64; e2 += blockDim.x) {
      const int st = e2 >> 11, e = e2 & 2047;
      const FastSide &fs = a.sd[st];
      const int ks = e >> 9, nt = (e >> 6) & 7, ln = e & 63;
      const int d = a_row_dim(nt, ln & 15);
      const int k0 = 32 * ks + 8 * (ln >> 4);
      uint32_t w[kParts > 0 ? kParts : 1][4];
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        uint32_t lo[kParts > 0 ? kParts : 1], hi[kParts > 0 ? kParts : 1];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int k = k0 + 2 * j2 + jj;
          if constexpr (KIND == KVQ_ROT_SIGNED_HADAMARD) {
            const bool neg = (fs.signs[h * D + k] < 0) != ((__popc(static_cast<unsigned>(k & d)) & 1) != 0);
            (jj ? hi : lo)[0] = neg ? 0xBF80u : 0x3F80u;
          } else {
            const float r = fs.matrix[(static_cast<size_t>(h) * D + k) * D + d];
            const uint32_t b0 = bf16_rne_bits(r);
            const float r1 = r - bf16_to_float(b0);
            const uint32_t b1 = bf16_rne_bits(r1);
            const float r2 = r1 - bf16_to_float(b1);
            const uint32_t b2 = bf16_rne_bits(r2);
            (jj ? hi : lo)[0] = b0;
            (jj ? hi : lo)[kParts > 1 ? 1 : 0] = b1;
            (jj ? hi : lo)[kParts > 2 ? 2 : 0] = b2;
          }
        }
#pragma unroll
        for (int pp = 0; pp < kParts; ++pp) w[pp][j2] = lo[pp] | (hi[pp] << 16);
      }
#pragma unroll
      for (int pp = 0; pp < kParts; ++pp)
        ash[(st * kParts + pp) * 2048 + e] = uint4{w[pp][0], w[pp][1], w[pp][2], w[pp][3]};
    }
  }
  if constexpr (kCenter) {
    const FastSide &fs = a.sd[0];
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
      const float *mu = a.mean + h * D;
      if constexpr (KIND == KVQ_ROT_IDENTITY) {
        mrot[d] = mu[d];
      } else {
        double acc = 0.0;
        for (int k = 0; k < D; ++k) {
          double r;
          if constexpr (KIND == KVQ_ROT_SIGNED_HADAMARD)
            r = static_cast<double>(fs.signs[h * D + k]) * ((__popc(static_cast<unsigned>(k & d)) & 1) ? -1.0 : 1.0) *
                (1.0 / __builtin_sqrt(128.0));
          else
            r = static_cast<double>(fs.matrix[(static_cast<size_t>(h) * D + k) * D + d]);
          acc += static_cast<double>(mu[k]) * r;
        }
        // stored divided by the scale applied after the product (1/sqrt(128) for signed Hadamard)
        mrot[d] = static_cast<float>(KIND == KVQ_ROT_SIGNED_HADAMARD ? acc * __builtin_sqrt(128.0) : acc);
      }
    }
  }
  __syncthreads();

  const int64_t n_tiles = (a.T + 15) / 16;
  const int64_t tile_begin = run * kQTiles;
  const int64_t tile_end = min(tile_begin + kQTiles, n_tiles);
  const int64_t slots = a.num_pages * a.P;
  const size_t row_stride = static_cast<size_t>(a.H) * D;  // elements between tokens
  const float scale = KIND == KVQ_ROT_SIGNED_HADAMARD ? 0.08838834764831845f : 1.0f;  // 1/sqrt(128)
  const int qi = tk & 3;

  // this lane's 4 x 16 B of token tk of `tile` (B operand k-slices, or 32
  // dims for the identity) from x
  auto load_tile = [&](const uint16_t *x, int64_t tile, uint4 (&xb)[4]) {
    const int64_t t = min(tile * 16 + tk, a.T - 1);
    const uint16_t *row = x + static_cast<size_t>(t) * row_stride + static_cast<size_t>(h) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int off = KIND == KVQ_ROT_IDENTITY ? 32 * g + 8 * ks : 32 * ks + 8 * g;
      xb[ks] = *reinterpret_cast<const uint4 *>(row + off);
    }
  };
  // destination slot of token tk of `tile` (-1: not written)
  auto load_slot = [&](int64_t tile) -> int64_t {
    const int64_t tt = tile * 16 + tk;
    const int64_t t = min(tt, a.T - 1);
    return tt < a.T ? (a.slot_mapping ? a.slot_mapping[t] : t) : -1;
  };

  // rotated values y[nt][i] = dim 32g + 4nt + i of token tk (for the
  // identity: its 32 dims directly), from the staged rotation `st`; the
  // rotation slices are read from LDS right before their matrix-core steps
  auto rotate = [&](const uint4 (&x0)[4], int st, bool center, float (&y0)[8][4]) {
    if constexpr (KIND == KVQ_ROT_IDENTITY) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t w0[4] = {x0[ks].x, x0[ks].y, x0[ks].z, x0[ks].w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          y0[2 * ks + (j >> 2)][j & 3] = bf16_to_float((w0[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      }
    } else {
      const uint4 *as = ash + st * kParts * 2048;
      v4f acc0[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc0[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      // (one k-step's slices at a time: the scheduler barrier keeps the LDS
      // reads of later steps from being hoisted, which would cost registers)
#pragma unroll
      for (int step = 0; step < kParts * 4; ++step) {
        const v8bf b0 = __builtin_bit_cast(v8bf, x0[step & 3]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          acc0[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, as[(step * 8 + nt) * 64 + lane]),
                                                             b0, acc0[nt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) y0[nt][i] = acc0[nt][i];  // rotated value / scale (applied in finish)
    }
    if constexpr (kCenter) {
      if (center) {
        // mrot holds mu R / scale for rotated kinds (mu for the identity)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const float4 m = *reinterpret_cast<const float4 *>(&mrot[32 * g + 4 * nt]);
          const float mm[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) y0[nt][i] = y0[nt][i] - mm[i];
        }
      }
    }
  };

  // quantize, pack and write token tk of a tile from its rotated values
  // quantize, pack and write token tk of a tile from its rotated values, for
  // every clip ratio of the side (one cache each; statistics and
  // destination computed once)
  auto finish_tile = [&](float (&y)[8][4], int64_t slot, const FastSide &fs) {
    const int side = fs.side;
    // ---- group statistics of token tk (its 4 lanes g hold 32 dims each)
    float mn = y[0][0], mx = y[0][0];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mn = fminf(mn, y[nt][i]);
        mx = fmaxf(mx, y[nt][i]);
      }
    // across the token's 4 lanes (l, l^16, l^32, l^48) with VALU lane permutes
    {
      const auto n16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mn = fminf(__uint_as_float(n16[0]), __uint_as_float(n16[1]));
      mx = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
      const auto n32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mn = fminf(__uint_as_float(n32[0]), __uint_as_float(n32[1]));
      mx = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
    }
    if constexpr (KIND != KVQ_ROT_IDENTITY) {  // min / max of y = u * scale (scale > 0: monotone)
      mn = mn * scale;
      mx = mx * scale;
    }

    // ---- destination of token tk
    const bool valid = slot >= 0 && slot < slots;
    int64_t page = 0;
    int p = 0;
    if (valid) {
      if constexpr (kWide) {
        page = slot / a.P;
        p = static_cast<int>(slot - page * a.P);
      } else if (a.p_shift >= 0) {  // power-of-two page size
        const uint32_t us = static_cast<uint32_t>(slot);
        page = us >> a.p_shift;
        p = static_cast<int>(us & static_cast<uint32_t>(a.P - 1));
      } else {
        const uint32_t us = static_cast<uint32_t>(slot), up = static_cast<uint32_t>(a.P);
        const uint32_t pg = us / up;
        page = pg;
        p = static_cast<int>(us - pg * up);
      }
    }
    uint8_t *base0 = a.pages + (static_cast<size_t>(page) * a.H + h) * static_cast<size_t>(72 * a.P);
    // values: 4 consecutive tokens of a tile form one interleaved 128-byte V
    // group when their slots are 4 consecutive, 4-aligned positions; then the
    // quad's code bytes are transposed (lane qi takes bytes 8g+2qi, 8g+2qi+1
    // of all 4 tokens) and each lane writes 8 bytes; otherwise bytes singly
    int ok = 0;
    if (side != 0) {
      const int slot_lo = static_cast<int>(slot);
      const int s0 = __builtin_amdgcn_mov_dpp(slot_lo, 0x00, 0xF, 0xF, false);  // quad lane 0
      ok = (valid && slot_lo == s0 + qi && (s0 & 3) == 0) ? 1 : 0;
      ok &= qdpp_xor1(ok);
      ok &= qdpp_xor2(ok);
    }

    const int nclip = kClips ? a.nclip : 1;
    for (int ci = 0; ci < nclip; ++ci) {
      const float clip = fs.clip[ci];
      uint8_t *base = base0 + static_cast<size_t>(ci) * a.clip_stride;
      float lo = clip * mn;
      const float hi = clip * mx;
      const float span = hi - lo;
      float s32 = span / 3.0f;
      asm volatile("" : "+v"(lo));
      asm volatile("" : "+v"(s32));
      const _Float16 sh = static_cast<_Float16>(s32);
      const _Float16 zh = static_cast<_Float16>(lo);
      const float s = static_cast<float>(sh);
      const float z = static_cast<float>(zh);
      const float inv = s != 0.0f ? 1.0f / s : 0.0f;  // s == 0: every code is 0
      // rotated kinds: t = (u scale - z) inv computed as u (scale inv) - z inv
      const float si = scale * inv, zi = z * inv;

      // ---- codes, packed 16 per dword by shift-add of magic-biased values
      uint32_t cw[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t acc = 0;
#pragma unroll
        for (int nt = 3; nt >= 0; --nt)
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            float tq;
            if constexpr (KIND == KVQ_ROT_IDENTITY) {
              const float t = (y[4 * half + nt][i] - z) * inv;
              tq = __builtin_amdgcn_fmed3f(t, 0.0f, 3.0f) + kMagic;
            } else {
              const float t = __builtin_fmaf(y[4 * half + nt][i], si, -zi);
              tq = __builtin_amdgcn_fmed3f(t, 0.0f, 3.0f) + kMagic;
            }
            acc = (acc << 2) + __float_as_uint(tq);
          }
        cw[half] = acc - magic_pack_offset();
      }

      if (side == 0) {
        if (valid) *reinterpret_cast<uint2 *>(base + 32 * p + 8 * g) = uint2{cw[0], cw[1]};
      } else {
        const bool odd = (qi & 1) != 0, up2 = (qi & 2) != 0;
        const uint32_t L = cw[0], Hh = cw[1];
        const uint32_t r1 = static_cast<uint32_t>(qdpp_xor2(static_cast<int>(up2 ? L : Hh)));
        const uint32_t X0 = up2 ? r1 : L, X1 = up2 ? Hh : r1;
        const uint32_t sel_send = odd ? 0x05040100u : 0x07060302u;
        const uint32_t sel_keep = odd ? 0x07060302u : 0x05040100u;
        const uint32_t send = __builtin_amdgcn_perm(X1, X0, sel_send);
        const uint32_t keep = __builtin_amdgcn_perm(X1, X0, sel_keep);
        const uint32_t r2 = static_cast<uint32_t>(qdpp_xor1(static_cast<int>(send)));
        const uint32_t E = odd ? r2 : keep, O = odd ? keep : r2;
        const uint32_t W0 = __builtin_amdgcn_perm(O, E, 0x06020400u);
        const uint32_t W1 = __builtin_amdgcn_perm(O, E, 0x07030501u);
        uint8_t *vg = base + 32 * a.P + 128 * (p >> 2);
        if (ok) {
          *reinterpret_cast<uint2 *>(vg + 32 * g + 8 * qi) = uint2{W0, W1};
        } else if (valid) {
#pragma unroll
          for (int m = 0; m < 8; ++m)
            vg[4 * (8 * g + m) + (p & 3)] = static_cast<uint8_t>(cw[m >> 2] >> (8 * (m & 3)));
        }
      }
      if (valid && g == 0) {
        const uint32_t meta = f16_bits(sh) | (f16_bits(zh) << 16);
        *reinterpret_cast<uint32_t *>(base + (side ? 68 : 64) * a.P + 4 * p) = meta;
      }
    }
  };

  // wave w takes tiles w, w+8, ...; the next tile (both sides) is fetched
  // while one is rotated and written (past the end loads re-read the last tile)
  // (two sides: the next tile's keys are fetched before this tile's keys are
  // processed, its values before this tile's values, so at most three tiles
  // of inputs are held at once)
  int64_t tile = tile_begin + wave;
  if (tile >= tile_end) return;
  uint4 xa[kSides][4];
  int64_t sa = load_slot(tile);
#pragma unroll
  for (int sd = 0; sd < kSides; ++sd) load_tile(a.sd[sd].x, tile, xa[sd]);
  for (; tile < tile_end; tile += kQWavesF) {
    const int64_t nxt = min(tile + kQWavesF, tile_end - 1);
    const int64_t sna = load_slot(nxt);
#pragma unroll
    for (int sd = 0; sd < kSides; ++sd) {
      uint4 nx[4];
      load_tile(a.sd[sd].x, nxt, nx);
      float ya[8][4];
      rotate(xa[sd], kStaged > 1 ? sd : 0, sd == 0 && a.sd[sd].side == 0, ya);
      finish_tile(ya, sa, a.sd[sd]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) xa[sd][ks] = nx[ks];
    }
    sa = sna;
  }
}

template <int KIND, bool kCenter, int kSides, int kStaged>
hipError_t launch_fast_kind(const FastArgs &a, bool wide, hipStream_t stream) {
  if (a.nclip > 1 && wide) return hipErrorInvalidValue;  // (several clips: workspace caches, never that large)
  constexpr int kParts = KIND == KVQ_ROT_DENSE ? 3 : (KIND == KVQ_ROT_SIGNED_HADAMARD ? 1 : 0);
  const size_t lds = static_cast<size_t>(kStaged) * kParts * 2048 * sizeof(uint4);
  const int64_t n_tiles = (a.T + 15) / 16;
  const dim3 grid(static_cast<unsigned>((n_tiles + kQTiles - 1) / kQTiles * a.H));
  auto kern = a.nclip > 1 ? quantize_fast_kernel<KIND, kCenter, false, kSides, kStaged, true>
              : wide      ? quantize_fast_kernel<KIND, kCenter, true, kSides, kStaged, false>
                          : quantize_fast_kernel<KIND, kCenter, false, kSides, kStaged, false>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(64 * kQWavesF), lds, stream, a);
  return hipGetLastError();
}

template <int kSides, int kStaged>
hipError_t launch_fast_sides(const FastArgs &a, int kind, bool wide, hipStream_t stream) {
  const bool center = a.mean != nullptr;
  if constexpr (kStaged == 2) {  // two dense rotations do not fit in LDS together
    if (kind == KVQ_ROT_DENSE) return hipErrorInvalidValue;
  }
  if (kind == KVQ_ROT_IDENTITY)
    return center ? launch_fast_kind<KVQ_ROT_IDENTITY, true, kSides, kStaged>(a, wide, stream)
                  : launch_fast_kind<KVQ_ROT_IDENTITY, false, kSides, kStaged>(a, wide, stream);
  if (kind == KVQ_ROT_SIGNED_HADAMARD)
    return center ? launch_fast_kind<KVQ_ROT_SIGNED_HADAMARD, true, kSides, kStaged>(a, wide, stream)
                  : launch_fast_kind<KVQ_ROT_SIGNED_HADAMARD, false, kSides, kStaged>(a, wide, stream);
  if constexpr (kStaged == 1)
    return center ? launch_fast_kind<KVQ_ROT_DENSE, true, kSides, kStaged>(a, wide, stream)
                  : launch_fast_kind<KVQ_ROT_DENSE, false, kSides, kStaged>(a, wide, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quantize_clips(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                                 const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean,
                                 const float *clips_k, const float *clips_v, int nclip, uint8_t *pages,
                                 int64_t num_pages, int page_size, size_t clip_stride, hipStream_t stream) {
  if (num_tokens == 0 || nclip <= 0) return hipSuccess;
  if (dtype != KVQ_BF16) {
    // fp32 inputs: the exact kernel, one launch per clip ratio
    const int64_t items = num_tokens * H;
    int64_t blocks = (items + 3) / 4;
    if (blocks > 16384) blocks = 16384;
    for (int c = 0; c < nclip; ++c) {
      QuantArgs a{k, v, num_tokens, H, slot_mapping, rk, rv, key_mean, clips_k[c], clips_v[c],
                  pages + static_cast<size_t>(c) * clip_stride, num_pages, page_size, 1.0 / __builtin_sqrt(128.0)};
      hipLaunchKernelGGL(quantize_exact_kernel<KVQ_F32>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const bool wide = num_pages * static_cast<int64_t>(page_size) > (static_cast<int64_t>(1) << 31);
  int p_shift = -1;
  for (int sh = 4; sh < 31; ++sh)
    if (page_size == (1 << sh)) p_shift = sh;
  for (int c0 = 0; c0 < nclip; c0 += kMaxClips) {
    const int n = nclip - c0 < kMaxClips ? nclip - c0 : kMaxClips;
    FastSide sk{static_cast<const uint16_t *>(k), rk.signs, rk.matrix, {}, 0};
    FastSide sv{static_cast<const uint16_t *>(v), rv.signs, rv.matrix, {}, 1};
    for (int c = 0; c < n; ++c) {
      sk.clip[c] = clips_k[c0 + c];
      sv.clip[c] = clips_v[c0 + c];
    }
    uint8_t *pg = pages + static_cast<size_t>(c0) * clip_stride;
    hipError_t e;
    // keys and values in one pass when both rotations fit in LDS together
    // (signed Hadamard / identity, or one dense matrix shared by both sides);
    // otherwise one launch per side
    if (rk.kind == rv.kind && rk.kind != KVQ_ROT_DENSE) {
      e = launch_fast_sides<2, 2>(FastArgs{{sk, sv}, num_tokens, H, slot_mapping, key_mean, pg, num_pages, page_size,
                                           p_shift, n, clip_stride}, rk.kind, wide, stream);
    } else if (rk.kind == rv.kind && rk.matrix == rv.matrix) {
      e = launch_fast_sides<2, 1>(FastArgs{{sk, sv}, num_tokens, H, slot_mapping, key_mean, pg, num_pages, page_size,
                                           p_shift, n, clip_stride}, rk.kind, wide, stream);
    } else {
      e = launch_fast_sides<1, 1>(FastArgs{{sk, sk}, num_tokens, H, slot_mapping, key_mean, pg, num_pages, page_size,
                                           p_shift, n, clip_stride}, rk.kind, wide, stream);
      if (e == hipSuccess)
        e = launch_fast_sides<1, 1>(FastArgs{{sv, sv}, num_tokens, H, slot_mapping, nullptr, pg, num_pages,
                                             page_size, p_shift, n, clip_stride}, rv.kind, wide, stream);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                           const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean, float clip_k,
                           float clip_v, uint8_t *pages, int64_t num_pages, int page_size, hipStream_t stream) {
  return launch_quantize_clips(k, v, dtype, num_tokens, H, slot_mapping, rk, rv, key_mean, &clip_k, &clip_v, 1, pages,
                               num_pages, page_size, 0, stream);
}

}  // namespace kvq
