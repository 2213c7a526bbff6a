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
// tokens per split: a value-accumulator column of the matrix-core decode
// gains at most 128 (digit magnitude) x 48 (code in the 16x slot) per token,
// so one wave taking a whole split keeps its int32 sums below
// 2^18 * 6144 < 2^31
constexpr int kMaxMfmaSplitTokens = 1 << 18;
constexpr int kMaxSplits = 4096;            // split partials merged per (row, head)
constexpr int kMfmaWaves = 8;               // waves per workgroup of the matrix-core decode kernel
constexpr int kMaxSplitsNoPremerge = 1;     // more splits: the waves' partials are merged per split first (the last
                                             // split then loads one partial per split: 16 x 32K 59.3 -> 57.6 us,
                                             // 4 x 131K 78.1 -> 75.3 us against merging the 8 waves' partials of
                                             // up to 8 splits at the end)
constexpr int64_t kMaxSeqLen = static_cast<int64_t>(1) << 26;  // max_seq_len accepted by the decode entry point

// Groups of 4 query rows that one workgroup of the matrix-core decode takes
// (of n_rg per (sequence, KV head)): two when there are two or more, the
// pages hold 16 tokens and there are no BF16 windows, so that each block's
// codes are unpacked once for both groups and read by half as many
// workgroups (with longer pages the kernel's per-tile page offsets leave
// too few registers for two groups).  page_size 0: not known yet (a
// workspace size), which takes the choice with more splits.
inline int mfma_row_groups_per_workgroup(int n_rg, int page_size, bool windows) {
  return (!windows && n_rg >= 2 && page_size <= 16) ? 2 : 1;
}

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
// The value of lane (this lane ^ d) of a wave, d a power of two below 64,
// without the LDS: DPP moves within rows of 16 lanes (d = 4: a half-row
// mirror, lane i <- 7 - i, then lanes ^3 within quads, i.e. i <- i ^ 4) and
// VALU row swaps across rows (d = 16, 32: the swap returns this lane's own
// value and its partner's; the one that is not its own bits is the partner's,
// and when both are, they are the same value).  (Every source lane of these
// DPP patterns exists, so bound_ctrl changes nothing.)
__device__ __forceinline__ int lane_xor(int x, int d) {
  if (d == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);
  if (d == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);
  if (d == 4) return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true), 0x1B, 0xF, 0xF, true);
  if (d == 8) return __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);
  const unsigned u = static_cast<unsigned>(x);
  const auto r = d == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return static_cast<int>(r[0] == u ? r[1] : r[0]);
}
__device__ __forceinline__ float lane_xor(float x, int d) { return __int_as_float(lane_xor(__float_as_int(x), d)); }
// (each half of the double separately: the row swaps' value test picks the
// partner's half or, when the two halves agree, either)
__device__ __forceinline__ double lane_xor(double x, int d) {
  const long long b = __double_as_longlong(x);
  const int lo = lane_xor(static_cast<int>(b), d), hi = lane_xor(static_cast<int>(b >> 32), d);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// In-place fast Walsh-Hadamard transform: x <- x H, H[i][j] = (-1)^popcount(i & j)
// (Sylvester order, unnormalized): one butterfly stage per index bit.
template <typename T>
__device__ __forceinline__ void fwht128(T &x0, T &x1, int lane) {
  const T a = x0 + x1, b = x0 - x1;  // bit 6: pairs (lane, lane + 64)
  x0 = a;
  x1 = b;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const T p0 = lane_xor(x0, d), p1 = lane_xor(x1, d);
    const bool upper = (lane & d) != 0;
    x0 = upper ? p0 - x0 : x0 + p0;
    x1 = upper ? p1 - x1 : x1 + p1;
  }
}

// butterfly reductions: every lane ends with the same value
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += lane_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_maxf(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, lane_xor(x, o));
  return x;
}

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// Rotation kind used inside the library only: the query rows were already
// rotated and scaled by an earlier launch (rotate_query_wave leaves them alone).
constexpr int32_t kRotPrescaled = -1;

// q' = q R_K * log2(e)/sqrt(128) of one 128-vector held by a wave for the
// kinds without a matrix (identity, signed Hadamard, already rotated), with
// the head's signs s0 = s[lane], s1 = s[lane + 64] already loaded (signed
// Hadamard only): x <- (x * s) H / sqrt(128) by the transform above.
__device__ __forceinline__ void rotate_query_signed(float &x0, float &x1, int32_t kind, float s0, float s1,
                                                    int lane) {
  if (kind == kRotPrescaled) return;
  if (kind == KVQ_ROT_SIGNED_HADAMARD) {
    x0 *= s0;
    x1 *= s1;
    fwht128(x0, x1, lane);
    x0 *= kInvSqrtD;
    x1 *= kInvSqrtD;
  }
  x0 *= kLog2eF * kInvSqrtD;
  x1 *= kLog2eF * kInvSqrtD;
}

// q' = q R_K * log2(e)/sqrt(128) of one 128-vector held by a wave (row-vector
// convention z' = z R), every rotation kind.
__device__ __forceinline__ void rotate_query_wave(float &x0, float &x1, const RotDev &rk, int h, int lane) {
  if (rk.kind == KVQ_ROT_DENSE) {
    const float *m = rk.matrix + static_cast<size_t>(h) * D * D;
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll 8
    for (int i = 0; i < D; ++i) {
      const float zi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(i < 64 ? x0 : x1), i & 63));
      a0 += zi * m[i * D + lane];
      a1 += zi * m[i * D + lane + 64];
    }
    x0 = a0 * (kLog2eF * kInvSqrtD);
    x1 = a1 * (kLog2eF * kInvSqrtD);
    return;
  }
  float s0 = 1.0f, s1 = 1.0f;
  if (rk.kind == KVQ_ROT_SIGNED_HADAMARD) {
    s0 = static_cast<float>(rk.signs[h * D + lane]);
    s1 = static_cast<float>(rk.signs[h * D + lane + 64]);
  }
  rotate_query_signed(x0, x1, rk.kind, s0, s1, lane);
}

// ----------------------------------------------------------------- split merge
// A split partial of one (query row, query head) is 132 floats: m (base-2 log
// of the split's scale), l = sum_t 2^(x_t - m), z = sum_t 2^(x_t - m) z_t,
// a flag word, and acc[c] = sum_t 2^(x_t - m) s_t code_t[c], over the split's
// tokens t with x_t = logit_t in log2 units (l = NaN marks a bad input).

// Device-scope load of a split partial written by another workgroup (of
// this launch or an earlier one).
__device__ __forceinline__ float load_partial(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same for two consecutive floats (8-byte aligned): one 8-byte load.
__device__ __forceinline__ float2 load_partial2(const float *p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32))};
}

// Merge of the `parts` partials at p (stride 132 floats) into the
// rotated-domain output o'[c] = (sum_s 2^(m_s - m*) (acc_s[c] + z_s)) /
// (sum_s 2^(m_s - m*) l_s), m* = max_s m_s, held by one wave as
// o0 = o'[lane], o1 = o'[lane + 64]: 0 when no token counted, NaN when a
// partial flagged a bad input; the value sums are added in partial order.
// Few memory round trips, in two stages so that a caller can issue
// other loads between them (a wave's loads complete in issue order, so
// loads issued after merge_load do not delay the partials).  Up to 64
// partials: lane u holds partial u's (m, l, z); the value sums come in
// batches of 16 partials, lane l reading dims 2l and 2l + 1 of each (one
// 8-byte load per partial), the first two batches requested by merge_load
// together with the statistics: 34 loads, within the 63 a wave can have in
// flight, so 32 partials arrive in one round trip.  The sums are moved to
// the (l, l + 64) lane layout at the end.  More partials: merge_load
// requests nothing; the statistics in a lane loop, value sums in batches of
// 8 with their scales.
constexpr int kMergeBatch = 16;
struct MergeIn {
  float ma, la, za;           // partial `lane`'s statistics
  float2 xa[kMergeBatch];     // value sums of batches 0, 2, ... (dims 2 lane, 2 lane + 1)
  float2 xb[kMergeBatch];     // value sums of batches 1, 3, ...
};
// N partials per batch (N <= kMergeBatch; a caller that knows parts <= N
// requests fewer copies of the last one)
template <int N = kMergeBatch>
__device__ __forceinline__ void merge_fetch(const float *p, int parts, int lane, float2 *v, int u0) {
#pragma unroll
  for (int u = 0; u < N; ++u)
    v[u] = load_partial2(p + static_cast<size_t>(min(u0 + u, parts - 1)) * (D + 4) + 4 + 2 * lane);
}
template <int N = kMergeBatch>
__device__ __forceinline__ void merge_load(const float *p, int parts, int lane, MergeIn &in) {
  if (parts > 4 * N) return;
  in.ma = -INFINITY;
  in.la = in.za = 0.0f;
  if (lane < parts) {
    const float *q = p + static_cast<size_t>(lane) * (D + 4);
    const float2 ml = load_partial2(q);
    in.ma = ml.x;
    in.la = ml.y;
    in.za = load_partial(q + 2);
  }
  merge_fetch<N>(p, parts, lane, in.xa, 0);
  if (parts > N) merge_fetch<N>(p, parts, lane, in.xb, N);
}
template <int N = kMergeBatch>
__device__ __forceinline__ void merge_reduce(const float *p, int parts, int lane, MergeIn &in, float &o0, float &o1,
                                             float *m_out = nullptr, float *l_out = nullptr) {
  if (parts <= 4 * N) {
    constexpr int kB = N;
    const float mstar = wave_maxf(in.ma);
    const float wa = (in.ma == -INFINITY) ? 0.0f : exp2f(in.ma - mstar);
    const bool any_nan = __any(in.la != in.la);
    const float l = wave_sum(wa != 0.0f ? wa * in.la : 0.0f), z = wave_sum(wa != 0.0f ? wa * in.za : 0.0f);
    float e0 = 0.0f, e1 = 0.0f;  // dims 2 lane, 2 lane + 1
    auto accumulate = [&](const float2 *v, int u0) {
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (u0 + u >= parts) break;
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa), u0 + u));
        if (w != 0.0f) {
          e0 += w * v[u].x;
          e1 += w * v[u].y;
        }
      }
    };
    for (int u0 = 0; u0 < parts; u0 += 2 * kB) {
      accumulate(in.xa, u0);
      if (u0 + 2 * kB < parts) merge_fetch<N>(p, parts, lane, in.xa, u0 + 2 * kB);
      if (u0 + kB < parts) {
        accumulate(in.xb, u0 + kB);
        if (u0 + 3 * kB < parts) merge_fetch<N>(p, parts, lane, in.xb, u0 + 3 * kB);
      }
    }
    // dim d sits in lane d / 2 (component d % 2): lane l takes dims l and l + 64
    const int src0 = lane >> 1, src1 = 32 + (lane >> 1);
    const float p00 = __shfl(e0, src0), p01 = __shfl(e1, src0);
    const float p10 = __shfl(e0, src1), p11 = __shfl(e1, src1);
    const float a0 = (lane & 1) ? p01 : p00, a1 = (lane & 1) ? p11 : p10;
    o0 = (l > 0.0f) ? (a0 + z) / l : 0.0f;
    o1 = (l > 0.0f) ? (a1 + z) / l : 0.0f;
    if (any_nan) o0 = o1 = __builtin_nanf("");
    if (m_out) *m_out = mstar;
    if (l_out) *l_out = l;
    return;
  }
  constexpr int kU = 8;
  float mv[kU], av0[kU], av1[kU];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float *q = p + static_cast<size_t>(min(s0 + u, parts - 1)) * (D + 4);
      mv[u] = load_partial(q);
      av0[u] = load_partial(q + 4 + lane);
      av1[u] = load_partial(q + 4 + 64 + lane);
    }
  };
  fetch(0);
  float mloc = -INFINITY;
  bool nanloc = false;
  // split statistics: lane s2 holds split s2 (and s2 + 64, ...)
  for (int s2 = lane; s2 < parts; s2 += 64) mloc = fmaxf(mloc, load_partial(p + static_cast<size_t>(s2) * (D + 4)));
  const float mstar = wave_maxf(mloc);
  float lloc = 0.0f, zloc = 0.0f;
  for (int s2 = lane; s2 < parts; s2 += 64) {
    const float *q = p + static_cast<size_t>(s2) * (D + 4);
    const float m = load_partial(q), l = load_partial(q + 1), z = load_partial(q + 2);
    const float w = (m == -INFINITY) ? 0.0f : exp2f(m - mstar);
    if (l != l) nanloc = true;
    if (w != 0.0f) {
      lloc += w * l;
      zloc += w * z;
    }
  }
  const float l = wave_sum(lloc), z = wave_sum(zloc);
  const bool any_nan = __any(nanloc);
  float a0 = 0.0f, a1 = 0.0f;
  for (int s0 = 0; s0 < parts; s0 += kU) {
    if (s0 > 0) fetch(s0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + u >= parts) break;
      const float w = (mv[u] == -INFINITY) ? 0.0f : exp2f(mv[u] - mstar);
      if (w != 0.0f) {
        a0 += w * av0[u];
        a1 += w * av1[u];
      }
    }
  }
  o0 = (l > 0.0f) ? (a0 + z) / l : 0.0f;
  o1 = (l > 0.0f) ? (a1 + z) / l : 0.0f;
  if (any_nan) o0 = o1 = __builtin_nanf("");
  if (m_out) *m_out = mstar;
  if (l_out) *l_out = l;
}
template <int N = kMergeBatch>
__device__ __forceinline__ void merge_partials(const float *p, int parts, int lane, float &o0, float &o1,
                                               float *m_out = nullptr, float *l_out = nullptr) {
  MergeIn in;
  merge_load<N>(p, parts, lane, in);
  merge_reduce<N>(p, parts, lane, in, o0, o1, m_out, l_out);
}

// out = o' R_V^T of KV head h (one wave, same register layout as above).
__device__ __forceinline__ void unrotate_value_wave(float &o0, float &o1, const RotDev &rv, int h, int lane) {
  if (rv.kind == KVQ_ROT_SIGNED_HADAMARD) {
    // R[i][c] = s_i H[i][c] / sqrt(128), H symmetric: out = s * (o' H) / sqrt(128)
    fwht128(o0, o1, lane);
    o0 *= static_cast<float>(rv.signs[h * D + lane]) * kInvSqrtD;
    o1 *= static_cast<float>(rv.signs[h * D + lane + 64]) * kInvSqrtD;
  } else if (rv.kind == KVQ_ROT_DENSE) {
    // out[i] = sum_c o'[c] R[i][c]
    const float *m0 = rv.matrix + (static_cast<size_t>(h) * D + lane) * D;
    const float *m1 = m0 + 64 * D;
    float r0 = 0.0f, r1 = 0.0f;
    for (int c = 0; c < D; c += 4) {
      const float4 e0 = *reinterpret_cast<const float4 *>(m0 + c);
      const float4 e1 = *reinterpret_cast<const float4 *>(m1 + c);
      const float src = c < 64 ? o0 : o1;
      const int cl = c & 63;
      const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), cl));
      const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), cl + 1));
      const float v2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), cl + 2));
      const float v3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(src), cl + 3));
      r0 += v0 * e0.x + v1 * e0.y + v2 * e0.z + v3 * e0.w;
      r1 += v0 * e1.x + v1 * e1.y + v2 * e1.z + v3 * e1.w;
    }
    o0 = r0;
    o1 = r1;
  }
}

constexpr int kWoRows = 16;  // rows of o per W_O pass

// Writes the output of (row, query head j) to out_o [rows][Hq][128] and, when
// ot is not null, to the W_O operand copy laid out [row / 16][Hq * 128][16].
__device__ __forceinline__ void store_output_wave(float *out_o, float *ot, size_t row, int j, int Hq, int lane,
                                                  float r0, float r1) {
  const size_t K = static_cast<size_t>(Hq) * D;
  const size_t base = row * K + static_cast<size_t>(j) * D;
  out_o[base + lane] = r0;
  out_o[base + lane + 64] = r1;
  if (ot) {
    float *dst = ot + ((row / kWoRows) * K + static_cast<size_t>(j) * D) * kWoRows + row % kWoRows;
    dst[static_cast<size_t>(lane) * kWoRows] = r0;
    dst[static_cast<size_t>(lane + 64) * kWoRows] = r1;
  }
}

// ----------------------------------------------------------------- arrivals
// Arrival of one of `parts` workgroups at a shared counter: the high 32
// bits hold the epoch of the launch, the low 32 bits the arrivals; a word of
// another epoch (an earlier launch, or memory never written by this kernel)
// or an impossible count reads as zero arrivals.  The last arrival writes
// zero arrivals back, so a replay with the same epoch starts from zero as
// well.  The first exchange assumes that all other parts have arrived (one
// round trip for the last one, which goes on to combine their results); each
// failed exchange means the guess was wrong or another part arrived in
// between, so the loop runs at most `parts` + 1 times.  The caller makes its
// results visible at device scope before arriving.
__device__ __forceinline__ bool arrive_last(unsigned long long *cnt, uint32_t epoch, int parts) {
  const unsigned long long tag = static_cast<unsigned long long>(epoch) << 32;
  unsigned long long old = tag | static_cast<uint32_t>(parts - 1);
  for (;;) {
    uint32_t n = (old >> 32) == epoch ? static_cast<uint32_t>(old) : 0u;
    if (n >= static_cast<uint32_t>(parts)) n = 0;
    ++n;
    const unsigned long long want = n == static_cast<uint32_t>(parts) ? tag : (tag | n);
    const unsigned long long seen = atomicCAS(cnt, old, want);
    if (seen == old) return n == static_cast<uint32_t>(parts);
    old = seen;
  }
}
// Arrival counting without compare-and-swap retries (many workgroups may
// arrive at once): c[0] counts arrivals with one fetch-add each and is reset
// to 0 by the last arrival, so it starts every launch at 0 once c[1] holds
// the validation value of this counter (read by the caller at kernel start:
// `valid`).  A counter not yet validated (fresh workspace) counts with the
// tagged compare-and-swap on c[2] for one launch, whose last arrival then
// zeroes c[0] and validates it.  Every arrival of a launch reads the same c[1]:
// only the launch's last arrival writes it.
// The validation value depends on the counter's address and its number of
// parts, so a word validated by a launch of another shape does not count.
__device__ __forceinline__ unsigned long long arrival_valid_value(const unsigned long long *c, int parts) {
  return (static_cast<unsigned long long>(reinterpret_cast<uintptr_t>(c)) ^ 0x6b76715f61727276ull) +
         (static_cast<unsigned long long>(parts) << 48);
}
__device__ __forceinline__ bool arrive_counted(unsigned long long *c, bool valid, uint32_t epoch, int parts) {
  if (valid) {
    const unsigned long long old = atomicAdd(c, 1ull);
    if (old < static_cast<unsigned long long>(parts)) {
      const bool last = old == static_cast<unsigned long long>(parts - 1);
      if (last) __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return last;
    }
    // c[0] holds a value no launch of this counter leaves behind (the word
    // was part of another workspace layout since): every arrival of this
    // launch sees such a value (the count only grows) and counts with the
    // tagged compare-and-swap instead, whose last arrival resets c[0]
  }
  const bool last = arrive_last(c + 2, epoch, parts);
  if (last) {
    __hip_atomic_store(c, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(c + 1, arrival_valid_value(c, parts), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return last;
}
constexpr int kArrivalWords = 3;  // uint64 words per counted arrival point

// A new arrival tag per launch (host side), starting from a per-process value
// so that counters left in memory by other processes rarely carry it.
uint32_t next_launch_epoch();
// Compute units of the current device (read once per device and kept).
int device_cu_count();

// ----------------------------------------------------------------- launchers
hipError_t launch_quantize(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                           const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean, float clip_k,
                           float clip_v, uint8_t *pages, int64_t num_pages, int page_size, hipStream_t stream);
// The same cache write for several clip ratios at once (keys: clips_k[c],
// values: clips_v[c]), cache c at pages + c * clip_stride: one rotation and
// one set of group statistics per tile for all of them.
hipError_t launch_quantize_clips(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                                 const int64_t *slot_mapping, RotDev rk, RotDev rv, const float *key_mean,
                                 const float *clips_k, const float *clips_v, int nclip, uint8_t *pages,
                                 int64_t num_pages, int page_size, size_t clip_stride, hipStream_t stream);

struct DecodePlan {
  int num_seqs, queries_per_seq, Hq, H, G, rows_per_head;  // rows_per_head = queries_per_seq * G
  int max_seq_len, splits, split_tokens;                   // split_tokens % kChunk == 0
  int d_model;
  size_t off_qrot, off_qsum, off_part;                     // workspace layout (bytes)
  size_t off_ot;                                           // o laid out for the W_O projection
  size_t off_cnt;                                          // split arrival counters (matrix-core kernel)
  size_t total;
};
// page_size, windows: of the decode the plan is for (they decide the row
// groups per workgroup of the matrix-core kernel, and so the default split
// count); page_size 0 sizes a workspace for any page size.
DecodePlan make_decode_plan(int num_seqs, int queries_per_seq, int Hq, int H, int max_seq_len, int d_model,
                            int num_splits, int page_size = 16, bool windows = false);

// Rotated, pre-scaled queries and their sums (prologue of the decode step).
hipError_t launch_query_rotation(const void *q, int dtype, const DecodePlan &pl, RotDev rk, float *qrot,
                                 float *qsum, hipStream_t stream);
// Split-K partial attention over the packed cache.
hipError_t launch_decode_split(const DecodePlan &pl, const uint8_t *pages, int64_t num_pages, int page_size,
                               const int32_t *page_table, int max_pages, const int32_t *seq_lens,
                               const float *qrot, const float *qsum, float *part, hipStream_t stream);
// Matrix-core decode attention (one launch): per (sequence, KV head, group
// of 4 query rows) and split, the query rows are rotated (q and rk as in
// launch_query_rotation; rk.kind == kRotPrescaled takes q as rotated fp32
// rows), attended over the split's tokens, and the last split to finish
// merges all splits, applies R_V^T and writes out_o (and ot when not null).
// `counters` holds one 64-bit arrival counter per (sequence, KV head, row
// group); `epoch` tags this launch's arrivals (counters of another epoch
// count as zero; the last arrival leaves its counter at zero arrivals).
bool decode_mfma_supported(const DecodePlan &pl, int page_size);
// BF16 sink and recent windows of a decode (device pointers, bf16 bits).
struct WindowDev {
  const uint16_t *sink_k, *sink_v, *recent_k, *recent_v;
  int num_sink, num_recent;
  const float *key_mean;
};
constexpr int kMaxWindowTokens = 384;  // num_sink + num_recent (the merge holds them in registers)
hipError_t launch_decode_mfma(const DecodePlan &pl, const void *q, int dtype, RotDev rk, RotDev rv,
                              const uint8_t *pages, int64_t num_pages, int page_size, const int32_t *page_table,
                              int max_pages, const int32_t *seq_lens, float *part, uint64_t *counters,
                              float *out_o, float *ot, hipStream_t stream, const WindowDev *win = nullptr,
                              bool causal = false, float *y_zero = nullptr, int d_model = 0);
// Split-K partial attention over raw (unquantized, unrotated) K and V that
// every query row attends in full (reference readout of the candidate search).
hipError_t launch_reference_split(const DecodePlan &pl, const void *k, const void *v, int dtype,
                                  int64_t num_tokens, const float *qrot, float *part, hipStream_t stream);
// Merge splits, inverse value rotation, write out_o (and the W_O operand
// copy `ot` when not null).  y_zero (rows x pl.d_model, or null) is cleared
// for the W_O projection, which adds into it.
hipError_t launch_combine(const DecodePlan &pl, const float *part, RotDev rv, float *out_o, float *ot,
                          hipStream_t stream, float *y_zero = nullptr);
// out_y = concat(out_o) W_O on the matrix cores, from the copy `ot` written
// with out_o.  With several K slices the slices add into out_y, which the
// launch that wrote `ot` has cleared (y_zero).
hipError_t launch_wo_projection(const DecodePlan &pl, const float *ot, const void *w_o, int dtype, float *out_y,
                                hipStream_t stream);
int wo_kslices(int K);          // K slices of the W_O projection
int wo_col_blocks(int d_model); // column blocks of the W_O projection

// Candidate search helpers.
hipError_t launch_window_write(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                               const int32_t *seq_idx, const int32_t *positions, const int32_t *seq_lens,
                               int num_seqs, uint16_t *sink_k,
                               uint16_t *sink_v, uint16_t *recent_k, uint16_t *recent_v, int num_sink,
                               int num_recent, hipStream_t stream);
hipError_t launch_fold_value_rotation(const void *w, int dtype, int num_blocks, int blocks_per_head, int cols,
                                      RotDev rv, void *out, hipStream_t stream);
hipError_t launch_fill_i32(int32_t *p, int32_t value, int n, hipStream_t stream);
// Post-W_O NMSE through the Gram matrix of W_O (see candidate.hip):
// prepare once per search (Gram blocks and the reference output's norms),
// then one launch per variant.
size_t nmse_gram_floats(int Hq, int H, int mode);
hipError_t launch_nmse_prepare(const float *o_ref, const void *w_o, int dtype, int Nq, int Hq, int H, int d_model,
                               int mode, float *gram, double *den, hipStream_t stream);
hipError_t launch_nmse_terms(const float *o_hat, const float *o_ref, const float *gram, const double *den, int Nq,
                             int Hq, int H, int mode, int nvar, float *nmse_q_out, size_t stride_u,
                             hipStream_t stream);
hipError_t launch_select(const float *nmse_q, int U, int C, int n_clip, int Nq, float *out_nmse, int32_t *out_best,
                         hipStream_t stream);

}  // namespace kvq
