// decode_mfma.hip -- split-K decode attention over the packed INT2 cache on
// the gfx950 matrix cores (v_mfma_i32_16x16x64_i8), for up to 4 query rows
// per KV head (GQA groups of <= 4 heads, one query per sequence).
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization":
//   Appendix Eq. (21)-(22), (26): logit = (q R_K) . k_R / sqrt(128) against the
//   stored rotated keys; §3 Eq. (1)-(2): softmax over the cached tokens and the
//   probability-weighted sum of the (rotated) values.
//
// Arithmetic (exact integer contractions on the matrix cores):
//   keys:   dot(q', c_t) with q' in fixed point, Q = round(q' 2^S), |Q| <= 2^26,
//           written as 4 int8 digits (7 bits each, top digit signed); each
//           digit is one MFMA column, so one 16x16x64 MFMA contracts 64 key
//           dims of 16 tokens for 4 query rows x 4 digits.  Codes 0..3 are the
//           int8 A operand, extracted from the packed bytes with one mask per
//           2-bit slot; slots 1 and 2 come out multiplied by 4 and 16, which is
//           divided out of the query digits of those dims.  Digits are
//           recombined in fp32 by a reduce-scatter inside each 4-lane quad,
//           after which every lane owns 4 distinct tokens.
//   values: sum_t w_t c_t with w_t = 2^(logit_t + kappa) s_t rounded to an
//           integer < 2^28 and split into 4 unsigned 7-bit digits (MFMA
//           columns); kappa is a per-row power-of-two scale chosen from a
//           running bound of logit + log2(s) with 2^6 of headroom, so the sums
//           stay exact int32 in the MFMA accumulators; if the bound outgrows the
//           headroom the accumulators are flushed to fp32 in LDS (rare) and the
//           scale moves.  l = sum 2^(logit+kappa) and z = sum 2^(logit+kappa) z_t
//           stay in fp32 per lane.
// Loads are branch-free (tiles past the end are clamped into the last valid
// tile and masked) and the next 64-token block is fetched while the current
// one is computed.  The per-split result is written in the same
// (m, l, z, acc[128]) form as the VALU kernel, with m = -kappa, and merged by
// the same combine kernel.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kM0 = 0x03030303u, kM1 = 0x0C0C0C0Cu, kM2 = 0x30303030u;
constexpr int kHeadroom = 6;  // log2 headroom of the value scale

// The 4 code slots of every byte of x as int8 lanes; slot 1 and 2 are scaled by 4 and 16.
__device__ __forceinline__ v4i slots(uint32_t x) {
  return v4i{static_cast<int>(x & kM0), static_cast<int>(x & kM1), static_cast<int>(x & kM2),
             static_cast<int>((x >> 6) & kM0)};
}
__device__ __forceinline__ int slot(uint32_t x, int e) {
  return static_cast<int>(e == 0 ? (x & kM0) : e == 1 ? (x & kM1) : e == 2 ? (x & kM2) : ((x >> 6) & kM0));
}
__device__ __forceinline__ float slot_inv(int e) { return e == 1 ? 0.25f : e == 2 ? 0.0625f : 1.0f; }

__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_xor1f(float v) { return __int_as_float(dpp_xor1(__float_as_int(v))); }
__device__ __forceinline__ float dpp_xor2f(float v) { return __int_as_float(dpp_xor2(__float_as_int(v))); }

// max / sum over the 16 lanes of one query row (4 quad lanes x 4 lane groups)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_xor1f(x));
  x = fmaxf(x, dpp_xor2f(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_xor1f(x);
  x += dpp_xor2f(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

struct MfmaArgs {
  int R, G, Hq, H, Nq;
  int split_tokens, splits, max_seq_len;
  const uint8_t *pages;
  int64_t num_pages;
  int P;
  const int32_t *page_table;
  int max_pages;
  const int32_t *seq_lens;
  const int32_t *qdig;  // [num_seqs][H][64 lanes][8] key-side B operand
  const int32_t *qexp;  // [num_seqs][H][4 rows] fixed-point shift S of each query row
  const float *qsum;
  float *part;
};

// Fixed-point digits of the rotated queries of one (sequence, KV head): lane
// (col, grp) gets the 8 dwords of its B-operand column (row col/4, digit col%4)
// for the two 64-dim MFMAs.  Dim 16*(2*grp + m) + 4*bb + e goes to dword
// [m][e], byte bb; slot e of the unpacked codes carries a factor 1/slot_inv(e),
// which is divided out here.  Q = round(q' 2^S) with |Q| <= 2^26.
__global__ __launch_bounds__(64) void query_digits_kernel(const float *qrot, int R, int G, int Hq, int H, int Nq,
                                                          int32_t *qdig, int32_t *qexp) {
  const int bh = blockIdx.x;  // b * H + h
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4, hr = col >> 2, dg = col & 3;
  const bool row_ok = hr < R;
  const size_t rj = (static_cast<size_t>(b) * Nq + hr / G) * Hq + h * G + hr % G;
  float qv[2][16];
  float qabs = 0.0f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float x = row_ok ? qrot[rj * D + 16 * (2 * grp + m) + 4 * bb + e] : 0.0f;
        qv[m][4 * e + bb] = x * slot_inv(e);
        qabs = fmaxf(qabs, fabsf(x));
      }
  qabs = fmaxf(qabs, __shfl_xor(qabs, 16));
  qabs = fmaxf(qabs, __shfl_xor(qabs, 32));
  int e2 = 0;
  (void)frexpf(qabs, &e2);  // qabs < 2^e2
  const int qshift = 26 - e2;
  int32_t *dst = qdig + (static_cast<size_t>(bh) * 64 + lane) * 8;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t word = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int Q = static_cast<int>(__builtin_rintf(ldexpf(qv[m][4 * e + bb], qshift)));
        const int dig = (dg == 0) ? (Q >> 21) : ((Q >> (21 - 7 * dg)) & 127);
        word |= (static_cast<uint32_t>(dig) & 0xffu) << (8 * bb);
      }
      dst[4 * m + e] = static_cast<int32_t>(word);
    }
  if (grp == 0 && dg == 0) qexp[static_cast<size_t>(bh) * 4 + hr] = qshift;
}

constexpr int kWaves = 4;
constexpr int kBlk = 64;  // tokens per wave iteration (4 tiles of 16)
constexpr int kMaxSplitTiles = kMaxMfmaSplitTokens / 16;
constexpr int kSlackTiles = (kWaves * kBlk) / 16 + 4;  // page ids read past the split end by the prefetch

// Per-lane data of one 64-token block.
struct Blk {
  uint2 kc[4];        // K codes: token `col` of tile q, bytes 8*grp .. 8*grp+7
  uint32_t vx[4][2];  // V codes: 4-group `grp` of tile q, dwords 2*col and 2*col+1 (dims 8*col..8*col+7)
  uint4 km, vm;       // K / V metadata of tokens 4*grp..4*grp+3 of tile dg
};

struct Ctx {
  const MfmaArgs *a;
  int b, h, col, grp, dg;
  int t_end, t_last;  // t_last: first token of the last tile that holds a valid token
  size_t block_bytes;
};

// Page ids of the split's 16-token tiles, validated and clamped into the last
// valid tile, are staged in shared memory by the workgroup prologue.
__device__ __forceinline__ void load_block(const Ctx &c, int t0, const int *tile_page, int t_begin, Blk &o) {
  const MfmaArgs &a = *c.a;
  const uint8_t *bp[4];
  int off[4];
  const int4 pid = *reinterpret_cast<const int4 *>(tile_page + (t0 - t_begin) / 16);
  const int pids[4] = {pid.x, pid.y, pid.z, pid.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tt = min(t0 + 16 * q, c.t_last);  // clamped into a valid tile (masked later)
    off[q] = static_cast<int>(static_cast<unsigned>(tt) % static_cast<unsigned>(a.P));
    bp[q] = a.pages + (static_cast<size_t>(pids[q]) * a.H + c.h) * c.block_bytes;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o.kc[q] = *reinterpret_cast<const uint2 *>(bp[q] + 32 * (off[q] + c.col) + 8 * c.grp);
    const uint2 v = *reinterpret_cast<const uint2 *>(bp[q] + 32 * a.P + 128 * ((off[q] >> 2) + c.grp) + 8 * c.col);
    o.vx[q][0] = v.x;
    o.vx[q][1] = v.y;
  }
  const uint8_t *ob = c.dg == 0 ? bp[0] : c.dg == 1 ? bp[1] : c.dg == 2 ? bp[2] : bp[3];
  const int oo = c.dg == 0 ? off[0] : c.dg == 1 ? off[1] : c.dg == 2 ? off[2] : off[3];
  o.km = *reinterpret_cast<const uint4 *>(ob + 64 * a.P + 4 * (oo + 4 * c.grp));
  o.vm = *reinterpret_cast<const uint4 *>(ob + 68 * a.P + 4 * (oo + 4 * c.grp));
}

struct State {
  v4i bk[2];        // key-side B operand (query digits), dims half m
  float qsum;       // sum of q' (for the zero-point term)
  float unscale;    // weight of this lane's key digit / 2^S
  v4i accv[8];      // value accumulators (int32, MFMA), 16 dims each
  float lsum, zsum;
  int kappa;
  bool have_ref;
};

__device__ __forceinline__ void compute_block(const Ctx &c, int t0, const Blk &blk, State &st, float *facc) {
  // ---- key side: 2 MFMAs per tile (64 dims each)
  v4i dk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    dk[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(slots(blk.kc[q].x), st.bk[0], v4i{0, 0, 0, 0}, 0, 0, 0);
    dk[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(slots(blk.kc[q].y), st.bk[1], dk[q], 0, 0, 0);
  }
  // ---- digits -> fp32, reduce-scatter inside the quad: lane keeps tile dg
  const bool hiA = (c.dg & 2) != 0, hiB = (c.dg & 1) != 0;
  float k2[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lo = static_cast<float>(dk[j][r]) * st.unscale;
      const float hi = static_cast<float>(dk[j + 2][r]) * st.unscale;
      const float send = hiA ? lo : hi;
      const float keep = hiA ? hi : lo;
      k2[j][r] = keep + dpp_xor2f(send);
    }
  float dot[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float send = hiB ? k2[0][r] : k2[1][r];
    const float keep = hiB ? k2[1][r] : k2[0][r];
    dot[r] = keep + dpp_xor1f(send);
  }

  // ---- logits of the 4 owned tokens (base-2 units); bound u = logit + log2 bound of s_v
  float logit[4], sv[4], zv[4];
  float umax = -INFINITY;
  const uint32_t kmw[4] = {blk.km.x, blk.km.y, blk.km.z, blk.km.w};
  const uint32_t vmw[4] = {blk.vm.x, blk.vm.y, blk.vm.z, blk.vm.w};
  const int tok0 = t0 + 16 * c.dg + 4 * c.grp;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float ks = half_bits_to_float(kmw[r] & 0xffffu), kz = half_bits_to_float(kmw[r] >> 16);
    sv[r] = half_bits_to_float(vmw[r] & 0xffffu);
    zv[r] = half_bits_to_float(vmw[r] >> 16);
    logit[r] = (tok0 + r < c.t_end) ? dot[r] * ks + kz * st.qsum : -INFINITY;
    const int es = static_cast<int>((vmw[r] >> 10) & 31u) - 14;  // s_v < 2^es
    umax = fmaxf(umax, logit[r] + static_cast<float>(es));
  }
  umax = row16_max(umax);
  int need = st.kappa;
  if (umax != -INFINITY) {
    need = 27 - static_cast<int>(ceilf(umax));
    if (!st.have_ref) {
      st.kappa = need - kHeadroom;
      st.have_ref = true;
    }
  }
  // wave-uniform decision: flush when any row outgrew its headroom
  if (__any(st.have_ref && need < st.kappa)) {
    const int newk = (st.have_ref && need < st.kappa) ? need - kHeadroom : st.kappa;
    const float f2 = ldexpf(1.0f, newk - st.kappa);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *p = facc + (4 * i + r) * 64;
        *p = (*p + static_cast<float>(st.accv[i][r])) * f2;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) st.accv[i] = v4i{0, 0, 0, 0};
    st.lsum *= f2;
    st.zsum *= f2;
    st.kappa = newk;
  }
  // ---- weights: p = 2^(logit + kappa), W = round(p s_v) < 2^28, 4 digits packed per tile
  uint32_t dw[4] = {0, 0, 0, 0};
  const float kf = static_cast<float>(st.kappa);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = exp2f(logit[r] + kf);
    st.lsum += p;
    st.zsum += p * zv[r];
    const uint32_t W = static_cast<uint32_t>(p * sv[r] + 0.5f);
    dw[0] |= __builtin_amdgcn_ubfe(W, 21, 7) << (8 * r);
    dw[1] |= __builtin_amdgcn_ubfe(W, 14, 7) << (8 * r);
    dw[2] |= __builtin_amdgcn_ubfe(W, 7, 7) << (8 * r);
    dw[3] |= (W & 127u) << (8 * r);
  }
  // quad transpose: lane dg gets digit dg of every tile (dword q from quad lane q)
  {
    const bool odd = (c.dg & 1) != 0, hi2 = (c.dg & 2) != 0;
    const uint32_t x0 = dpp_xor1(dw[0]), x1 = dpp_xor1(dw[1]), x2 = dpp_xor1(dw[2]), x3 = dpp_xor1(dw[3]);
    const uint32_t t0v = odd ? x1 : dw[0], t1v = odd ? dw[1] : x0, t2v = odd ? x3 : dw[2], t3v = odd ? dw[3] : x2;
    const uint32_t y0 = dpp_xor2(t0v), y1 = dpp_xor2(t1v), y2 = dpp_xor2(t2v), y3 = dpp_xor2(t3v);
    dw[0] = hi2 ? y2 : t0v;
    dw[1] = hi2 ? y3 : t1v;
    dw[2] = hi2 ? t2v : y0;
    dw[3] = hi2 ? t3v : y1;
  }
  const v4i bv{static_cast<int>(dw[0]), static_cast<int>(dw[1]), static_cast<int>(dw[2]), static_cast<int>(dw[3])};

  // ---- value side: 8 MFMAs (16 dims each), k = the 64 tokens of the block
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const v4i av{slot(blk.vx[0][hf], e), slot(blk.vx[1][hf], e), slot(blk.vx[2][hf], e), slot(blk.vx[3][hf], e)};
      st.accv[4 * hf + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, st.accv[4 * hf + e], 0, 0, 0);
    }
}

template <bool kPaged>
__global__ __launch_bounds__(256) void decode_mfma_kernel(MfmaArgs a) {
  __shared__ float red[kWaves][4][4 + D];  // per wave, per row: m, l, z, flag, acc[128]
  __shared__ float facc_all[kWaves][32 * 64];  // flushed value accumulators, [slot][lane]
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  Ctx c;
  c.a = &a;
  c.b = b;
  c.h = h;
  c.col = lane & 15;
  c.grp = lane >> 4;
  c.dg = c.col & 3;
  const int hr = c.col >> 2;  // query row of this lane's column
  float *facc = &facc_all[wave][lane];

  int L = a.seq_lens[b];
  bool bad = L < 0 || L > a.max_seq_len;
  if (bad) L = 0;
  const int t_begin = s * a.split_tokens;
  c.t_end = min(t_begin + a.split_tokens, L);
  c.t_last = c.t_end > 0 ? ((c.t_end - 1) / 16) * 16 : 0;
  c.block_bytes = static_cast<size_t>(72) * a.P;

  // ---- precomputed query digits of this lane's column (key-side B operand)
  State st;
  const bool row_ok = hr < a.R;
  const int qi = hr / a.G, gh = hr % a.G;
  const size_t rj = (static_cast<size_t>(b) * a.Nq + qi) * a.Hq + h * a.G + gh;
  {
    const int4 *dsrc = reinterpret_cast<const int4 *>(a.qdig + ((static_cast<size_t>(b) * a.H + h) * 64 + lane) * 8);
    const int4 d0 = dsrc[0], d1 = dsrc[1];
    st.bk[0] = v4i{d0.x, d0.y, d0.z, d0.w};
    st.bk[1] = v4i{d1.x, d1.y, d1.z, d1.w};
  }
  const int qshift = a.qexp[(static_cast<size_t>(b) * a.H + h) * 4 + hr];
  st.qsum = row_ok ? a.qsum[rj] : 0.0f;
  st.unscale = ldexpf(1.0f, 21 - 7 * c.dg - qshift);
#pragma unroll
  for (int i = 0; i < 8; ++i) st.accv[i] = v4i{0, 0, 0, 0};
  st.lsum = st.zsum = 0.0f;
  st.kappa = 0;
  st.have_ref = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) facc[i * 64] = 0.0f;

  // ---- page id of every 16-token tile of the split, validated; entries past
  // the end (read by the over-fetch of the last block) clamp to the last tile
  __shared__ __attribute__((aligned(16))) int tile_page[kMaxSplitTiles + kSlackTiles];
  __shared__ int page_fault;
  if (threadIdx.x == 0) page_fault = 0;
  __syncthreads();
  if (c.t_end > t_begin) {
    const int n_fill = (c.t_end - t_begin + 15) / 16 + kSlackTiles;
    for (int i = threadIdx.x; i < n_fill; i += 256) {
      const int tt = min(t_begin + 16 * i, c.t_last);
      const int pi = tt / a.P;
      int64_t p = kPaged ? static_cast<int64_t>(a.page_table[static_cast<size_t>(b) * a.max_pages + pi])
                         : static_cast<int64_t>(b) * a.max_pages + pi;
      if (p < 0 || p >= a.num_pages) {
        page_fault = 1;
        p = 0;
      }
      tile_page[i] = static_cast<int>(p);
    }
  }
  __syncthreads();
  if (page_fault) bad = true;

  // ---- main loop: wave w takes blocks w, w+4, ...; the next block is always
  // fetched while the current one is computed (past the end it re-reads the
  // clamped last tile, which is masked)
  // (the trip count is fixed up front so the loop has a single exit and the
  // prefetched block is the only load in flight across the back edge)
  constexpr int kStride = kWaves * kBlk;
  int t0 = t_begin + wave * kBlk;
  const int n_blk = t0 < c.t_end ? (c.t_end - t0 + kStride - 1) / kStride : 0;
  if (n_blk > 0) {
    Blk b0, b1;
    load_block(c, t0, tile_page, t_begin, b0);
    for (int i = 0; i < n_blk / 2; ++i) {
      load_block(c, t0 + kStride, tile_page, t_begin, b1);
      compute_block(c, t0, b0, st, facc);
      load_block(c, t0 + 2 * kStride, tile_page, t_begin, b0);
      compute_block(c, t0 + kStride, b1, st, facc);
      t0 += 2 * kStride;
    }
    if (n_blk & 1) compute_block(c, t0, b0, st, facc);
  }

  // ---- per-wave result for each row: totals over the row's 16 lanes, digits recombined
  const float lrow = row16_sum(st.lsum);
  const float zrow = row16_sum(st.zsum);
  const float wdig = ldexpf(1.0f, 21 - 7 * c.dg);
  const bool any_bad = __any(bad);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * hf + e;
        float x = (facc[(4 * i + r) * 64] + static_cast<float>(st.accv[i][r])) * (wdig * slot_inv(e));
        x += dpp_xor1f(x);
        x += dpp_xor2f(x);
        if (c.dg == 0 && row_ok) red[wave][hr][4 + 8 * (4 * c.grp + r) + 4 * hf + e] = x;
      }
  if (c.dg == 0 && c.grp == 0 && row_ok) {
    red[wave][hr][0] = st.have_ref ? -static_cast<float>(st.kappa) : -INFINITY;
    red[wave][hr][1] = lrow;
    red[wave][hr][2] = zrow;
    red[wave][hr][3] = any_bad ? 1.0f : 0.0f;
  }
  __syncthreads();

  // ---- merge the 4 waves (base-2 log-sum-exp) and write this split's partial
  for (int idx = threadIdx.x; idx < a.R * D; idx += 256) {
    const int r = idx / D, i = idx % D;
    float mstar = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mstar = fmaxf(mstar, red[w][r][0]);
      nan = nan || red[w][r][3] != 0.0f;
    }
    float l = 0.0f, z = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (red[w][r][0] == -INFINITY) continue;
      const float sc = exp2f(red[w][r][0] - mstar);
      l += sc * red[w][r][1];
      z += sc * red[w][r][2];
      acc += sc * red[w][r][4 + i];
    }
    const int qq = r / a.G, g2 = r % a.G;
    const size_t row = static_cast<size_t>(b) * a.Nq + qq;
    float *dst = a.part + ((row * a.Hq + h * a.G + g2) * a.splits + s) * (D + 4);
    dst[4 + i] = mstar == -INFINITY ? 0.0f : acc;
    if (i == 0) {
      dst[0] = mstar;
      dst[1] = nan ? __builtin_nanf("") : (mstar == -INFINITY ? 0.0f : l);
      dst[2] = mstar == -INFINITY ? 0.0f : z;
      dst[3] = 0.0f;
    }
  }
}

}  // namespace

bool decode_mfma_supported(const DecodePlan &pl, int page_size) {
  return pl.rows_per_head <= 4 && page_size % 16 == 0;
}

hipError_t launch_query_digits(const DecodePlan &pl, const float *qrot, int32_t *qdig, int32_t *qexp,
                               hipStream_t stream) {
  const int n = pl.num_seqs * pl.H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(query_digits_kernel, dim3(n), dim3(64), 0, stream, qrot, pl.rows_per_head, pl.G, pl.Hq, pl.H,
                     pl.queries_per_seq, qdig, qexp);
  return hipGetLastError();
}

hipError_t launch_decode_split_mfma(const DecodePlan &pl, const uint8_t *pages, int64_t num_pages, int page_size,
                                    const int32_t *page_table, int max_pages, const int32_t *seq_lens,
                                    const int32_t *qdig, const int32_t *qexp, const float *qsum, float *part,
                                    hipStream_t stream) {
  if (pl.num_seqs == 0) return hipSuccess;
  MfmaArgs a{};
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
  a.qdig = qdig;
  a.qexp = qexp;
  a.qsum = qsum;
  a.part = part;
  if (page_table)
    hipLaunchKernelGGL(decode_mfma_kernel<true>, dim3(pl.splits, pl.H, pl.num_seqs), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_mfma_kernel<false>, dim3(pl.splits, pl.H, pl.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
