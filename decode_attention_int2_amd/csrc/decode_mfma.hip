// decode_mfma.hip -- split-K decode attention over the packed INT2 cache on
// the gfx950 matrix cores (v_mfma_i32_16x16x64_i8), for up to 4 query rows
// per KV head (GQA groups of <= 4 heads, one query per sequence).
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization":
//   Appendix Eq. (21)-(22), (26): logit = (q R_K) . k_R / sqrt(128) against the
//   stored rotated keys; §3 Eq. (1)-(2): softmax over the cached tokens and the
//   probability-weighted sum of the (rotated) values.
//
// Lane l = 16 g + c of a wave.  A wave takes 64-token blocks (4 tiles of 16).
// Keys (exact integer products):
//   q' is held in fixed point, Q = round(q' 2^S), |Q| <= 2^26, as 4 int8
//   digits (7 bits, top digit signed).  The MFMA's A operand is the digits
//   (row 4 r + d = digit d of query row r), its B operand the codes of 16
//   tokens (column = token), k = 64 key dims; codes 0..3 are extracted from
//   the packed bytes with one mask per 2-bit slot (slots 1 and 2 come out
//   multiplied by 4 and 16, which the digits divide out).  Lane (c, g) thus
//   receives the 4 digit sums of query row g against token c of the tile and
//   forms the logit alone: no cross-lane reduction.
// Values:
//   w_t = 2^(logit_t + kappa) s_t rounded to an integer < 2^24 is split into
//   its 3 bytes; each byte b is fed as the int8 b - 128, and a fourth column
//   of ones accumulates sum_t c_t to undo the offset.  kappa is a per-row
//   power-of-two scale chosen from a running bound of logit + log2(s) with
//   2^2 of headroom; if the bound outgrows it the int32 accumulators are
//   flushed to fp32 in LDS (rare) and the scale moves.  l = sum 2^(logit +
//   kappa) and z = sum 2^(logit + kappa) z_t stay in fp32 per lane.  The bytes
//   reach the MFMA's B layout (column 4 r + byte, k = 16 tokens per lane
//   group) by a byte transpose inside each lane quad and one lane permutation.
// Addresses: a small kernel resolves the page of every 16-token tile once per
// decode step into absolute code / metadata base addresses; the split kernel
// reads them with scalar loads and issues every vector load as scalar base +
// per-lane constant offset.  The next 64-token block is fetched while the
// current one is computed; tiles past the split end are clamped into its last
// tile and masked.  The per-split result is written in the same (m, l, z,
// acc[128]) form as the VALU kernel, with m = -kappa, and merged by the same
// combine kernel.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr uint32_t kM0 = 0x03030303u, kM1 = 0x0C0C0C0Cu, kM2 = 0x30303030u;
constexpr int kHeadroom = 2;       // log2 headroom of the value scale
constexpr int kWeightBits = 24;    // value weights are integers < 2^24 (3 bytes)
constexpr uint32_t kByteOffset = 0x01808080u;  // bytes 0-2: b -> b - 128 as int8; byte 3: the ones column

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
__device__ __forceinline__ int dpp_ror4(int v) { return __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_ror8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false); }
__device__ __forceinline__ float fdpp_xor1(float v) { return __int_as_float(dpp_xor1(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_xor2(float v) { return __int_as_float(dpp_xor2(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_ror4(float v) { return __int_as_float(dpp_ror4(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_ror8(float v) { return __int_as_float(dpp_ror8(__float_as_int(v))); }

// max / sum over the 16 lanes of a DPP row (rotations reach every lane of the row)
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, fdpp_xor1(x));
  x = fmaxf(x, fdpp_xor2(x));
  x = fmaxf(x, fdpp_ror4(x));
  x = fmaxf(x, fdpp_ror8(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += fdpp_xor1(x);
  x += fdpp_xor2(x);
  x += fdpp_ror4(x);
  x += fdpp_ror8(x);
  return x;
}

// 4x4 byte transpose inside each lane quad: afterwards byte j of quad lane x
// is byte x of quad lane j before.  sel1/sel2 are the lane's v_perm selectors.
__device__ __forceinline__ uint32_t quad_byte_transpose(uint32_t a, uint32_t sel1, uint32_t sel2) {
  a = __builtin_amdgcn_perm(static_cast<uint32_t>(dpp_xor1(static_cast<int>(a))), a, sel1);
  a = __builtin_amdgcn_perm(static_cast<uint32_t>(dpp_xor2(static_cast<int>(a))), a, sel2);
  return a;
}

// Sum over tokens of (byte x of W) * code for value-accumulator lane x of a
// quad (x < 3): the MFMA summed (byte - 128) * code, the quad's lane 3 holds
// sum code; the correction is applied in int32 (|.| < 2^31 over a split) so
// that no large offset is cancelled in fp32.  Lane x = 3 yields 0.
__device__ __forceinline__ int byte_sum(int d, int x) {
  const int ones = __builtin_amdgcn_mov_dpp(d, 0xFF, 0xF, 0xF, false);  // quad lane 3
  return x < 3 ? d + 128 * ones : 0;
}

struct MfmaArgs {
  int R, G, Hq, H, Nq, n_rg;  // n_rg: groups of 4 query rows per KV head
  int split_tokens, splits, max_seq_len;
  int P;
  int tiles_per_seq;
  const int32_t *seq_lens;
  const int32_t *qdig;     // [num_seqs][H][n_rg][64 lanes][8] key-side A operand
  const int32_t *qexp;     // [num_seqs][H][n_rg][4 rows] fixed-point shift S of each query row
  const float *qsum;
  const uint64_t *tiles;   // [num_seqs][tiles_per_seq][2] code base, metadata base (bit 0: bad page)
  float *part;
};

// Prologue of the split kernel, one launch:
//  * blocks [0, num_seqs*H*n_rg): one per (sequence, KV head, group of 4
//    query rows).  Wave r rotates row 4 rg + r of the head's R rows (q' = q R_K
//    log2(e)/sqrt(128)), writes q' and sum(q'); then wave 0 writes the
//    fixed-point int8 digits of the group's rows in the key-side A-operand
//    layout: lane (col, grp) gets the 8 dwords of query row col/4, digit
//    col%4, for the two 64-dim MFMAs; dim 16*(2*grp + m) + 4*bb + e goes to
//    dword [m][e], byte bb.  Slot e of the unpacked codes carries a factor
//    1/slot_inv(e), divided out here.  Q = round(q' 2^S) with |Q| < 2^26 (S
//    per query row from its largest |q'|).
//  * the remaining blocks: absolute addresses of every 16-token tile of every
//    sequence (head 0 of its page; the head's offset is part of the lanes'
//    constant offsets):
//      [0] page block + 32 * (position of the tile in its page)   K/V codes
//      [1] page block + 64 P + 4 * (position)                     K/V metadata
//    A page index outside the cache is replaced by page 0 and flagged in
//    bit 0 of the metadata address.
struct PrologueArgs {
  const void *q;
  RotDev rk;
  int R, G, Hq, H, Nq, num_seqs, n_rg;
  float *qrot, *qsum;
  int32_t *qdig, *qexp;
  const uint8_t *pages;
  int64_t num_pages;
  int P;
  const int32_t *page_table;
  int max_pages, tiles_per_seq, table_chunks;
  uint64_t *tiles;
};

template <int DT>
__global__ __launch_bounds__(256) void decode_prologue_kernel(PrologueArgs p) {
  const int n_bh = p.num_seqs * p.H * p.n_rg;
  if (static_cast<int>(blockIdx.x) >= n_bh) {
    const int idx = blockIdx.x - n_bh;
    const int b = idx / p.table_chunks;
    const int i = (idx % p.table_chunks) * 256 + threadIdx.x;
    if (i >= p.tiles_per_seq) return;
    const int pi = (16 * i) / p.P, off = (16 * i) % p.P;
    int64_t pg = (p.page_table && pi < p.max_pages)
                     ? static_cast<int64_t>(p.page_table[static_cast<size_t>(b) * p.max_pages + pi])
                     : static_cast<int64_t>(b) * p.max_pages + pi;
    uint64_t flag = 0;
    if (pi >= p.max_pages || pg < 0 || pg >= p.num_pages) {
      pg = 0;
      flag = 1;
    }
    const uint64_t blk = reinterpret_cast<uint64_t>(p.pages) + static_cast<uint64_t>(pg) * p.H * 72 * p.P;
    uint64_t *e = p.tiles + (static_cast<size_t>(b) * p.tiles_per_seq + i) * 2;
    e[0] = blk + 32 * off;
    e[1] = (blk + 64 * static_cast<uint64_t>(p.P) + 4 * off) | flag;
    return;
  }
  __shared__ float qs[4][D];
  const int b = blockIdx.x / (p.H * p.n_rg), h = (blockIdx.x / p.n_rg) % p.H, rg = blockIdx.x % p.n_rg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  {
    float y0 = 0.0f, y1 = 0.0f;
    const int r = 4 * rg + wave;  // query row of this wave within the head's R rows
    if (r < p.R) {
      const size_t rj = (static_cast<size_t>(b) * p.Nq + r / p.G) * p.Hq + h * p.G + r % p.G;
      y0 = load_elem<DT>(p.q, rj * D + lane);
      y1 = load_elem<DT>(p.q, rj * D + lane + 64);
      rotate_query_wave(y0, y1, p.rk, h, lane);
      p.qrot[rj * D + lane] = y0;
      p.qrot[rj * D + lane + 64] = y1;
      float sum = y0 + y1;
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) p.qsum[rj] = sum;
    }
    qs[wave][lane] = y0;
    qs[wave][lane + 64] = y1;
  }
  __syncthreads();
  if (wave != 0) return;
  const int col = lane & 15, grp = lane >> 4, hr = col >> 2, dg = col & 3;
  float qv[2][16];
  float qabs = 0.0f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float x = qs[hr][16 * (2 * grp + m) + 4 * bb + e];
        qv[m][4 * e + bb] = x * slot_inv(e);
        qabs = fmaxf(qabs, fabsf(x));
      }
  // one shift S per query row: the row's 16 lanes x 4 lane groups hold all its dims
  qabs = fmaxf(qabs, __shfl_xor(qabs, 16));
  qabs = fmaxf(qabs, __shfl_xor(qabs, 32));
  int e2 = 0;
  (void)frexpf(qabs, &e2);  // qabs < 2^e2
  const int qshift = 26 - e2;
  int32_t *dst = p.qdig + (static_cast<size_t>(blockIdx.x) * 64 + lane) * 8;
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
  if (grp == 0 && dg == 0) p.qexp[static_cast<size_t>(blockIdx.x) * 4 + hr] = qshift;
}

constexpr int kWaves = 4;
constexpr int kBlk = 64;  // tokens per wave iteration (4 tiles of 16)

// Per-lane data of one 64-token block.
struct Blk {
  uint2 kc[4];      // K codes of token c of tile q, bytes 8g .. 8g+7
  uint2 vx[4];      // V codes of 4-token group g of tile q, dims 8c .. 8c+7
  uint32_t km[4];   // K metadata of token c of tile q
  uint32_t vm[4];   // V metadata of token c of tile q
};

struct Addr {
  uint64_t code[4], meta[4];
};

struct Ctx {
  const MfmaArgs *a;
  const uint64_t *tab;  // this sequence's tile table
  int last_tile;        // last tile index of the split (loads clamp into it)
  int t_end;
  int c, g;
  uint32_t vo_k, vo_v, vo_km, vo_vm;  // per-lane constant byte offsets
};

__device__ __forceinline__ void load_addr(const Ctx &c, int t0, Addr &ad) {
  // the table is read-only for the kernel's lifetime: constant address space, scalar loads
  const __attribute__((address_space(4))) uint64_t *tab =
      (const __attribute__((address_space(4))) uint64_t *)(reinterpret_cast<uintptr_t>(c.tab));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = min(t0 / 16 + q, c.last_tile);
    ad.code[q] = tab[2 * idx];
    ad.meta[q] = tab[2 * idx + 1];
  }
}

// global-memory pointers (address space 1): scalar base + 32-bit lane offset
typedef const __attribute__((address_space(1))) uint8_t *gbyte_ptr;
__device__ __forceinline__ uint2 gload_u64(gbyte_ptr base, uint32_t off) {
  const uint64_t v = *reinterpret_cast<const __attribute__((address_space(1))) uint64_t *>(base + off);
  return uint2{static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32)};
}
__device__ __forceinline__ uint32_t gload_u32(gbyte_ptr base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(1))) uint32_t *>(base + off);
}

__device__ __forceinline__ void load_block(const Ctx &c, const Addr &ad, Blk &o, bool &bad) {
  // (the empty asm keeps the 32-bit offsets in this block, so that the
  // loads are selected as scalar base + 32-bit VGPR offset)
  uint32_t vo_k = c.vo_k, vo_v = c.vo_v, vo_km = c.vo_km, vo_vm = c.vo_vm;
  asm volatile("" : "+v"(vo_k), "+v"(vo_v), "+v"(vo_km), "+v"(vo_vm));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const gbyte_ptr cb = reinterpret_cast<gbyte_ptr>(ad.code[q]);
    const gbyte_ptr mb = reinterpret_cast<gbyte_ptr>(ad.meta[q] & ~static_cast<uint64_t>(1));
    bad = bad || (ad.meta[q] & 1) != 0;
    o.kc[q] = gload_u64(cb, vo_k);
    o.vx[q] = gload_u64(cb, vo_v);
    o.km[q] = gload_u32(mb, vo_km);
    o.vm[q] = gload_u32(mb, vo_vm);
  }
}

struct State {
  v4i bk[2];        // key-side A operand (query digits), dims half m
  float qsum;       // sum of q' of this lane's query row (zero-point term)
  float unscale;    // 2^-S of this lane's query row
  bool row_ok;
  uint32_t sel1, sel2;  // byte-transpose selectors
  int src_lane4;        // 4 * lane whose bytes this lane takes for the value operand
  int krow_lane4;       // 4 * a lane of the query row of this lane's value accumulators
  int vx_lane;          // this lane's column within its quad (byte index, 3 = ones)
  v4i accv[8];      // value accumulators (int32, MFMA), 16 dims each
  float lsum, zsum;
  int kappa;
  bool have_ref;
};

__device__ __forceinline__ void compute_block(const Ctx &c, int t0, const Blk &blk, State &st, float *facc) {
  // ---- keys: lane (c, g) gets the 4 digit sums of query row g and token (q, c)
  float logit[4], sv[4], zv[4];
  float umax = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v4i dk = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.bk[0], slots(blk.kc[q].x), v4i{0, 0, 0, 0}, 0, 0, 0);
    dk = __builtin_amdgcn_mfma_i32_16x16x64_i8(st.bk[1], slots(blk.kc[q].y), dk, 0, 0, 0);
    const int low = (dk[2] << 7) + dk[3];  // |.| < 2^26: no int32 overflow
    const float dot = fmaf(static_cast<float>(dk[0]), 2097152.0f,
                           fmaf(static_cast<float>(dk[1]), 16384.0f, static_cast<float>(low)));
    const float ks = half_bits_to_float(blk.km[q] & 0xffffu), kz = half_bits_to_float(blk.km[q] >> 16);
    sv[q] = half_bits_to_float(blk.vm[q] & 0xffffu);
    zv[q] = half_bits_to_float(blk.vm[q] >> 16);
    const bool valid = st.row_ok && (t0 + 16 * q + c.c < c.t_end);
    logit[q] = valid ? dot * (ks * st.unscale) + kz * st.qsum : -INFINITY;
    int es;
    (void)frexpf(sv[q], &es);  // s_v < 2^es
    umax = fmaxf(umax, logit[q] + static_cast<float>(es));
  }
  umax = row16_max(umax);
  int need = st.kappa;
  if (umax != -INFINITY) {
    need = (kWeightBits - 1) - static_cast<int>(ceilf(umax));
    if (!st.have_ref) {
      st.kappa = need - kHeadroom;
      st.have_ref = true;
    }
  }
  // wave-uniform decision: flush when any row outgrew its headroom
  if (__any(st.have_ref && need < st.kappa)) {
    const int newk = (st.have_ref && need < st.kappa) ? need - kHeadroom : st.kappa;
    const float f2 = ldexpf(1.0f, newk - st.kappa);  // factor of query row g
    // the value accumulators of this lane belong to query row (c >> 2)
    const float f2v = __int_as_float(__builtin_amdgcn_ds_bpermute(st.krow_lane4, __float_as_int(f2)));
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *p = facc + (4 * i + r) * 64;
        *p = (*p + static_cast<float>(byte_sum(st.accv[i][r], st.vx_lane))) * f2v;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) st.accv[i] = v4i{0, 0, 0, 0};
    st.lsum *= f2;
    st.zsum *= f2;
    st.kappa = newk;
  }
  // ---- weights W = round(2^(logit + kappa) s_v) < 2^24, bytes offset to int8
  const float kf = static_cast<float>(st.kappa);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float p = exp2f(logit[q] + kf);
    st.lsum += p;
    st.zsum += p * zv[q];
    const uint32_t W = static_cast<uint32_t>(fmaf(p, sv[q], 0.5f));
    w[q] = W ^ kByteOffset;
  }
  // quad lane x takes byte x (digit x, or the ones for x = 3) of its quad's 4 tokens;
  // then the lanes move to the B layout: column 4 r + x, k-slice = token group
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = quad_byte_transpose(w[q], st.sel1, st.sel2);
    w[q] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(st.src_lane4, static_cast<int>(w[q])));
  }
  const v4i bv{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]), static_cast<int>(w[3])};

  // ---- values: 8 MFMAs (16 dims each), k = the 64 tokens of the block
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x0 = hf ? blk.vx[0].y : blk.vx[0].x, x1 = hf ? blk.vx[1].y : blk.vx[1].x;
      const uint32_t x2 = hf ? blk.vx[2].y : blk.vx[2].x, x3 = hf ? blk.vx[3].y : blk.vx[3].x;
      const v4i av{slot(x0, e), slot(x1, e), slot(x2, e), slot(x3, e)};
      st.accv[4 * hf + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, st.accv[4 * hf + e], 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void decode_mfma_kernel(MfmaArgs a) {
  __shared__ float red[kWaves][4][4 + D];  // per wave, per row: m, l, z, flag, acc[128]
  __shared__ float facc_all[kWaves][32 * 64];  // flushed value accumulators, [slot][lane]
  const int s = blockIdx.x, b = blockIdx.z;
  const int h = blockIdx.y / a.n_rg, rg = blockIdx.y % a.n_rg;  // KV head, group of 4 query rows
  const int row0 = 4 * rg, nrows = min(4, a.R - row0);
  const size_t unit = (static_cast<size_t>(b) * a.H + h) * a.n_rg + rg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  Ctx c;
  c.a = &a;
  c.c = lane & 15;
  c.g = lane >> 4;
  float *facc = &facc_all[wave][lane];

  int L = a.seq_lens[b];
  bool bad = L < 0 || L > a.max_seq_len;
  if (bad) L = 0;
  const int t_begin = s * a.split_tokens;
  c.t_end = min(t_begin + a.split_tokens, L);
  c.last_tile = c.t_end > t_begin ? (c.t_end - 1) / 16 : t_begin / 16;
  c.tab = a.tiles + static_cast<size_t>(b) * a.tiles_per_seq * 2;
  const uint32_t hoff = static_cast<uint32_t>(h) * 72u * static_cast<uint32_t>(a.P);
  c.vo_k = hoff + 32u * c.c + 8u * c.g;
  c.vo_v = hoff + 32u * a.P + 128u * c.g + 8u * c.c;
  c.vo_km = hoff + 4u * c.c;
  c.vo_vm = hoff + 4u * a.P + 4u * c.c;

  // ---- query digits (key-side A operand: row c = 4 r + d, k-slice g) and this lane's query row g
  State st;
  {
    const int4 *dsrc = reinterpret_cast<const int4 *>(a.qdig + (unit * 64 + lane) * 8);
    const int4 d0 = dsrc[0], d1 = dsrc[1];
    st.bk[0] = v4i{d0.x, d0.y, d0.z, d0.w};
    st.bk[1] = v4i{d1.x, d1.y, d1.z, d1.w};
  }
  const int hr = c.g;  // query row (within the group) of the key-side lanes
  st.row_ok = hr < nrows;
  {
    const int r = row0 + hr, qi = r / a.G, gh = r % a.G;
    const size_t rj = (static_cast<size_t>(b) * a.Nq + qi) * a.Hq + h * a.G + gh;
    st.qsum = st.row_ok ? a.qsum[rj] : 0.0f;
    st.unscale = ldexpf(1.0f, -a.qexp[unit * 4 + hr]);
  }
  const int x = lane & 3;
  st.sel1 = (x & 1) ? 0x03070105u : 0x06020400u;
  st.sel2 = (x & 2) ? 0x03020706u : 0x05040100u;
  // value operand lane 16 g' + 4 r + x takes from lane 16 r + 4 g' + x
  st.src_lane4 = 4 * (16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + x);
  st.krow_lane4 = 4 * (16 * ((lane >> 2) & 3));
  st.vx_lane = x;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.accv[i] = v4i{0, 0, 0, 0};
  st.lsum = st.zsum = 0.0f;
  st.kappa = 0;
  st.have_ref = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) facc[i * 64] = 0.0f;

  // ---- main loop: wave w takes blocks w, w+4, ...; block i+1 is in flight
  // while block i is computed and the addresses of block i+2 are fetched
  constexpr int kStride = kWaves * kBlk;
  int t0 = t_begin + wave * kBlk;
  const int n_blk = t0 < c.t_end ? (c.t_end - t0 + kStride - 1) / kStride : 0;
  if (n_blk > 0) {
    Blk b0, b1;
    Addr a0, a1;
    load_addr(c, t0, a0);
    load_block(c, a0, b0, bad);
    load_addr(c, t0 + kStride, a1);
    for (int i = 0; i < n_blk / 2; ++i) {
      load_block(c, a1, b1, bad);
      load_addr(c, t0 + 2 * kStride, a0);
      compute_block(c, t0, b0, st, facc);
      load_block(c, a0, b0, bad);
      load_addr(c, t0 + 3 * kStride, a1);
      compute_block(c, t0 + kStride, b1, st, facc);
      t0 += 2 * kStride;
    }
    if (n_blk & 1) compute_block(c, t0, b0, st, facc);
  }

  // ---- per-wave result for each row
  const float lrow = row16_sum(st.lsum);
  const float zrow = row16_sum(st.zsum);
  const bool any_bad = __any(bad);
  // value accumulators: lane (4 r + x, g') holds column x (byte x, or the
  // ones for x = 3) of query row r for dims 8 (4 g' + i) + 4 hf + e
  const int vr = (lane >> 2) & 3;
  const float wbyte = x == 0 ? 1.0f : x == 1 ? 256.0f : x == 2 ? 65536.0f : 0.0f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = 4 * hf + e;
        float v = (facc[(4 * k + i) * 64] + static_cast<float>(byte_sum(st.accv[k][i], x))) * (wbyte * slot_inv(e));
        v += fdpp_xor1(v);
        v += fdpp_xor2(v);
        if (x == 0 && vr < nrows) red[wave][vr][4 + 8 * (4 * c.g + i) + 4 * hf + e] = v;
      }
  if (c.c == 0 && st.row_ok) {
    red[wave][hr][0] = st.have_ref ? -static_cast<float>(st.kappa) : -INFINITY;
    red[wave][hr][1] = lrow;
    red[wave][hr][2] = zrow;
    red[wave][hr][3] = any_bad ? 1.0f : 0.0f;
  }
  __syncthreads();

  // ---- merge the 4 waves (base-2 log-sum-exp) and write this split's partial
  for (int idx = threadIdx.x; idx < nrows * D; idx += 256) {
    const int r = idx / D, i = idx % D;
    float mstar = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      mstar = fmaxf(mstar, red[w2][r][0]);
      nan = nan || red[w2][r][3] != 0.0f;
    }
    float l = 0.0f, z = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      if (red[w2][r][0] == -INFINITY) continue;
      const float sc = exp2f(red[w2][r][0] - mstar);
      l += sc * red[w2][r][1];
      z += sc * red[w2][r][2];
      acc += sc * red[w2][r][4 + i];
    }
    const int qq = (row0 + r) / a.G, g2 = (row0 + r) % a.G;
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
  return pl.rows_per_head <= kMaxRows && page_size % 16 == 0 &&
         static_cast<int64_t>(pl.H) * 72 * page_size < (static_cast<int64_t>(1) << 31);
}

hipError_t launch_decode_prologue(const DecodePlan &pl, const void *q, int dtype, RotDev rk, const uint8_t *pages,
                                  int64_t num_pages, int page_size, const int32_t *page_table, int max_pages,
                                  float *qrot, float *qsum, int32_t *qdig, int32_t *qexp, uint64_t *tiles,
                                  hipStream_t stream) {
  if (pl.num_seqs == 0) return hipSuccess;
  PrologueArgs p{};
  p.q = q;
  p.rk = rk;
  p.R = pl.rows_per_head;
  p.G = pl.G;
  p.Hq = pl.Hq;
  p.H = pl.H;
  p.Nq = pl.queries_per_seq;
  p.num_seqs = pl.num_seqs;
  p.n_rg = (pl.rows_per_head + 3) / 4;
  p.qrot = qrot;
  p.qsum = qsum;
  p.qdig = qdig;
  p.qexp = qexp;
  p.pages = pages;
  p.num_pages = num_pages;
  p.P = page_size;
  p.page_table = page_table;
  p.max_pages = max_pages;
  p.tiles_per_seq = pl.tiles_per_seq;
  p.table_chunks = (pl.tiles_per_seq + 255) / 256;
  p.tiles = tiles;
  const dim3 grid(pl.num_seqs * pl.H * p.n_rg + pl.num_seqs * p.table_chunks);
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(decode_prologue_kernel<KVQ_F32>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_prologue_kernel<KVQ_BF16>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_split_mfma(const DecodePlan &pl, int page_size, const int32_t *seq_lens,
                                    const int32_t *qdig, const int32_t *qexp, const float *qsum,
                                    const uint64_t *tiles, float *part, hipStream_t stream) {
  if (pl.num_seqs == 0) return hipSuccess;
  const int tps = pl.tiles_per_seq;
  MfmaArgs a{};
  a.R = pl.rows_per_head;
  a.G = pl.G;
  a.Hq = pl.Hq;
  a.H = pl.H;
  a.Nq = pl.queries_per_seq;
  a.n_rg = (pl.rows_per_head + 3) / 4;
  a.split_tokens = pl.split_tokens;
  a.splits = pl.splits;
  a.max_seq_len = pl.max_seq_len;
  a.P = page_size;
  a.tiles_per_seq = tps;
  a.seq_lens = seq_lens;
  a.qdig = qdig;
  a.qexp = qexp;
  a.qsum = qsum;
  a.tiles = tiles;
  a.part = part;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(pl.splits, pl.H * a.n_rg, pl.num_seqs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
