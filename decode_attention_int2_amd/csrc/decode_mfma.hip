// decode_mfma.hip -- decode attention over the packed INT2 cache on the
// gfx950 matrix cores (v_mfma_i32_16x16x64_i8) in one launch: query
// rotation, split-K attention, split merge and inverse value rotation.  A
// workgroup takes one or two groups of 4 query rows of one (sequence, KV
// head) -- up to 64 rows per KV head: GQA group x queries per sequence --
// and one split of the sequence's tokens; with two groups each block's codes
// are unpacked once and serve both.
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
//   w_t = 2^(logit_t + kappa) s_t rounded to an integer < 2^27 is split into
//   four balanced base-256 digits in [-128, 127] (int8 lanes; two integer
//   operations per weight); column x of a row accumulates
//   sum_t digit_x(w_t) c_t exactly in int32 and the row's value sum is
//   sum_x 256^x column_x.  kappa is a per-row power-of-two
//   scale chosen from a running bound of logit + log2(s) with 2^2 of
//   headroom, so the split's largest weight carries at least 2^23 units; if
//   the bound outgrows it the int32 accumulators are flushed to fp32 in LDS
//   (rare) and the scale moves.  l = sum 2^(logit + kappa) and z = sum
//   2^(logit + kappa) z_t stay in fp32 per lane.  The digits reach the
//   MFMA's B layout (column 4 r + digit, k = 16 tokens per lane group) by a
//   byte transpose inside each lane quad and one lane permutation.
// Query: each workgroup rotates its own query rows (signed Hadamard by the
//   fast transform, a dense R_K as a product with the matrix in registers)
//   and forms their digits while its first key / value loads are in flight.
// Addresses: the page of every 16-token tile is read from the page table with
//   scalar loads one block ahead and turned into the (page, head) block base
//   on the scalar unit (32-bit bounds check, one 32 x 32 -> 64-bit product);
//   every vector load is scalar base + per-lane constant offset.  The next
//   two 64-token blocks are in flight while the current one is computed;
//   tiles past the split end are clamped into its last tile and masked.
// Merge: each split writes an (m, l, z, acc[128]) partial with m = -kappa;
//   the last split of a (sequence, KV head, row group) to arrive (a tagged
//   arrival counter) merges the partials, applies R_V^T and writes the output.
// BF16 windows (kWin): after its main loop each split attends its slice of
//   the sink and recent window tokens on the bf16 matrix cores and stores a
//   window partial of its own, merged beside the INT2 partials.
#include <type_traits>

#include "kvq_internal.h"

#ifdef KVQ_PHASE_TIMESTAMPS
// Diagnostic build (libkvq_phases.so) only: every wave of a launch records
// the wall clock at its phase boundaries -- entry, main loop start, main loop
// end, arrival counted, and in the merging workgroup: partials merged, value
// rotation applied, outputs stored -- with the hardware ids of its compute
// unit.  Waves past kPhaseWaves record nothing.
constexpr int kPhaseWaves = 8192;
constexpr int kPhaseFields = 14;  // hw id, xcc id, blocks, t entry, t loop, t loop end, t arrived, t merged,
                                  // t rotated, t stored, t query digits ready, t first block's data,
                                  // t first blocks' loads issued, t query row loaded
__device__ unsigned long long kvq_phase_ts[kPhaseWaves * kPhaseFields];
#define KVQ_PHASE(i) (phase_t[i] = wall_clock64())
#else
#define KVQ_PHASE(i) ((void)0)
#endif

namespace kvq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf_w __attribute__((ext_vector_type(8)));
typedef float v4bf_f __attribute__((ext_vector_type(4)));

constexpr uint32_t kM0 = 0x03030303u, kM1 = 0x0C0C0C0Cu, kM2 = 0x30303030u;
constexpr int kHeadroom = 2;       // log2 headroom of the value scale
constexpr int kWeightBits = 28;    // value weights are integers < 2^27: four base-256 digits

// The balanced base-256 digits of w < 2^31 - 2^24 as int8 lanes, digit x in
// byte x: with b_x the bytes of w + 0x80808080 (no carry out of the word),
// w = sum_x (b_x - 128) 256^x, and b_x - 128 as an int8 is b_x with its top
// bit flipped.
__device__ __forceinline__ uint32_t weight_digits(uint32_t w) { return (w + 0x80808080u) ^ 0x80808080u; }

// The 4 code slots of every byte of x as int8 lanes; slot 1 and 2 are scaled by 4 and 16.
__device__ __forceinline__ v4i slots(uint32_t x) {
  return v4i{static_cast<int>(x & kM0), static_cast<int>(x & kM1), static_cast<int>(x & kM2),
             static_cast<int>((x >> 6) & kM0)};
}
__device__ __forceinline__ int slot(uint32_t x, int e) {
  return static_cast<int>(e == 0 ? (x & kM0) : e == 1 ? (x & kM1) : e == 2 ? (x & kM2) : ((x >> 6) & kM0));
}
__device__ __forceinline__ float slot_inv(int e) { return e == 1 ? 0.25f : e == 2 ? 0.0625f : 1.0f; }

// (every source lane of these patterns exists, so bound_ctrl changes nothing;
// it lets the compiler fold the move into the instruction that uses it)
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_xor2(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_ror4(int v) { return __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_ror8(int v) { return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true); }
__device__ __forceinline__ float fdpp_xor1(float v) { return __int_as_float(dpp_xor1(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_xor2(float v) { return __int_as_float(dpp_xor2(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_ror4(float v) { return __int_as_float(dpp_ror4(__float_as_int(v))); }
__device__ __forceinline__ float fdpp_ror8(float v) { return __int_as_float(dpp_ror8(__float_as_int(v))); }

// max / sum over the 16 lanes of a DPP row (rotations reach every lane of the row)
// (integer maximum: the moves fold into v_max_i32's DPP form; a float
// maximum would canonicalize each moved value first)
__device__ __forceinline__ int row16_max(int x) {
  x = max(x, dpp_xor1(x));
  x = max(x, dpp_xor2(x));
  x = max(x, dpp_ror4(x));
  x = max(x, dpp_ror8(x));
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

struct MfmaArgs {
  int R, G, Hq, H, Nq, n_rg;  // n_rg: groups of 4 query rows per KV head
  int n_wy;                   // workgroups per KV head along grid y: n_rg / RG rounded up
  int split_tokens, splits, max_seq_len;
  int P, p_shift;             // page size in tokens (a power of two) and its log2
  int max_pages;
  uint32_t np32;              // number of pages, at most 2^31 - 1 (page-table entries are int32)
  uint32_t page_bytes;        // H * 72 * P (< 2^31)
  const uint8_t *pages;
  // page of entry i of sequence b: (ptab[b * tab_stride + (i & tab_mask)] & val_mask) + (i & id_mask) + b * base_mul;
  // with a page table: stride max_pages, masks ~0, ~0, 0, base_mul 0;
  // without (pages b * max_pages + i): ptab = any readable int32, stride 0, masks 0, 0, ~0, base_mul max_pages
  const int32_t *ptab;
  int tab_stride, tab_mask, val_mask, id_mask, base_mul;
  const int32_t *seq_lens;
  const void *q;              // query rows (dtype of the launch), or rotated fp32 rows
  RotDev rk, rv;
  float *part;                // [rows][Hq][parts][132] partials, one per (split, wave) or per split
  int parts;                  // splits * 8, or splits when the waves' partials are merged first (premerge)
  int pstride;                // partial slots per (row, head): parts, plus one window slot per split
  int causal;                 // row qi of a sequence attends its first L - (Nq - 1 - qi) tokens
  int premerge;
  // BF16 windows (decode with windows): sink [num_seqs][win_S][H][128] and
  // recent [num_seqs][win_W][H][128] (position p in slot p % win_W), bf16;
  // the window keys' centering win_mu [H][128] or null
  const uint16_t *win_sk, *win_sv, *win_rk, *win_rv;
  int win_S, win_W;
  const float *win_mu;
  unsigned long long *counters;  // [num_seqs][H][n_rg][kArrivalWords] arrival counters
  uint32_t epoch;
  float *out_o, *ot;
  float *y_zero;              // [num_seqs * Nq][d_model] to clear (the W_O launch adds into it), or null
  int d_model;
};

// Fixed-point int8 digits of the 4 query rows of a row group (qs: their q',
// zero rows past the head's last row) in the key-side A-operand layout of
// lane (col, grp): query row col/4, digit col%4; dim 16 (2 grp + m) + 4 bb + e
// goes to dword [m][e], byte bb.  Slot e of the unpacked codes carries a
// factor 1/slot_inv(e), divided out here.  Q = round(q' 2^S) with
// |Q| < 2^26, S = qshift[r] per query row from its largest |q'|.  Returns
// dword (m, e) of the lane's operand.
__device__ __forceinline__ uint32_t query_digit_word(const float (*qs)[D], const int *qshift, int lane, int m,
                                                    int e) {
  const int col = lane & 15, grp = lane >> 4, hr = col >> 2, dg = col & 3;
  const int sh = qshift[hr];
  uint32_t word = 0;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const float x = qs[hr][16 * (2 * grp + m) + 4 * bb + e] * slot_inv(e);
    const int Q = static_cast<int>(__builtin_rintf(ldexpf(x, sh)));
    const int dig = (dg == 0) ? (Q >> 21) : ((Q >> (21 - 7 * dg)) & 127);
    word |= (static_cast<uint32_t>(dig) & 0xffu) << (8 * bb);
  }
  return word;
}

// Device-scope store of a split partial (read by the merging workgroup).
__device__ __forceinline__ void store_partial(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kWaves = kMfmaWaves;  // waves per workgroup (one workgroup per CU)
constexpr int kBlk = 64;  // tokens per wave iteration (4 tiles of 16)

// Per-lane data of one 64-token block.
struct Blk {
  uint2 kc[4];      // K codes of token c of tile q, bytes 8g .. 8g+7
  uint2 vx[4];      // V codes of 4-token group g of tile q, dims 8c .. 8c+7
  uint32_t km[4];   // K metadata of token c of tile q
  uint32_t vm[4];   // V metadata of token c of tile q
};

// Page of each tile of a block as read from the page table (wave-uniform)
// and, for pages longer than one tile, the tile's first token in its page.
struct Addr {
  int32_t pg[4], off[4];
};

struct Ctx {
  const MfmaArgs *a;
  const int32_t *ptab;  // this sequence's page-table row
  int32_t pg_base;
  int last_tile;        // last tile index of the split (loads clamp into it)
  int t_end;
  int c, g;
  uint32_t vo_k, vo_v, vo_km, vo_vm;  // per-lane constant byte offsets from the (page, head) block
};

// Page-table entries of the 4 tiles of the block at t0 (scalar loads; they
// are used one block later).  Every token read lies below the sequence
// length, which is at most max_pages * P, so the index stays inside the row.
template <bool P16>
__device__ __forceinline__ void load_addr(const Ctx &c, int t0, Addr &ad) {
  // the page table is read-only for the kernel's lifetime: constant address space, scalar loads
  const __attribute__((address_space(4))) int32_t *pt =
      (const __attribute__((address_space(4))) int32_t *)(reinterpret_cast<uintptr_t>(c.ptab));
  const MfmaArgs &a = *c.a;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tile = min((t0 >> 4) + q, c.last_tile);
    const int pi = P16 ? tile : tile >> (a.p_shift - 4);
    ad.off[q] = P16 ? 0 : (tile << 4) & (a.P - 1);
    ad.pg[q] = (pt[pi & a.tab_mask] & a.val_mask) + (pi & a.id_mask) + c.pg_base;
  }
}

__device__ __forceinline__ void repoint_all(Addr &ad) {
#pragma unroll
  for (int q = 0; q < 4; ++q) ad.pg[q] = 0;
}

// global-memory pointers (address space 1): scalar base + 32-bit lane offset.
// NT: the cache is read once per launch (one group of query rows per KV
// head): non-temporal loads (streaming hint), so that its bytes do not
// displace the page table, the partials and the queries from the caches
// (16 x 32K tokens: 61.9 -> 58-59 us per launch).  With several row groups
// per KV head every group reads the same bytes: ordinary loads, which leave
// them in the caches for the other groups.
typedef const __attribute__((address_space(1))) uint8_t *gbyte_ptr;
template <bool NT>
__device__ __forceinline__ uint2 gload_u64(gbyte_ptr base, uint32_t off) {
  const auto *p = reinterpret_cast<const __attribute__((address_space(1))) uint64_t *>(base + off);
  const uint64_t v = NT ? __builtin_nontemporal_load(p) : *p;
  return uint2{static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32)};
}
template <bool NT>
__device__ __forceinline__ uint32_t gload_u32(gbyte_ptr base, uint32_t off) {
  const auto *p = reinterpret_cast<const __attribute__((address_space(1))) uint32_t *>(base + off);
  return NT ? __builtin_nontemporal_load(p) : *p;
}

// Issues the block's loads.  A page index outside the cache (compared as
// unsigned 32-bit, so negative entries fail too) reads page 0 instead and
// sets `bad` (the rows' outputs become NaN).  The (page, head) block base is
// pages + page * page_bytes (a 32 x 32 -> 64-bit product on the scalar
// unit); the per-lane offsets carry the head and the section offsets.
template <bool P16, bool NT>
__device__ __forceinline__ void load_block(const Ctx &c, const Addr &ad, Blk &o, bool &bad) {
  // (the empty asm keeps the 32-bit offsets in this block, so that the
  // loads are selected as scalar base + 32-bit VGPR offset)
  uint32_t vo_k = c.vo_k, vo_v = c.vo_v, vo_km = c.vo_km, vo_vm = c.vo_vm;
  asm volatile("" : "+v"(vo_k), "+v"(vo_v), "+v"(vo_km), "+v"(vo_vm));
  const MfmaArgs &a = *c.a;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t pg = static_cast<uint32_t>(ad.pg[q]);
    const bool ok = pg < a.np32;
    bad = bad || !ok;
    const uint64_t blk = reinterpret_cast<uint64_t>(a.pages) +
                         static_cast<uint64_t>(ok ? pg : 0u) * static_cast<uint64_t>(a.page_bytes);
    const uint64_t cb = P16 ? blk : blk + 32u * static_cast<uint32_t>(ad.off[q]);
    const uint64_t mb = P16 ? blk : blk + 4u * static_cast<uint32_t>(ad.off[q]);
    o.kc[q] = gload_u64<NT>(reinterpret_cast<gbyte_ptr>(cb), vo_k);
    o.vx[q] = gload_u64<NT>(reinterpret_cast<gbyte_ptr>(cb), vo_v);
    o.km[q] = gload_u32<NT>(reinterpret_cast<gbyte_ptr>(mb), vo_km);
    o.vm[q] = gload_u32<NT>(reinterpret_cast<gbyte_ptr>(mb), vo_vm);
  }
}

// The split's last block may hold slots at or past the sequence's end, whose
// bytes may be anything: their tokens are masked, and the value metadata is
// zeroed so that no inf or NaN scale or zero-point reaches the sums (0 * inf).
__device__ __forceinline__ void mask_tail_meta(const Ctx &c, int t0, Blk &blk) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (t0 + 16 * q + c.c >= c.t_end) blk.vm[q] = 0u;
}

// Per-lane state of one group of 4 query rows.
struct State {
  v4i bk[2];        // key-side A operand (query digits), dims half m
  float qsum;       // sum of q' of this lane's query row (zero-point term)
  float unscale;    // 2^-S of this lane's query row
  uint32_t sel1, sel2;  // byte-transpose selectors
  int src_lane4;        // 4 * lane whose bytes this lane takes for the value operand
  int krow_lane4;       // 4 * a lane of the query row of this lane's value accumulators
  v4i accv[8];      // value accumulators (int32, MFMA), 16 dims each
  float lsum, zsum;
  int kappa;
  bool have_ref;
  bool flushed;         // (wave-uniform) the LDS accumulators hold flushed values
  int tlim;             // tokens below tlim count for this lane's query row (split end, or the row's causal length)
};

constexpr int kFaccFloats = 32 * 64;  // flushed value accumulators of one row group per wave: [slot][lane]

// One 64-token block for RG groups of 4 query rows.  What depends on the
// block alone -- the key and value code slots, the metadata, the bound of
// log2 s_v -- is formed once and serves every row group (each extra row
// group costs its MFMAs and its per-row work only).  facc: this lane's word
// of the wave's flushed accumulators, row group r at facc + r kFaccFloats.
template <int RG>
__device__ __forceinline__ void compute_block(const Ctx &c, int t0, const Blk &blk, State (&st)[RG], float *facc) {
  // ---- keys: lane (c, g) gets the 4 digit sums of query row g and token (q, c)
  float logit[RG][4], sv[4], zv[4];
  float umax[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) umax[r] = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4i kx = slots(blk.kc[q].x), ky = slots(blk.kc[q].y);
    const float ks = half_bits_to_float(blk.km[q] & 0xffffu), kz = half_bits_to_float(blk.km[q] >> 16);
    sv[q] = half_bits_to_float(blk.vm[q] & 0xffffu);
    zv[q] = half_bits_to_float(blk.vm[q] >> 16);
    int es;
    (void)frexpf(sv[q], &es);  // s_v < 2^es
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      v4i dk = __builtin_amdgcn_mfma_i32_16x16x64_i8(st[r].bk[0], kx, v4i{0, 0, 0, 0}, 0, 0, 0);
      dk = __builtin_amdgcn_mfma_i32_16x16x64_i8(st[r].bk[1], ky, dk, 0, 0, 0);
      // digit sums over 128 dims (32 per slot, digits below 2^7, the top one
      // below 2^5 in magnitude, against codes of at most 3, 12, 48, 3 per
      // slot): |dk0| < 2^17 and 0 <= dk1..3 < 2^19, so dk0 128 + dk1 is exact
      // in fp32 (< 2^24) and dk2 128 + dk3 (< 2^26) is rounded once
      const int high = dk[0] * 128 + dk[1];
      const int low = dk[2] * 128 + dk[3];
      const float dot = fmaf(static_cast<float>(high), 16384.0f, static_cast<float>(low));
      // (rows past the group's last hold q' = 0: finite logits, never stored;
      // the value is formed first, so that the mask is a select, not a branch)
      const bool valid = 16 * q + c.c < st[r].tlim - t0;
      const float lv = dot * (ks * st[r].unscale) + kz * st[r].qsum;
      logit[r][q] = valid ? lv : -INFINITY;
      umax[r] = fmaxf(umax[r], logit[r][q] + static_cast<float>(es));
    }
  }
  v4i bv[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    State &sr = st[r];
    // the row's largest ceil(logit + es) (ceil is monotonic, so this is the
    // ceiling of the row's largest bound); a lane with every token masked
    // contributes kNoBound
    constexpr int kNoBound = -(1 << 30);
    const int ubound = row16_max(umax[r] == -INFINITY ? kNoBound : static_cast<int>(ceilf(umax[r])));
    // (selects, no branch; a row whose tokens are all masked keeps its scale)
    const bool fin = ubound != kNoBound;
    const int need = fin ? (kWeightBits - 1) - ubound : sr.kappa;
    sr.kappa = fin && !sr.have_ref ? need - kHeadroom : sr.kappa;
    sr.have_ref = sr.have_ref || fin;
    // wave-uniform decision: flush when any row outgrew its headroom
    if (__any(sr.have_ref && need < sr.kappa)) {
      const int newk = (sr.have_ref && need < sr.kappa) ? need - kHeadroom : sr.kappa;
      const float f2 = ldexpf(1.0f, newk - sr.kappa);  // factor of query row g
      // the value accumulators of this lane belong to query row (c >> 2)
      const float f2v = __int_as_float(__builtin_amdgcn_ds_bpermute(sr.krow_lane4, __float_as_int(f2)));
      float *fr = facc + r * kFaccFloats;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float *pk = fr + (4 * i + k) * 64;
          *pk = ((sr.flushed ? *pk : 0.0f) + static_cast<float>(sr.accv[i][k])) * f2v;
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) sr.accv[i] = v4i{0, 0, 0, 0};
      sr.lsum *= f2;
      sr.zsum *= f2;
      sr.kappa = newk;
      sr.flushed = true;
    }
    // ---- weights W = round(2^(logit + kappa) s_v) < 2^27 as four base-256 digits
    const float kf = static_cast<float>(sr.kappa);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // (hardware exp2: results below 2^-126 weigh nothing against the
      // split's largest weight, >= 2^23, and masked tokens give exp2(-inf) = 0)
      const float pq = __builtin_amdgcn_exp2f(logit[r][q] + kf);
      sr.lsum += pq;
      sr.zsum += pq * zv[q];
      const uint32_t W = static_cast<uint32_t>(fmaf(pq, sv[q], 0.5f));
      w[q] = weight_digits(W);
    }
    // quad lane x takes digit x (byte x) of its quad's 4 tokens;
    // then the lanes move to the B layout: column 4 r + x, k-slice = token group
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q] = quad_byte_transpose(w[q], sr.sel1, sr.sel2);
      w[q] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(sr.src_lane4, static_cast<int>(w[q])));
    }
    bv[r] = v4i{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]), static_cast<int>(w[3])};
  }

  // ---- values: 8 MFMAs (16 dims each) per row group, k = the 64 tokens of the block
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x0 = hf ? blk.vx[0].y : blk.vx[0].x, x1 = hf ? blk.vx[1].y : blk.vx[1].x;
      const uint32_t x2 = hf ? blk.vx[2].y : blk.vx[2].x, x3 = hf ? blk.vx[3].y : blk.vx[3].x;
      const v4i av{slot(x0, e), slot(x1, e), slot(x2, e), slot(x3, e)};
#pragma unroll
      for (int r = 0; r < RG; ++r)
        st[r].accv[4 * hf + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv[r], st[r].accv[4 * hf + e], 0, 0, 0);
    }
}

// RG: groups of 4 query rows per workgroup (1, or 2 without BF16 windows):
// every wave computes each of its blocks for the RG groups.
template <int DT, bool P16, bool kDense, bool kWin, bool NT, int RG>
__global__ __launch_bounds__(64 * kWaves) void decode_mfma_kernel(MfmaArgs a) {
  static_assert(RG == 1 || (RG == 2 && !kWin), "two row groups per workgroup only without windows");
  constexpr int kRows = 4 * RG;  // query rows of the workgroup
  // per wave, per row: m, l, z, flag, acc[128]; row kRows: unused stores.
  // With one row group these rows have their own array (the window code
  // uses them while facc_all holds its values); with two, each wave's rows
  // lie in its own flushed accumulators, free once the main loop is done
  // (LDS: the accumulators of two row groups are 128 KB)
  __shared__ __attribute__((aligned(16))) float red_own[RG == 1 ? kWaves : 1][RG == 1 ? 5 : 1][4 + D];
  __shared__ __attribute__((aligned(16))) float facc_all[kWaves][RG * kFaccFloats];  // flushed value accumulators, [row group][slot][lane]
  __shared__ __attribute__((aligned(16))) float qs[kRows][D];            // q' of the workgroup's rows
  __shared__ float qsum_s[kRows];
  __shared__ int qshift_s[kRows];          // fixed-point shift S of each row's digits
  __shared__ uint32_t digit_s[RG][8][64];  // key-side A operand: dword [m][e] of each lane, per row group
  auto red = [&](int w, int r) -> float * {
    if constexpr (RG == 1) return &red_own[w][r][0];
    else return &facc_all[w][r * (D + 4)];
  };
  __shared__ uint32_t s_last;
  // word 0: the next unclaimed 64-token block of the split; words 1-63: the
  // other lanes' targets of a claim (each adds 0 to a word of its own)
  __shared__ uint32_t s_claim[64];
#ifdef KVQ_PHASE_TIMESTAMPS
  unsigned long long phase_t[11] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#endif
  KVQ_PHASE(0);
  const int s = blockIdx.x, b = blockIdx.z;
  // KV head, first group of 4 query rows (of RG)
  const int h = blockIdx.y / a.n_wy, rg = (blockIdx.y % a.n_wy) * RG;
  const int row0 = 4 * rg, nrows = min(kRows, a.R - row0);
  const size_t unit = (static_cast<size_t>(b) * a.H + h) * a.n_rg + rg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  Ctx c;
  c.a = &a;
  c.c = lane & 15;
  c.g = lane >> 4;
  float *facc = &facc_all[wave][lane];

  // the arrival counter and its validation word (read by wave 0 once the
  // prologue's loads are out -- loads complete in issue order, so the
  // coherent read's round trip delays none of them -- and compared at the
  // arrival)
  unsigned long long *cnt = a.counters + unit * kArrivalWords;
  unsigned long long cnt_word = 0;
  int L = a.seq_lens[b];
  bool bad = L < 0 || L > a.max_seq_len;
  if (bad) L = 0;
  // INT2 positions [lo, hi): with windows the sink [0, lo) and the recent
  // tokens [hi, L) are read from the BF16 windows in the merge
  int lo = 0, hi = L;
  if constexpr (kWin) {
    lo = min(a.win_S, L);
    hi = max(lo, L - a.win_W);
  }
  const int t_begin = max(s * a.split_tokens, lo);
  c.t_end = min(s * a.split_tokens + a.split_tokens, hi);
  c.last_tile = c.t_end > t_begin ? (c.t_end - 1) / 16 : 0;  // (empty split: loads read tile 0, unused)
  c.ptab = a.ptab + static_cast<size_t>(b) * a.tab_stride;
  c.pg_base = b * a.base_mul;
  const uint32_t hoff = static_cast<uint32_t>(h) * 72u * static_cast<uint32_t>(a.P);
  c.vo_k = hoff + 32u * c.c + 8u * c.g;
  c.vo_v = hoff + 32u * a.P + 128u * c.g + 8u * c.c;
  c.vo_km = hoff + 64u * a.P + 4u * c.c;
  c.vo_vm = hoff + 68u * a.P + 4u * c.c;

  // ---- loads of the query row of this wave (row0 + wave), then of the
  // first block, so that the query is prepared while the block is in flight
  // (loads complete in issue order)
  // (raw bits, unconditionally from valid addresses: a use right after a
  // load would wait for it before the block's loads are issued)
  uint32_t qb0, qb1;
  int32_t sb0, sb1;
  {
    const int r = row0 + min(wave, nrows - 1);
    const size_t rj = (static_cast<size_t>(b) * a.Nq + r / a.G) * a.Hq + h * a.G + r % a.G;
    if constexpr (DT == KVQ_F32) {
      qb0 = static_cast<const uint32_t *>(a.q)[rj * D + lane];
      qb1 = static_cast<const uint32_t *>(a.q)[rj * D + lane + 64];
    } else {
      qb0 = static_cast<const uint16_t *>(a.q)[rj * D + lane];
      qb1 = static_cast<const uint16_t *>(a.q)[rj * D + lane + 64];
    }
    // signs of the head (signed Hadamard); any readable bytes otherwise
    const int8_t *sp = a.rk.kind == KVQ_ROT_SIGNED_HADAMARD ? a.rk.signs + h * D : static_cast<const int8_t *>(a.q);
    sb0 = sp[lane];
    sb1 = sp[lane + 64];
  }
  // BF16 windows: this split's slice [wu0, wu1) of the window tokens (sink
  // positions [0, lo), then recent positions [hi, L)), in tiles of 16,
  // computed after the main loop
  const int n_sink = lo, n_win = lo + (L - hi);
  int wu0 = 0, wu1 = 0;
  if constexpr (kWin) {
    const int slice = 16 * ((((n_win + 15) / 16) + a.splits - 1) / a.splits);
    wu0 = min(s * slice, n_win);
    wu1 = min(wu0 + slice, n_win);
  }
  // dense R_K: thread (quarter kq = t / 128, column j = t % 128) holds
  // R_K[32 kq + i][j], i < 32, for the query rows' product below (each load
  // instruction reads 64 consecutive floats of one matrix row)
  // (eight named registers: an array here would be placed in LDS)
  float4 rs0, rs1, rs2, rs3, rs4, rs5, rs6, rs7;
  if constexpr (kDense) {
    const float *rm = a.rk.matrix + static_cast<size_t>(h) * D * D + (threadIdx.x >> 7) * 32 * D + (threadIdx.x & 127);
    auto col4 = [&](int i0) { return float4{rm[i0 * D], rm[(i0 + 1) * D], rm[(i0 + 2) * D], rm[(i0 + 3) * D]}; };
    rs0 = col4(0);
    rs1 = col4(4);
    rs2 = col4(8);
    rs3 = col4(12);
    rs4 = col4(16);
    rs5 = col4(20);
    rs6 = col4(24);
    rs7 = col4(28);
  }
  // blocks of the split: wave w starts with blocks w, w + 8, w + 16 and then
  // claims the next unclaimed block from an LDS counter (waves of one CU
  // progress at unequal speed; a static share would leave the slow waves'
  // tail unhidden)
  const int nb = c.t_end > t_begin ? (c.t_end - t_begin + kBlk - 1) / kBlk : 0;
  if (threadIdx.x == 0) s_claim[0] = 3 * kWaves;  // (read after the barriers below)
  // blocks jc[k] are in flight in buffer b[k]; ja[k] is a block whose
  // page-table entries were fetched into ad[k]
  int jc0 = wave, jc1 = wave + kWaves, jc2 = wave + 2 * kWaves, ja0 = 0, ja1 = 0, ja2 = 0;
  Blk b0, b1, b2;
  Addr a0, a1, a2;
  // the first two blocks are in flight while the query rows are prepared,
  // the third is issued after them (more loads ahead of the query rows'
  // slow down their arrival at the start of the kernel); unconditional:
  // every address is clamped into the split, or tile 0
  // (the third block's table entries are read after the first two blocks'
  // loads are out: scalar loads are awaited all at once, so reading them
  // with the first entries would hold those loads back by a round trip)
  load_addr<P16>(c, t_begin + kBlk * jc0, a0);
  load_addr<P16>(c, t_begin + kBlk * jc1, a1);
  if (nb == 0) {
    // an empty split (a sequence with no token here, perhaps none at all)
    // reads page 0, unused: its table entry 0 need not be valid
    repoint_all(a0);
    repoint_all(a1);
  }
  load_block<P16, NT>(c, a0, b0, bad);
  load_block<P16, NT>(c, a1, b1, bad);
  load_addr<P16>(c, t_begin + kBlk * jc2, a2);
  if (nb == 0) repoint_all(a2);
#ifdef KVQ_PHASE_TIMESTAMPS
  phase_t[9] = wall_clock64();  // (diagnostic: the first blocks' loads issued)
  {
    // (diagnostic: waits for this wave's query row)
    uint32_t qv = qb0;
    asm volatile("" : "+v"(qv));
    phase_t[10] = wall_clock64() + (qv & 0u);
  }
#endif

  // ---- query rows: q' = q R_K log2(e)/sqrt(128)
  {
    float y0 = 0.0f, y1 = 0.0f;
    if (wave < nrows) {
      y0 = DT == KVQ_F32 ? __uint_as_float(qb0) : __uint_as_float(qb0 << 16);
      y1 = DT == KVQ_F32 ? __uint_as_float(qb1) : __uint_as_float(qb1 << 16);
      if constexpr (!kDense)
        rotate_query_signed(y0, y1, a.rk.kind, static_cast<float>(sb0), static_cast<float>(sb1), lane);
    }
    if constexpr (kDense) {
      // q' = q R_K of the workgroup's rows (rows past the last are zero):
      // the raw rows go to qs; thread (kq, j) sums its quarter of column j
      // for the rows (fp32, four interleaved partial sums over i mod 4, added
      // pairwise; the rows' values are read by all lanes of a wave at once,
      // a row's eight reads issued together), the quarters meet in facc_all
      // (unused until the first flush) and are added in quarter order
      if (wave < kRows) {
        qs[wave][lane] = y0;
        qs[wave][lane + 64] = y1;
      }
      __syncthreads();
      const int kq = threadIdx.x >> 7, jc = threadIdx.x & 127;
      float pr[kRows];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const float4 *x4 = reinterpret_cast<const float4 *>(&qs[r][32 * kq]);
        const float4 rq[8] = {rs0, rs1, rs2, rs3, rs4, rs5, rs6, rs7};
        float4 x[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) x[m] = x4[m];
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          a0 += x[m].x * rq[m].x;
          a1 += x[m].y * rq[m].y;
          a2 += x[m].z * rq[m].z;
          a3 += x[m].w * rq[m].w;
        }
        pr[r] = (a0 + a1) + (a2 + a3);
      }
      float *qpart = &facc_all[0][0];  // [quarter][row][column]: 4 kRows D floats, within facc_all[0]
      static_assert(4 * kRows * D <= RG * kFaccFloats, "quarter sums fit in wave 0's accumulators");
#pragma unroll
      for (int r = 0; r < kRows; ++r) qpart[(kq * kRows + r) * D + jc] = pr[r];
      __syncthreads();
      if (wave < kRows) {
        auto col = [&](int j) {
          return ((qpart[(0 * kRows + wave) * D + j] + qpart[(1 * kRows + wave) * D + j]) +
                  qpart[(2 * kRows + wave) * D + j]) +
                 qpart[(3 * kRows + wave) * D + j];
        };
        y0 = col(lane) * (kLog2eF * kInvSqrtD);
        y1 = col(lane + 64) * (kLog2eF * kInvSqrtD);
      }
    }
    if (wave < kRows) {
      const float sum = wave_sum(y0 + y1);
      const float qabs = wave_maxf(fmaxf(fabsf(y0), fabsf(y1)));
      int e2 = 0;
      (void)frexpf(qabs, &e2);  // qabs < 2^e2
      qs[wave][lane] = y0;
      qs[wave][lane + 64] = y1;
      if (lane == 0) {
        qsum_s[wave] = sum;
        qshift_s[wave] = 26 - e2;
      }
    }
  }
  __syncthreads();
  // key-side A operand of each row group (row c = 4 r + d, k-slice g), one
  // dword per wave and row group, and this lane's query row g
  for (int d = wave; d < 8 * RG; d += kWaves)
    digit_s[d >> 3][d & 7][lane] = query_digit_word(&qs[4 * (d >> 3)], &qshift_s[4 * (d >> 3)], lane, (d & 7) >> 2, d & 3);
  __syncthreads();
  KVQ_PHASE(7);  // query digits ready
  State st[RG];
  const int hr = c.g;  // query row (within each group) of the key-side lanes
#pragma unroll
  for (int r = 0; r < RG; ++r) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[r].bk[m][e] = static_cast<int>(digit_s[r][4 * m + e][lane]);
    st[r].unscale = ldexpf(1.0f, -qshift_s[4 * r + hr]);
    st[r].qsum = qsum_s[4 * r + hr];
  }
  load_block<P16, NT>(c, a2, b2, bad);
  if (wave == 0) cnt_word = __hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // BF16 windows: the window rows' loads (win_load: lane (token n, g) takes
  // dims 32 ks + 8 g .. + 7 of token n of a tile; tokens past the slice read
  // its last token and are masked), issued when the wave's main loop ends
  const int wn = lane & 15, wg = lane >> 4, wr = wn >> 2, wpart = wn & 3;
  const int w_tiles = kWin ? (wu1 - wu0 + 15) / 16 : 0;
  uint4 wkr[kWin ? 2 : 1][4], wvr[kWin ? 2 : 1][4];
  auto win_load = [&](int t0, uint4 (&kr)[kWin ? 2 : 1][4], uint4 (&vr)[kWin ? 2 : 1][4]) {
    const size_t hstride = static_cast<size_t>(a.H) * D;  // elements between window tokens
    // the four window pointers as uniform values: a per-lane choice between
    // two argument fields would otherwise become a per-lane load of the
    // chosen field, and its wait would hold back every load in flight
    using gu16 = const __attribute__((address_space(1))) uint16_t;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    using gu4 = const __attribute__((address_space(1))) u32x4;
    auto uniform = [](const uint16_t *ptr) {
      // (readfirstlane returns an int: each half is widened as unsigned)
      const uint64_t v = reinterpret_cast<uint64_t>(ptr);
      const uint64_t w0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
      const uint64_t w1 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
      return (gu16 *)((w1 << 32) | w0);  // (global memory: loads stay off the LDS counter)
    };
    gu16 *sk = uniform(a.win_sk), *rk = uniform(a.win_rk), *sv = uniform(a.win_sv), *rv = uniform(a.win_rv);
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      const int u = min(wu0 + 16 * (t0 + kWaves * tl) + wn, wu1 - 1);
      const bool sink = u < n_sink;
      const size_t tok = sink ? static_cast<size_t>(b) * a.win_S + u
                              : static_cast<size_t>(b) * a.win_W + (hi + u - n_sink) % a.win_W;
      const size_t off = tok * hstride + static_cast<size_t>(h) * D + 8 * wg;
      gu16 *kp = (sink ? sk : rk) + off;
      gu16 *vp = (sink ? sv : rv) + off;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 kx = *reinterpret_cast<gu4 *>(kp + 32 * ks), vx = *reinterpret_cast<gu4 *>(vp + 32 * ks);
        kr[tl][ks] = uint4{kx.x, kx.y, kx.z, kx.w};
        vr[tl][ks] = uint4{vx.x, vx.y, vx.z, vx.w};
      }
    }
  };
  const int x = lane & 3;
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    st[r].tlim = c.t_end;
    if (a.causal) st[r].tlim = min(c.t_end, L - (a.Nq - 1 - (row0 + 4 * r + hr) / a.G));
    st[r].sel1 = (x & 1) ? 0x03070105u : 0x06020400u;
    st[r].sel2 = (x & 2) ? 0x03020706u : 0x05040100u;
    // value operand lane 16 g' + 4 r + x takes from lane 16 r + 4 g' + x
    st[r].src_lane4 = 4 * (16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + x);
    st[r].krow_lane4 = 4 * (16 * ((lane >> 2) & 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) st[r].accv[i] = v4i{0, 0, 0, 0};
    st[r].lsum = st[r].zsum = 0.0f;
    st[r].kappa = 0;
    st[r].have_ref = false;
    st[r].flushed = false;
  }

  // ---- main loop.  At the top of a step that computes block jc[k] (buffer
  // b[k]): the wave's next two blocks are in flight in the other buffers,
  // and ad[k] holds the page-table entries of the block after them (ja[k]).
  // A step claims one more block before the computation, then issues the
  // loads of ja[k] into the freed buffer and fetches the entries of the
  // claimed block into ad[k+1] (whose block was issued two steps earlier).
  // Claims increase, so a block past the split's end ends the loop; loads of
  // such blocks re-read the split's last tile and are not used.
  // (every lane takes part, lane 0 adding 1 to the counter and the others 0
  // to words of their own: no divergent branch in the loop, whose exits then
  // stay direct -- a restructured exit that could reach the loop head from
  // mid-body would make the first step wait for all three blocks in flight
  // -- and no bank conflict: 64 lanes on the counter's one word serialize)
  auto claim = [&]() -> uint32_t { return atomicAdd(&s_claim[lane], lane == 0 ? 1u : 0u); };
  ja0 = __builtin_amdgcn_readfirstlane(claim());
  load_addr<P16>(c, t_begin + kBlk * min(ja0, nb), a0);
  auto step = [&](Blk &bk, int &jc, Addr &ak, int &ja, Addr &ak1, int &ja1n) {
    const uint32_t v = claim();
    if (jc == nb - 1) mask_tail_meta(c, t_begin + kBlk * jc, bk);  // (wave-uniform: one block per split)
    compute_block<RG>(c, t_begin + kBlk * jc, bk, st, facc);
    load_block<P16, NT>(c, ak, bk, bad);
    jc = ja;
    ja1n = __builtin_amdgcn_readfirstlane(v);
    load_addr<P16>(c, t_begin + kBlk * min(ja1n, nb), ak1);
  };
  KVQ_PHASE(1);
#ifdef KVQ_PHASE_TIMESTAMPS
  {
    // (diagnostic: waits for the first block's key codes)
    uint32_t first = b0.kc[0].x;
    asm volatile("" : "+v"(first));
    phase_t[8] = wall_clock64() + (first & 0u);
  }
#endif
  // With BF16 windows the loop also ends once a round's last claim is past
  // the split's end; the blocks still in flight in b0, b1, b2 (claimed in
  // that order: a valid prefix) are then computed after the wave's first
  // window tiles are requested, so the tiles arrive while they are computed.
  bool drain = false;  // (wave-uniform)
  for (;;) {
    if (jc0 >= nb) break;
    step(b0, jc0, a0, ja0, a1, ja1);
    if (jc1 >= nb) break;
    step(b1, jc1, a1, ja1, a2, ja2);
    if (jc2 >= nb) break;
    step(b2, jc2, a2, ja2, a0, ja0);
    if constexpr (kWin) {
      if (ja0 >= nb) {
        drain = true;
        break;
      }
    }
  }
  if constexpr (kWin) {
    if (drain) {
      auto last = [&](int jc, Blk &bk) {
        if (jc == nb - 1) mask_tail_meta(c, t_begin + kBlk * jc, bk);
        compute_block<RG>(c, t_begin + kBlk * jc, bk, st, facc);
      };
      auto last3 = [&]() {
        if (jc0 < nb) last(jc0, b0);
        if (jc1 < nb) last(jc1, b1);
        if (jc2 < nb) last(jc2, b2);
      };
      if (w_tiles > 0) {
        // (every wave loads: past the slice's tiles the clamped tokens repeat
        // its last; no branch around the loads, so the blocks' waits stay exact)
        win_load(wave, wkr, wvr);
        last3();
      } else {
        last3();
      }
    }
  }

  KVQ_PHASE(2);
  uint4 wqv[kWin ? (DT == KVQ_F32 ? 8 : 4) : 1];
  float4 wmu[kWin ? 8 : 1];
  if constexpr (kWin) {
    // the raw query values and mu of the window key products' B operands
    // (lane (n, g), n = 4 r + part: row r, dims 32 ks + 8 g .. + 7), then
    // the wave's first window tiles (loads complete in issue order: the
    // operands are built while the tiles are on their way)
    const int r = row0 + min(wr, nrows - 1);
    const size_t rj = (static_cast<size_t>(b) * a.Nq + r / a.G) * a.Hq + h * a.G + r % a.G;
    const float *mu = a.win_mu ? a.win_mu + static_cast<size_t>(h) * D : nullptr;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d0 = 32 * ks + 8 * wg;
      if constexpr (DT == KVQ_F32) {
        const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.q) + rj * D + d0);
        wqv[2 * ks] = qp[0];
        wqv[2 * ks + 1] = qp[1];
      } else {
        wqv[ks] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + rj * D + d0);
      }
      const float4 *mp = reinterpret_cast<const float4 *>(mu ? mu + d0 : static_cast<const float *>(a.q));
      wmu[2 * ks] = mp[0];
      wmu[2 * ks + 1] = mp[1];
    }
    if (!drain && wave < w_tiles) win_load(wave, wkr, wvr);
  }
  // ---- this wave's partial of each row: m = -kappa, l, z, flag, acc[128]
  // (rows past the workgroup's last are computed and never stored)
  const bool any_bad = __any(bad);
  float *rw = red(wave, 0);  // [kRows + 1][132], private to this wave
  // value accumulators: lane (4 r + x, g') holds column x (digit x) of
  // query row r for dims 8 (4 g' + i) + 4 hf + e (an exact int32 sum).  The
  // lane's column times 256^x and the slot scale, summed over the quad (x = 0
  // keeps the sum).
  const int vr = (lane >> 2) & 3;
  const float wdig = x == 0 ? 1.0f : x == 1 ? 256.0f : x == 2 ? 65536.0f : 16777216.0f;
  const float wsc[4] = {wdig, wdig * 0.25f, wdig * 0.0625f, wdig};  // times slot_inv(e)
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    // (with two row groups, rw lies in this wave's flushed accumulators of
    // group 0: group g's are read before its rows are written, and rows
    // 0..kRows end before group 1's accumulators begin)
    static_assert(RG == 1 || (kRows + 1) * (D + 4) <= kFaccFloats, "partial rows within group 0's accumulators");
    const float lrow = row16_sum(st[g].lsum);
    const float zrow = row16_sum(st[g].zsum);
    float t[32];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) t[4 * k + i] = static_cast<float>(st[g].accv[k][i]);
    if (st[g].flushed) {
#pragma unroll
      for (int j = 0; j < 32; ++j) t[j] += facc[g * kFaccFloats + j * 64];
    }
    {
#pragma clang fp contract(off)
      // lanes x != 0 store their (unused) quad sums to row kRows
      const int lbase = x == 0 ? (4 * g + vr) * (D + 4) + 4 + 32 * c.g : kRows * (D + 4) + lane;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = t[4 * (4 * hf + e) + i] * wsc[e];
            v = v + fdpp_xor1(v);
            v = v + fdpp_xor2(v);
            rw[lbase + 8 * i + 4 * hf + e] = v;
          }
    }
    if (c.c == 0) {
      const bool empty = !st[g].have_ref;  // no token of this wave counted for row hr of group g
      float *rr = rw + (4 * g + hr) * (D + 4);
      rr[0] = empty ? -INFINITY : -static_cast<float>(st[g].kappa);
      rr[1] = any_bad ? __builtin_nanf("") : (empty ? 0.0f : lrow);
      rr[2] = empty ? 0.0f : zrow;
      rr[3] = 0.0f;
    }
  }
  // (an empty wave's accumulators are zero; the lanes of this wave read
  // each other's LDS writes below: LDS operations of a wave complete in
  // order, the fence keeps the compiler from reordering them)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // the INT2 partials of this split: merged over its waves (premerge) or
  // one per wave, stored for the merging workgroup (with BF16 windows before
  // the window work, so that the query and mu loads of the window operands
  // and the stores' acknowledgement overlap it)
  auto int2_partials = [&]() {
    if (a.premerge) {
      // more than one split: the 8 waves' partials of each row are merged
      // here first (one partial per split and row), so that the last split
      // merges one per split
      __syncthreads();
      if (wave < nrows) {
        const int r = wave;
        float mw[kWaves], mstar = -INFINITY;
  #pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          mw[w] = red(w, r)[0];
          mstar = fmaxf(mstar, mw[w]);
        }
        // every wave's (l, z, acc) read at once, then summed in wave order (a
        // wave without tokens adds nothing): one LDS round trip, not one per wave
        float lw[kWaves], zw[kWaves], x0[kWaves], x1[kWaves];
  #pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float *rwr = red(w, r);
          lw[w] = rwr[1];
          zw[w] = rwr[2];
          x0[w] = rwr[4 + lane];
          x1[w] = rwr[4 + 64 + lane];
        }
        float l = 0.0f, z = 0.0f, a0 = 0.0f, a1 = 0.0f;
        bool nan = false;
  #pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          nan = nan || lw[w] != lw[w];
          const float al = mw[w] == -INFINITY ? 0.0f : exp2f(mw[w] - mstar);
          const bool on = al != 0.0f;
          l += on ? al * lw[w] : 0.0f;
          z += on ? al * zw[w] : 0.0f;
          a0 += on ? al * x0[w] : 0.0f;
          a1 += on ? al * x1[w] : 0.0f;
        }
        const int rr = row0 + r;
        const size_t row = static_cast<size_t>(b) * a.Nq + rr / a.G;
        float *dst = a.part + ((row * a.Hq + h * a.G + rr % a.G) * a.pstride + s) * (D + 4);
        store_partial(dst + 4 + lane, a0);
        store_partial(dst + 4 + 64 + lane, a1);
        if (lane < 4) store_partial(dst + lane, lane == 0 ? mstar : lane == 1 ? (nan ? __builtin_nanf("") : l)
                                                                : lane == 2 ? z : 0.0f);
      }
    } else {
      // partial slot of this wave: split s, wave w -> s * kWaves + w; stored with
      // device-scope stores, consecutive lanes on consecutive floats
      {
        const int slot_w = s * kWaves + wave;
        float *rb[kRows];  // partial base of each row of the workgroup
  #pragma unroll
        for (int r = 0; r < kRows; ++r) {
          const int rr = min(row0 + r, a.R - 1);
          const size_t row = static_cast<size_t>(b) * a.Nq + rr / a.G;
          rb[r] = a.part + ((row * a.Hq + h * a.G + rr % a.G) * a.pstride + slot_w) * (D + 4);
        }
        constexpr int kN = (kRows * (D + 4) + 63) / 64;
        float vals[kN];
  #pragma unroll
        for (int k = 0; k < kN; ++k) vals[k] = rw[min(lane + 64 * k, kRows * (D + 4) - 1)];  // all reads, then the stores
  #pragma unroll
        for (int k = 0; k < kN; ++k) {
          const int idx = lane + 64 * k;
          // rows covered by idx in [64k, 64k + 63]: (64k) / 132 and (64k + 63) / 132
          constexpr int kRowStride = D + 4;
          const int r_lo = (64 * k) / kRowStride, r_hi = (64 * k + 63) / kRowStride;
          const int r = idx >= (r_lo + 1) * kRowStride ? r_hi : r_lo;
          if (idx < nrows * kRowStride) store_partial(rb[r] + (idx - r * kRowStride), vals[k]);
        }
      }
    }

  };
  if constexpr (kWin) {
    int2_partials();
    // ---- this split's window tokens [wu0, wu1) (fp32 products on the bf16
    // matrix cores), once its INT2 blocks are done: the window bytes are
    // read after the INT2 stream, not in the burst of the first blocks.  Each
    // wave takes 16-token tiles w, w + 8, ... in pairs (the first pair's
    // rows requested when its main loop ended):
    //   S^T = K Q^T (v_mfma_f32_16x16x32_bf16): A = the tile's key rows (bf16,
    //   exact), B = the raw query rows as 3 bf16 parts (built before the
    //   loop): lane (4 r + part, g) receives the part's products for tokens
    //   4g..4g+3, summed over the parts by two quad lane exchanges;
    //   out = P V: A = the weights p = 2^(x - m) as 3 bf16 parts (row 4 r +
    //   part; the k order of the 32 tokens is (tile 0, 4g + i), (tile 1,
    //   4g + i), which is where the key product left them), B = the values in
    //   that k order, transposed through the wave's 8 KB of facc_all (free
    //   once its partial rows are formed).
    // The 8 waves' (m, l, acc) meet in LDS; the split's window partial is
    // (m, l, 0, acc[128]), merged after the INT2 partials.
    // the B operands of the window key products: the raw query rows, scaled
    // to base-2 logits, as 3 bf16 parts (column n = 4 r + part, part 3 zero;
    // k-slice ks of lane (n, g) holds dims 32 ks + 8 g .. + 7), and q . mu of
    // the lane's row
    v8bf_w qop[4];
    float qmu_r = 0.0f;
    {
    const bool row_live = wr < nrows;
    float qm = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float qv[8];
      if constexpr (DT == KVQ_F32) {
        const uint4 u0 = wqv[2 * ks], u1 = wqv[2 * ks + 1];
        const uint32_t w8[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = __uint_as_float(w8[i]);
      } else {
        const uint4 u0 = wqv[ks];
        const uint32_t w4[4] = {u0.x, u0.y, u0.z, u0.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[i] = __uint_as_float((w4[i >> 1] >> (16 * (i & 1))) << 16);
      }
      const float4 m0 = wmu[2 * ks], m1 = wmu[2 * ks + 1];
      const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = row_live ? qv[i] * (kLog2eF * kInvSqrtD) : 0.0f;
        if (a.win_mu) qm += v * mv[i];
        const __bf16 hb = static_cast<__bf16>(v);
        const float r1 = v - static_cast<float>(hb);
        const __bf16 md = static_cast<__bf16>(r1);
        const __bf16 lo2 = static_cast<__bf16>(r1 - static_cast<float>(md));
        qop[ks][i] = wpart == 0 ? hb : wpart == 1 ? md : wpart == 2 ? lo2 : static_cast<__bf16>(0.0f);
      }
    }
    // q . mu of row wr: the lane holds 32 of its dims, the 4 lanes g the rest
    qm += lane_xor(qm, 16);
    qm += lane_xor(qm, 32);
    qmu_r = qm;
    }
    uint16_t *vt = reinterpret_cast<uint16_t *>(&facc_all[wave][0]);  // [128 dims][32 k positions] bf16
    float m_run = -INFINITY, l_part = 0.0f;  // row wr
    v4bf_f acc_o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc_o[dt] = v4bf_f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int t0 = wave; t0 < w_tiles; t0 += 2 * kWaves) {
      if (t0 != wave) win_load(t0, wkr, wvr);
      const int tt[2] = {t0, t0 + kWaves};
      // logits of row wr, tokens 4 wg + i of each tile
      float x[2][4];
      float cm = -INFINITY;
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        v4bf_f sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf_w, wkr[tl][ks]), qop[ks], sacc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[i];
          v += lane_xor(v, 1);
          v += lane_xor(v, 2);
          const bool ok = tt[tl] < w_tiles && wu0 + 16 * tt[tl] + 4 * wg + i < wu1;
          x[tl][i] = ok ? v - qmu_r : -INFINITY;
          cm = fmaxf(cm, x[tl][i]);
        }
      }
      cm = fmaxf(cm, lane_xor(cm, 16));
      cm = fmaxf(cm, lane_xor(cm, 32));
      const float mn = fmaxf(m_run, cm);  // finite: tile t0 holds a token
      const float al = m_run == -INFINITY ? 0.0f : exp2f(m_run - mn);
      m_run = mn;
      l_part *= al;
      // the output rows' rescale: lane (dim, g) holds rows g (parts 0..3)
      const float al_g = __shfl(al, 4 * wg);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc_o[dt] *= al_g;
      // weights as the A operand of P V: row 4 wr + wpart, k = 8 wg + 4 tile + i
      v8bf_w pa;
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = x[tl][i] == -INFINITY ? 0.0f : exp2f(x[tl][i] - mn);
          if (wpart == 0) l_part += pv;
          const __bf16 hb = static_cast<__bf16>(pv);
          const float r1 = pv - static_cast<float>(hb);
          const __bf16 md = static_cast<__bf16>(r1);
          const __bf16 lo2 = static_cast<__bf16>(r1 - static_cast<float>(md));
          pa[4 * tl + i] = wpart == 0 ? hb : wpart == 1 ? md : wpart == 2 ? lo2 : static_cast<__bf16>(0.0f);
        }
      // values transposed through LDS: vt[dim][8 (n / 4) + 4 tile + n % 4] from lane (token n, g)
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        const int pos = 8 * (wn >> 2) + 4 * tl + (wn & 3);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint32_t w4[4] = {wvr[tl][ks].x, wvr[tl][ks].y, wvr[tl][ks].z, wvr[tl][ks].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t hv = (w4[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            vt[(32 * ks + 8 * wg + i) * 32 + pos] = tt[tl] < w_tiles ? static_cast<uint16_t>(hv) : 0;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint4 vb = *reinterpret_cast<const uint4 *>(vt + (16 * dt + wn) * 32 + 8 * wg);
        acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(v8bf_w, vb), acc_o[dt], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    // the wave's row sums: l over the row's 16 lanes of part 0; out[row wg]
    // [16 dt + wn] = the parts' sum of acc_o[dt]
    l_part += lane_xor(l_part, 16);
    l_part += lane_xor(l_part, 32);
    float *wps = &facc_all[wave][0];  // [4 rows][4 + 128]: m, l, -, -, acc (after this wave's vt reads)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) wps[wg * (D + 4) + 4 + 16 * dt + wn] = acc_o[dt][0] + acc_o[dt][1] + acc_o[dt][2];
    if (wg == 0 && wpart == 0) {
      wps[wr * (D + 4)] = m_run;
      wps[wr * (D + 4) + 1] = l_part;
    }
    __syncthreads();
    // the 8 waves' partials of each (row, dim), then the window partial of
    // this split: slot parts + s (an empty slice stores m = -inf, l = 0)
    const int vrow = threadIdx.x >> 7, ad = threadIdx.x & 127;
    float ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) ms = fmaxf(ms, facc_all[w][vrow * (D + 4)]);
    float o = 0.0f, lw = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = facc_all[w][vrow * (D + 4)];
      const float sc = mw == -INFINITY ? 0.0f : exp2f(mw - ms);
      o += sc * facc_all[w][vrow * (D + 4) + 4 + ad];
      lw += sc * facc_all[w][vrow * (D + 4) + 1];
    }
    if (vrow < nrows) {
      const int rr = row0 + vrow;
      const size_t row = static_cast<size_t>(b) * a.Nq + rr / a.G;
      float *slot = a.part + ((row * a.Hq + h * a.G + rr % a.G) * a.pstride + a.parts + s) * (D + 4);
      store_partial(slot + 4 + ad, o);
      if (ad < 4) store_partial(slot + ad, ad == 0 ? ms : ad == 1 ? lw : 0.0f);
    }
    __syncthreads();  // (the partials read before LDS is used again)
  }
  if constexpr (!kWin) int2_partials();

  // ---- the last split of this row group to arrive merges all partials.
  // The partials travel between workgroups (and XCDs) through device-scope
  // stores and loads only; every store of this workgroup is acknowledged
  // (all counters drained) before its arrival is counted, and the merging
  // workgroup issues its loads after it has seen the final count.  No cache
  // write-back or invalidation is needed for that.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive_counted(cnt, cnt_word == arrival_valid_value(cnt, a.splits), a.epoch, a.splits) ? 1u : 0u;
  __syncthreads();
  KVQ_PHASE(3);
#ifdef KVQ_PHASE_TIMESTAMPS
  // (vector stores by lanes 0-11, one field each)
  auto phase_store = [&]() {
    const unsigned wid = ((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * kWaves + wave;
    if (wid < kPhaseWaves && lane < kPhaseFields) {
      const unsigned long long hw = static_cast<unsigned>(__builtin_amdgcn_s_getreg((31 << 11) | 4));  // HW_ID
      const unsigned long long xcc = static_cast<unsigned>(__builtin_amdgcn_s_getreg((3 << 11) | 20));  // XCC_ID
      const unsigned long long f[kPhaseFields] = {hw, xcc, static_cast<unsigned long long>(nb), phase_t[0],
                                                  phase_t[1], phase_t[2], phase_t[3], phase_t[4], phase_t[5],
                                                  phase_t[6], phase_t[7], phase_t[8], phase_t[9], phase_t[10]};
      unsigned long long v = f[0];
#pragma unroll
      for (int i = 1; i < kPhaseFields; ++i) v = lane == i ? f[i] : v;
      kvq_phase_ts[wid * kPhaseFields + lane] = v;
    }
  };
  if (s_last == 0) {
    phase_store();
    return;
  }
#else
  if (s_last == 0) return;
#endif
  const int qq = (row0 + min(wave, nrows - 1)) / a.G, j = h * a.G + (row0 + min(wave, nrows - 1)) % a.G;
  const size_t row = static_cast<size_t>(b) * a.Nq + qq;
  const float *base = a.part + (row * a.Hq + j) * a.pstride * (D + 4);
  // the merging waves request their partials first, then (dense R_V) the
  // matrix: a wave's loads complete in issue order, so the merge does not
  // wait for the matrix's 64 KB
  // (without a dense R_V, two copies of the merge: batches of 8 partials
  // when every count is at most 8, so that few copies of the last partial
  // are requested, and of 16, each with its own exact waits; with one, the
  // second copy alone: measured slower with both)
  const bool vdense = a.rv.kind == KVQ_ROT_DENSE;
  // (thread t holds R_V[t / 4][32 (t % 4) .. 32 (t % 4) + 31], 128 consecutive bytes)
  float4 v0, v1, v2, v3, v4, v5, v6, v7;
  float o0 = 0.0f, o1 = 0.0f, mi = -INFINITY, li = 0.0f;
  float ow0 = 0.0f, ow1 = 0.0f, mw = -INFINITY, lw = 0.0f;  // the windows' partials (one per split)
  auto merge_all = [&](auto batch) {
    constexpr int N = decltype(batch)::value;
    MergeIn in;
    if (wave < nrows) merge_load<N>(base, a.parts, lane, in);
    __builtin_amdgcn_sched_barrier(0);
    if (vdense) {
      const float4 *rm =
          reinterpret_cast<const float4 *>(a.rv.matrix + static_cast<size_t>(h) * D * D) + threadIdx.x * 8;
      v0 = rm[0];
      v1 = rm[1];
      v2 = rm[2];
      v3 = rm[3];
      v4 = rm[4];
      v5 = rm[5];
      v6 = rm[6];
      v7 = rm[7];
    }
    if (wave < nrows) {
      if constexpr (kWin)
        merge_partials<N>(base + static_cast<size_t>(a.parts) * (D + 4), a.splits, lane, ow0, ow1, &mw, &lw);
      merge_reduce<N>(base, a.parts, lane, in, o0, o1, &mi, &li);
    }
  };
  if constexpr (kDense) {
    MergeIn in;
    if (wave < nrows) merge_load(base, a.parts, lane, in);
    __builtin_amdgcn_sched_barrier(0);
    if (vdense) {
      const float4 *rm =
          reinterpret_cast<const float4 *>(a.rv.matrix + static_cast<size_t>(h) * D * D) + threadIdx.x * 8;
      v0 = rm[0];
      v1 = rm[1];
      v2 = rm[2];
      v3 = rm[3];
      v4 = rm[4];
      v5 = rm[5];
      v6 = rm[6];
      v7 = rm[7];
    }
    if (wave < nrows) {
      if constexpr (kWin)
        merge_partials(base + static_cast<size_t>(a.parts) * (D + 4), a.splits, lane, ow0, ow1, &mw, &lw);
      merge_reduce(base, a.parts, lane, in, o0, o1, &mi, &li);
    }
  } else if (a.parts <= 8 && (!kWin || a.splits <= 8)) {
    merge_all(std::integral_constant<int, 8>{});
  } else {
    merge_all(std::integral_constant<int, kMergeBatch>{});
  }
#ifdef KVQ_PHASE_TIMESTAMPS
  __builtin_amdgcn_s_waitcnt(0);
  KVQ_PHASE(4);
#endif
  if (vdense) {
    // out[r][i] = sum_c o'[r][c] R_V[i][c]: the rows' o' to LDS (rows past
    // the last are zero); thread t sums its 32 columns of row i = t / 4 for
    // each row (fp32, four interleaved partial sums over c mod 4, added
    // pairwise; a row's eight reads issued together, 4 addresses per
    // instruction), and the 4 threads of row i add their sums (lanes t ^ 1,
    // then t ^ 2)
    if (wave < kRows) {
      red(wave, 0)[lane] = o0;
      red(wave, 0)[lane + 64] = o1;
    }
    __syncthreads();
    const int ri = threadIdx.x >> 2, c0 = 32 * (threadIdx.x & 3);
    const float4 rv4[8] = {v0, v1, v2, v3, v4, v5, v6, v7};
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float4 *x4 = reinterpret_cast<const float4 *>(red(r, 0) + c0);
      float4 x[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = x4[m];
      float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        a0 += x[m].x * rv4[m].x;
        a1 += x[m].y * rv4[m].y;
        a2 += x[m].z * rv4[m].z;
        a3 += x[m].w * rv4[m].w;
      }
      float acc = (a0 + a1) + (a2 + a3);
      acc += fdpp_xor1(acc);
      acc += fdpp_xor2(acc);
      if ((threadIdx.x & 3) == 0) red(r, 1)[ri] = acc;
    }
    __syncthreads();
    o0 = red(wave < kRows ? wave : 0, 1)[lane];
    o1 = red(wave < kRows ? wave : 0, 1)[lane + 64];
  } else if (wave < nrows) {
    unrotate_value_wave(o0, o1, a.rv, h, lane);
  }
  if constexpr (kWin) {
    // o = (2^(m_int2 - M) l_int2 o_int2 + 2^(m_win - M) l_win o_win) / (2^(m_int2 - M) l_int2 + 2^(m_win - M) l_win),
    // both parts normalized and in the unrotated domain (NaN stays NaN)
    if (wave < nrows) {
      const float M = fmaxf(mi, mw);
      if (M == -INFINITY) {
        o0 = o1 = o0 != o0 ? o0 : 0.0f;
      } else {
        const float w1 = (mi == -INFINITY ? 0.0f : exp2f(mi - M)) * li;
        const float w2 = (mw == -INFINITY ? 0.0f : exp2f(mw - M)) * lw;
        const float den = w1 + w2;
        o0 = (w1 * o0 + w2 * ow0) / den;
        o1 = (w1 * o1 + w2 * ow1) / den;
      }
    }
  }
  KVQ_PHASE(5);
  if (wave < nrows) store_output_wave(a.out_o, a.ot, row, j, a.Hq, lane, o0, o1);
  if (a.y_zero && h == 0) {
    // the query positions of this group start their W_O rows at zero (the
    // projection that follows on the stream adds its K slices into them)
    for (int r = 0; r < nrows; ++r) {
      const int qr = (row0 + r) / a.G;
      if (r > 0 && qr == (row0 + r - 1) / a.G) continue;
      float *yr = a.y_zero + (static_cast<size_t>(b) * a.Nq + qr) * a.d_model;
      for (int i = threadIdx.x; i < a.d_model; i += 64 * kWaves) yr[i] = 0.0f;
    }
  }
#ifdef KVQ_PHASE_TIMESTAMPS
  __builtin_amdgcn_s_waitcnt(0);
  KVQ_PHASE(6);
  phase_store();
#endif
}

}  // namespace

bool decode_mfma_supported(const DecodePlan &pl, int page_size) {
  return pl.rows_per_head <= kMaxRows && page_size >= 16 && (page_size & (page_size - 1)) == 0 &&
         static_cast<int64_t>(pl.H) * 72 * page_size < (static_cast<int64_t>(1) << 31);
}

hipError_t launch_decode_mfma(const DecodePlan &pl, const void *q, int dtype, RotDev rk, RotDev rv,
                              const uint8_t *pages, int64_t num_pages, int page_size, const int32_t *page_table,
                              int max_pages, const int32_t *seq_lens, float *part, uint64_t *counters,
                              float *out_o, float *ot, hipStream_t stream, const WindowDev *win, bool causal,
                              float *y_zero, int d_model) {
  if (pl.num_seqs == 0) return hipSuccess;
  const uint32_t epoch = next_launch_epoch();
  MfmaArgs a{};
  a.R = pl.rows_per_head;
  a.G = pl.G;
  a.Hq = pl.Hq;
  a.H = pl.H;
  a.Nq = pl.queries_per_seq;
  a.n_rg = (pl.rows_per_head + 3) / 4;
  // two row groups per workgroup when there are two or more (the blocks'
  // codes are unpacked once for both), one with BF16 windows
  const int rg_per_wg = mfma_row_groups_per_workgroup(a.n_rg, page_size, win != nullptr);
  a.n_wy = (a.n_rg + rg_per_wg - 1) / rg_per_wg;
  a.split_tokens = pl.split_tokens;
  a.splits = pl.splits;
  a.premerge = pl.splits > kMaxSplitsNoPremerge ? 1 : 0;
  a.parts = a.premerge ? pl.splits : pl.splits * kWaves;
  a.pstride = a.parts + (win ? pl.splits : 0);
  a.causal = causal ? 1 : 0;
  a.max_seq_len = pl.max_seq_len;
  a.P = page_size;
  a.p_shift = __builtin_ctz(static_cast<unsigned>(page_size));
  a.max_pages = max_pages;
  if (page_table) {
    a.ptab = page_table;
    a.tab_stride = max_pages;
    a.tab_mask = a.val_mask = -1;
    a.id_mask = a.base_mul = 0;
  } else {
    a.ptab = seq_lens;  // read, then masked to zero
    a.tab_stride = a.tab_mask = a.val_mask = 0;
    a.id_mask = -1;
    a.base_mul = max_pages;
  }
  a.np32 = static_cast<uint32_t>(num_pages < INT32_MAX ? num_pages : INT32_MAX);
  a.page_bytes = static_cast<uint32_t>(pl.H) * 72u * static_cast<uint32_t>(page_size);
  a.pages = pages;
  a.seq_lens = seq_lens;
  a.q = q;
  a.rk = rk;
  a.rv = rv;
  a.part = part;
  a.counters = reinterpret_cast<unsigned long long *>(counters);
  a.epoch = epoch;
  a.out_o = out_o;
  a.ot = ot;
  a.y_zero = y_zero;
  a.d_model = d_model;
  if (win) {
    a.win_sk = win->sink_k;
    a.win_sv = win->sink_v;
    a.win_rk = win->recent_k;
    a.win_rv = win->recent_v;
    a.win_S = win->num_sink;
    a.win_W = win->num_recent;
    a.win_mu = win->key_mean;
  }
  const dim3 grid(pl.splits, pl.H * a.n_wy, pl.num_seqs);
  const bool f32 = dtype == KVQ_F32 || rk.kind == kRotPrescaled;
  const bool dense = rk.kind == KVQ_ROT_DENSE;
  const dim3 block(64 * kWaves);
  // (one workgroup per KV head along y: the cache bytes are read once, streamed)
  const bool nt = a.n_wy == 1;
#define KVQ_DECODE_LAUNCH(F32, P16, DENSE, WIN, NT, RG)                                                          \
  hipLaunchKernelGGL((decode_mfma_kernel<(F32) ? KVQ_F32 : KVQ_BF16, P16, DENSE, WIN, NT, RG>), grid, block, 0, \
                     stream, a)
  // 16-token pages: one row group (n_rg == 1: streamed) or two per workgroup
#define KVQ_DECODE_LAUNCH_16(F32, DENSE)                                        \
  do {                                                                          \
    if (win) KVQ_DECODE_LAUNCH(F32, true, DENSE, true, true, 1);                \
    else if (rg_per_wg == 1) KVQ_DECODE_LAUNCH(F32, true, DENSE, false, true, 1); \
    else if (nt) KVQ_DECODE_LAUNCH(F32, true, DENSE, false, true, 2);           \
    else KVQ_DECODE_LAUNCH(F32, true, DENSE, false, false, 2);                  \
  } while (0)
  // longer pages: one row group per workgroup
#define KVQ_DECODE_LAUNCH_P(F32, DENSE)                             \
  do {                                                              \
    if (win) KVQ_DECODE_LAUNCH(F32, false, DENSE, true, true, 1);   \
    else if (nt) KVQ_DECODE_LAUNCH(F32, false, DENSE, false, true, 1); \
    else KVQ_DECODE_LAUNCH(F32, false, DENSE, false, false, 1);     \
  } while (0)
  if (page_size == 16) {
    if (dense) {
      if (f32) KVQ_DECODE_LAUNCH_16(true, true); else KVQ_DECODE_LAUNCH_16(false, true);
    } else {
      if (f32) KVQ_DECODE_LAUNCH_16(true, false); else KVQ_DECODE_LAUNCH_16(false, false);
    }
  } else {
    if (dense) {
      if (f32) KVQ_DECODE_LAUNCH_P(true, true); else KVQ_DECODE_LAUNCH_P(false, true);
    } else {
      if (f32) KVQ_DECODE_LAUNCH_P(true, false); else KVQ_DECODE_LAUNCH_P(false, false);
    }
  }
#undef KVQ_DECODE_LAUNCH_P
#undef KVQ_DECODE_LAUNCH_16
#undef KVQ_DECODE_LAUNCH
  return hipGetLastError();
}

}  // namespace kvq

#ifdef KVQ_PHASE_TIMESTAMPS
// Diagnostic entry points of the phase-timestamp build (not part of
// libkvq.so): copy the per-wave records of the last launches to host memory
// (`bytes` at most kPhaseWaves x kPhaseFields x 8) and clear them; the wall
// clock's rate in kHz.
extern "C" int kvq_phase_timestamps(void *host, size_t bytes) {
  const size_t n = bytes < sizeof(kvq_phase_ts) ? bytes : sizeof(kvq_phase_ts);
  if (hipDeviceSynchronize() != hipSuccess) return 5;
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(kvq_phase_ts), n, 0, hipMemcpyDeviceToHost) != hipSuccess) return 5;
  static unsigned long long zeros[kPhaseWaves * kPhaseFields];
  return hipMemcpyToSymbol(HIP_SYMBOL(kvq_phase_ts), zeros, sizeof(zeros), 0, hipMemcpyHostToDevice) == hipSuccess
             ? 0
             : 5;
}
extern "C" int kvq_phase_clock_khz() {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1;
  return khz;
}
#endif
