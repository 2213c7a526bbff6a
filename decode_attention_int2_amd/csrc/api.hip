// api.hip -- the C ABI of libkvq: argument validation and launch order.
// Every check that can run on the host runs before the first launch.
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

uint32_t kvq::next_launch_epoch() {
  static std::atomic<uint32_t> next{
      static_cast<uint32_t>(std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761ull)};
  return next.fetch_add(1);
}

int kvq::device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;  // (no device visible: the sizes of an MI355X)
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

bool valid_dtype(int32_t dt) { return dt == KVQ_F32 || dt == KVQ_BF16; }

// 0 = ok, else a kvq_status.
int check_rotation(const kvq_rotation *r) {
  if (!r) return KVQ_ERR_INVALID_ARGUMENT;
  switch (r->kind) {
    case KVQ_ROT_IDENTITY:
      return KVQ_OK;
    case KVQ_ROT_SIGNED_HADAMARD:
      return r->signs ? KVQ_OK : KVQ_ERR_INVALID_ARGUMENT;
    case KVQ_ROT_DENSE:  // (read with 16-byte vector loads)
      return r->matrix && (reinterpret_cast<uintptr_t>(r->matrix) & 15u) == 0 ? KVQ_OK : KVQ_ERR_INVALID_ARGUMENT;
    default:
      return KVQ_ERR_UNSUPPORTED;
  }
}

bool valid_clip(float c) { return std::isfinite(c) && c > 0.0f && c <= 1.0f; }

int check_cache(const kvq_cache *c) {
  if (!c || !c->pages) return KVQ_ERR_INVALID_ARGUMENT;
  if (c->num_pages < 1 || c->num_kv_heads < 1 || c->page_size < 16 || c->page_size % 16) return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

// 0 = ok, else a kvq_status.
int check_windows(const kvq_windows *w, int H) {
  if (!w) return KVQ_ERR_INVALID_ARGUMENT;
  if (w->num_seqs < 1 || w->num_kv_heads != H || H < 1 || w->num_sink < 0 || w->num_recent < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (w->num_sink % 16) return KVQ_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(w->num_sink) + w->num_recent > kMaxWindowTokens) return KVQ_ERR_UNSUPPORTED;
  if (w->num_sink > 0 && (!w->sink_k || !w->sink_v)) return KVQ_ERR_INVALID_ARGUMENT;
  if (w->num_recent > 0 && (!w->recent_k || !w->recent_v)) return KVQ_ERR_INVALID_ARGUMENT;
  for (const void *p : {static_cast<const void *>(w->sink_k), static_cast<const void *>(w->sink_v),
                        static_cast<const void *>(w->recent_k), static_cast<const void *>(w->recent_v)})
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// K, V, q and W_O are read with 16-byte vector loads (null passes: checked elsewhere)
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct CandidateLayout {
  int64_t num_pages;
  DecodePlan plan;      // matrix-core decode of the quantized variants
  DecodePlan ref_plan;  // full-precision reference readout (fp32 matrix cores): more splits
  size_t cache_bytes;
  size_t off_cache, off_dec, off_refdec, off_seqlen, off_ohat, off_oref, off_nmse, off_gram, off_den, total;
};

CandidateLayout candidate_layout(int64_t T, int H, int Hq, int Nq, int C, int n_clip) {
  CandidateLayout L{};
  L.num_pages = (T + 15) / 16;
  L.plan = make_decode_plan(1, Nq, Hq, H, static_cast<int>(T), 0, 0);
  // the reference kernel runs one wave per (split, KV head, 16 rows): ~4096 waves
  const int ref_waves = H * ((Nq * (Hq / H) + 15) / 16);
  const int ref_splits = (4096 + ref_waves - 1) / ref_waves;
  L.ref_plan = make_decode_plan(1, Nq, Hq, H, static_cast<int>(T), 0, ref_splits);
  const int U = H;  // upper bound over both modes
  size_t off = 0;
  L.off_cache = off;  // one cache per clip ratio
  L.cache_bytes = align256(kvq_cache_bytes(L.num_pages, 16, H));
  off = align256(off + L.cache_bytes * n_clip);
  L.off_dec = off;
  off = align256(off + L.plan.total);
  L.off_refdec = off;
  off = align256(off + L.ref_plan.total);
  L.off_seqlen = off;
  off = align256(off + sizeof(int32_t));
  L.off_ohat = off;  // decoded outputs of every variant [C * n_clip][Nq][Hq][128]
  off = align256(off + static_cast<size_t>(C) * n_clip * Nq * Hq * D * sizeof(float));
  L.off_oref = off;
  off = align256(off + static_cast<size_t>(Nq) * Hq * D * sizeof(float));
  L.off_nmse = off;
  off = align256(off + static_cast<size_t>(U) * C * n_clip * Nq * sizeof(float));
  L.off_gram = off;  // Gram blocks of W_O, sized for the larger of the two modes
  off = align256(off + std::max(nmse_gram_floats(Hq, H, KVQ_SELECT_JOINT), nmse_gram_floats(Hq, H, KVQ_SELECT_PER_HEAD)) *
                           sizeof(float));
  L.off_den = off;   // reference output norms [U][Nq]
  off = align256(off + static_cast<size_t>(U) * Nq * sizeof(double));
  L.total = off;
  return L;
}

#define KVQ_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return KVQ_ERR_HIP; \
  } while (0)

}  // namespace

extern "C" {

size_t kvq_cache_bytes(int64_t num_pages, int32_t page_size, int32_t num_kv_heads) {
  if (num_pages < 0 || page_size < 0 || num_kv_heads < 0) return 0;
  return static_cast<size_t>(num_pages) * static_cast<size_t>(num_kv_heads) * 72u * static_cast<size_t>(page_size);
}

int kvq_quantize(const void *k, const void *v, int32_t dtype, int64_t num_tokens, const int64_t *slot_mapping,
                 const kvq_rotation *rot_k, const kvq_rotation *rot_v, const float *key_mean, float clip_k,
                 float clip_v, const kvq_cache *cache, hipStream_t stream) {
  if (!valid_dtype(dtype)) return KVQ_ERR_UNSUPPORTED;
  if (num_tokens < 0) return KVQ_ERR_INVALID_ARGUMENT;
  int rc = check_rotation(rot_k);
  if (rc) return rc;
  rc = check_rotation(rot_v);
  if (rc) return rc;
  rc = check_cache(cache);
  if (rc) return rc;
  if (!valid_clip(clip_k) || !valid_clip(clip_v)) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && (!k || !v)) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return KVQ_OK;
  KVQ_TRY(launch_quantize(k, v, dtype, num_tokens, cache->num_kv_heads, slot_mapping, to_dev(*rot_k),
                          to_dev(*rot_v), key_mean, clip_k, clip_v, cache->pages, cache->num_pages, cache->page_size,
                          stream));
  return KVQ_OK;
}

size_t kvq_decode_workspace_bytes(int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t max_seq_len, int32_t d_model, int32_t num_splits) {
  if (num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  return make_decode_plan(num_seqs, queries_per_seq, num_q_heads, num_kv_heads, max_seq_len, d_model > 0 ? d_model : 0,
                          num_splits, 0)
      .total;
}

// kvq_decode_attn and kvq_decode_attn_windows (windows: NULL for none)
static int decode_attn(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                       const kvq_cache *cache, const int32_t *page_table, int32_t max_pages_per_seq,
                       const int32_t *seq_lens, int32_t max_seq_len, const kvq_rotation *rot_k,
                       const kvq_rotation *rot_v, const kvq_windows *windows, const float *key_mean, const void *w_o,
                       int32_t d_model, float *out_o, float *out_y, void *workspace, size_t workspace_bytes,
                       int32_t num_splits, const kvq_decode_events *events, hipStream_t stream,
                       bool causal = false) {
  if (!valid_dtype(dtype)) return KVQ_ERR_UNSUPPORTED;
  int rc = check_cache(cache);
  if (rc) return rc;
  rc = check_rotation(rot_k);
  if (rc) return rc;
  rc = check_rotation(rot_v);
  if (rc) return rc;
  if (num_seqs < 0 || queries_per_seq < 1 || num_q_heads < 1 || max_pages_per_seq < 1 || max_seq_len < 0 ||
      num_splits < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  const int H = cache->num_kv_heads;
  if (num_q_heads % H) return KVQ_ERR_INVALID_ARGUMENT;
  if (static_cast<int64_t>(queries_per_seq) * (num_q_heads / H) > kMaxRows) return KVQ_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_pages_per_seq) * cache->page_size)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (static_cast<int64_t>(max_seq_len) > kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  if (!page_table && static_cast<int64_t>(num_seqs) * max_pages_per_seq > cache->num_pages)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (w_o && (d_model < 1 || !out_y)) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0 && (!q || !seq_lens || !out_o)) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(w_o)) return KVQ_ERR_INVALID_ARGUMENT;
  if (windows) {
    rc = check_windows(windows, H);
    if (rc) return rc;
    if (windows->num_seqs < num_seqs) return KVQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(key_mean)) return KVQ_ERR_INVALID_ARGUMENT;  // (read with 16-byte loads)
  }
  const DecodePlan pl = make_decode_plan(num_seqs, queries_per_seq, num_q_heads, H, max_seq_len,
                                         w_o ? d_model : 0, num_splits, cache->page_size, windows != nullptr);
  if (pl.total > 0 && (!workspace || workspace_bytes < pl.total)) return KVQ_ERR_WORKSPACE;
  if (num_seqs == 0) return KVQ_OK;
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  float *qrot = reinterpret_cast<float *>(ws + pl.off_qrot);
  float *qsum = reinterpret_cast<float *>(ws + pl.off_qsum);
  float *part = reinterpret_cast<float *>(ws + pl.off_part);
  float *ot = w_o ? reinterpret_cast<float *>(ws + pl.off_ot) : nullptr;
  const RotDev rk = to_dev(*rot_k), rv = to_dev(*rot_v);
  if ((windows || causal) && !decode_mfma_supported(pl, cache->page_size)) return KVQ_ERR_UNSUPPORTED;
  if (windows && causal) return KVQ_ERR_UNSUPPORTED;
  WindowDev wd{};
  if (windows) {
    wd.sink_k = static_cast<const uint16_t *>(windows->sink_k);
    wd.sink_v = static_cast<const uint16_t *>(windows->sink_v);
    wd.recent_k = static_cast<const uint16_t *>(windows->recent_k);
    wd.recent_v = static_cast<const uint16_t *>(windows->recent_v);
    wd.num_sink = windows->num_sink;
    wd.num_recent = windows->num_recent;
    wd.key_mean = key_mean;
  }
  if (decode_mfma_supported(pl, cache->page_size)) {
    // one launch: query rotation, split attention, merge, R_V^T
    if (events && events->split_start) KVQ_TRY(hipEventRecord(events->split_start, stream));
    KVQ_TRY(launch_decode_mfma(pl, q, dtype, rk, rv, cache->pages, cache->num_pages, cache->page_size, page_table,
                               max_pages_per_seq, seq_lens, part, reinterpret_cast<uint64_t *>(ws + pl.off_cnt),
                               out_o, ot, stream, windows ? &wd : nullptr, causal, w_o ? out_y : nullptr,
                               pl.d_model));
    if (events && events->split_stop) KVQ_TRY(hipEventRecord(events->split_stop, stream));
  } else {
    KVQ_TRY(launch_query_rotation(q, dtype, pl, rk, qrot, qsum, stream));
    if (events && events->split_start) KVQ_TRY(hipEventRecord(events->split_start, stream));
    KVQ_TRY(launch_decode_split(pl, cache->pages, cache->num_pages, cache->page_size, page_table, max_pages_per_seq,
                                seq_lens, qrot, qsum, part, stream));
    if (events && events->split_stop) KVQ_TRY(hipEventRecord(events->split_stop, stream));
    KVQ_TRY(launch_combine(pl, part, rv, out_o, ot, stream, w_o ? out_y : nullptr));
  }
  if (events && events->attn_stop) KVQ_TRY(hipEventRecord(events->attn_stop, stream));
  if (w_o)
    KVQ_TRY(launch_wo_projection(pl, ot, w_o, dtype, out_y, stream));
  return KVQ_OK;
}

int kvq_decode_attn(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq, int32_t num_q_heads,
                    const kvq_cache *cache, const int32_t *page_table, int32_t max_pages_per_seq,
                    const int32_t *seq_lens, int32_t max_seq_len, const kvq_rotation *rot_k,
                    const kvq_rotation *rot_v, const void *w_o, int32_t d_model, float *out_o, float *out_y,
                    void *workspace, size_t workspace_bytes, int32_t num_splits, const kvq_decode_events *events,
                    hipStream_t stream) {
  return decode_attn(q, dtype, num_seqs, queries_per_seq, num_q_heads, cache, page_table, max_pages_per_seq, seq_lens,
                     max_seq_len, rot_k, rot_v, nullptr, nullptr, w_o, d_model, out_o, out_y, workspace,
                     workspace_bytes, num_splits, events, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation decode
// Scratch of kvq_decode_attn_noalloc: a file-scope device array, one copy per
// GPU for the life of the process.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device, with that device current, and kept.
namespace {
static __device__ __align__(256) uint8_t scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxScratchDevices];

// 0 = ok (the current device's scratch address in *out), else a kvq_status.
int current_scratch(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace

extern "C" {

int kvq_decode_attn_noalloc(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                            int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                            int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            const kvq_rotation *rot_k, const kvq_rotation *rot_v, const void *w_o, int32_t d_model,
                            float *out_o, float *out_y, int32_t num_splits, hipStream_t stream) {
  void *ws = nullptr;
  const int rc = current_scratch(&ws);
  if (rc) return rc;
  // (the shared decode path validates every argument first and returns
  // KVQ_ERR_WORKSPACE, launching nothing, when the plan needs more scratch)
  return decode_attn(q, dtype, num_seqs, queries_per_seq, num_q_heads, cache, page_table, max_pages_per_seq, seq_lens,
                     max_seq_len, rot_k, rot_v, nullptr, nullptr, w_o, d_model, out_o, out_y, ws,
                     KVQ_NOALLOC_SCRATCH_BYTES, num_splits, nullptr, stream);
}

int kvq_decode_attn_windows(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                            int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                            int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            const kvq_rotation *rot_k, const kvq_rotation *rot_v, const kvq_windows *windows,
                            const float *key_mean, const void *w_o, int32_t d_model, float *out_o, float *out_y,
                            void *workspace, size_t workspace_bytes, int32_t num_splits, hipStream_t stream) {
  if (!windows) return KVQ_ERR_INVALID_ARGUMENT;
  return decode_attn(q, dtype, num_seqs, queries_per_seq, num_q_heads, cache, page_table, max_pages_per_seq, seq_lens,
                     max_seq_len, rot_k, rot_v, windows, key_mean, w_o, d_model, out_o, out_y, workspace,
                     workspace_bytes, num_splits, nullptr, stream);
}

int kvq_decode_attn_causal(const void *q, int32_t dtype, int32_t num_seqs, int32_t queries_per_seq,
                           int32_t num_q_heads, const kvq_cache *cache, const int32_t *page_table,
                           int32_t max_pages_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                           const kvq_rotation *rot_k, const kvq_rotation *rot_v, const void *w_o, int32_t d_model,
                           float *out_o, float *out_y, void *workspace, size_t workspace_bytes, int32_t num_splits,
                           hipStream_t stream) {
  return decode_attn(q, dtype, num_seqs, queries_per_seq, num_q_heads, cache, page_table, max_pages_per_seq, seq_lens,
                     max_seq_len, rot_k, rot_v, nullptr, nullptr, w_o, d_model, out_o, out_y, workspace,
                     workspace_bytes, num_splits, nullptr, stream, true);
}

int kvq_window_write(const void *k, const void *v, int32_t dtype, int64_t num_tokens, const int32_t *seq_idx,
                     const int32_t *positions, const int32_t *seq_lens, const kvq_windows *windows,
                     hipStream_t stream) {
  if (!valid_dtype(dtype)) return KVQ_ERR_UNSUPPORTED;
  if (!windows) return KVQ_ERR_INVALID_ARGUMENT;
  const int rc = check_windows(windows, windows->num_kv_heads);
  if (rc) return rc;
  if (num_tokens < 0 || num_tokens > INT32_MAX) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens > 0 && (!k || !v || !seq_idx || !positions)) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v)) return KVQ_ERR_INVALID_ARGUMENT;
  KVQ_TRY(launch_window_write(k, v, dtype, num_tokens, windows->num_kv_heads, seq_idx, positions, seq_lens,
                              windows->num_seqs,
                              static_cast<uint16_t *>(windows->sink_k), static_cast<uint16_t *>(windows->sink_v),
                              static_cast<uint16_t *>(windows->recent_k), static_cast<uint16_t *>(windows->recent_v),
                              windows->num_sink, windows->num_recent, stream));
  return KVQ_OK;
}

int kvq_fold_value_rotation(const void *w, int32_t dtype, int32_t num_blocks, int32_t blocks_per_head, int32_t cols,
                            const kvq_rotation *rot_v, void *out, hipStream_t stream) {
  if (!valid_dtype(dtype)) return KVQ_ERR_UNSUPPORTED;
  const int rc = check_rotation(rot_v);
  if (rc) return rc;
  if (!w || !out || num_blocks < 1 || blocks_per_head < 1 || cols < 1 || num_blocks % blocks_per_head ||
      num_blocks > 65535)
    return KVQ_ERR_INVALID_ARGUMENT;
  const size_t bytes = static_cast<size_t>(num_blocks) * D * cols * (dtype == KVQ_F32 ? 4 : 2);
  const uintptr_t wa = reinterpret_cast<uintptr_t>(w), oa = reinterpret_cast<uintptr_t>(out);
  if (wa < oa + bytes && oa < wa + bytes) return KVQ_ERR_INVALID_ARGUMENT;  // overlapping buffers
  KVQ_TRY(launch_fold_value_rotation(w, dtype, num_blocks, blocks_per_head, cols, to_dev(*rot_v), out, stream));
  return KVQ_OK;
}

double kvq_bits_per_element(int64_t seq_len, int32_t num_sink, int32_t num_recent) {
  if (seq_len <= 0 || num_sink < 0 || num_recent < 0) return 0.0;
  // window tokens: 128 bf16 per (head, side); INT2 tokens: 32 code bytes + fp16 scale and zero
  const int64_t in_sink = seq_len < num_sink ? seq_len : num_sink;
  const int64_t in_recent = seq_len - in_sink < num_recent ? seq_len - in_sink : num_recent;
  const int64_t int2 = seq_len - in_sink - in_recent;
  const double bits = static_cast<double>(int2) * (8.0 * (32 + 4)) + static_cast<double>(in_sink + in_recent) * 2048.0;
  return bits / (static_cast<double>(seq_len) * 128.0);
}

size_t kvq_candidate_workspace_bytes(int64_t num_tokens, int32_t num_kv_heads, int32_t num_q_heads,
                                     int32_t num_queries, int32_t num_candidates, int32_t num_clips,
                                     int32_t d_model) {
  (void)d_model;
  if (num_tokens < 1 || num_tokens > INT32_MAX || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads || num_queries < 1 || num_candidates < 1 || num_clips < 1)
    return 0;
  return candidate_layout(num_tokens, num_kv_heads, num_q_heads, num_queries, num_candidates, num_clips).total;
}

int kvq_candidate_nmse(const void *k, const void *v, const void *q, int32_t dtype, int64_t num_tokens,
                       int32_t num_kv_heads, int32_t num_q_heads, int32_t num_queries,
                       const kvq_rotation *candidates, int32_t num_candidates, const float *clips,
                       int32_t num_clips, const float *key_mean, const void *w_o, int32_t d_model, int32_t mode,
                       float *out_nmse, float *out_nmse_per_query, int32_t *out_best, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return KVQ_ERR_UNSUPPORTED;
  if (mode != KVQ_SELECT_JOINT && mode != KVQ_SELECT_PER_HEAD) return KVQ_ERR_UNSUPPORTED;
  if (!k || !v || !q || !candidates || !clips || !w_o || !out_nmse || !out_best) return KVQ_ERR_INVALID_ARGUMENT;
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(w_o)) return KVQ_ERR_INVALID_ARGUMENT;
  if (num_tokens < 1 || num_tokens > INT32_MAX || num_kv_heads < 1 || num_q_heads < 1 || num_queries < 1 ||
      num_candidates < 1 || num_clips < 1 || d_model < 1)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (num_q_heads % num_kv_heads) return KVQ_ERR_INVALID_ARGUMENT;
  const int H = num_kv_heads, Hq = num_q_heads, G = Hq / H, Nq = num_queries;
  if (static_cast<int64_t>(Nq) * G > kMaxRows) return KVQ_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(num_candidates) * num_clips > INT32_MAX) return KVQ_ERR_UNSUPPORTED;
  if (mode == KVQ_SELECT_JOINT && Hq > 64) return KVQ_ERR_UNSUPPORTED;  // joint Gram block of Hq * 128 rows
  for (int r = 0; r < num_candidates; ++r) {
    const int rc = check_rotation(&candidates[r]);
    if (rc) return rc;
  }
  for (int i = 0; i < num_clips; ++i)
    if (!valid_clip(clips[i])) return KVQ_ERR_INVALID_ARGUMENT;
  const CandidateLayout L = candidate_layout(num_tokens, H, Hq, Nq, num_candidates, num_clips);
  if (!workspace || workspace_bytes < L.total) return KVQ_ERR_WORKSPACE;

  uint8_t *ws = static_cast<uint8_t *>(workspace);
  uint8_t *pages = ws + L.off_cache;
  uint8_t *dec = ws + L.off_dec;
  int32_t *seq_len = reinterpret_cast<int32_t *>(ws + L.off_seqlen);
  float *o_hat_all = reinterpret_cast<float *>(ws + L.off_ohat);
  float *o_ref = reinterpret_cast<float *>(ws + L.off_oref);
  float *nmse_q = out_nmse_per_query ? out_nmse_per_query : reinterpret_cast<float *>(ws + L.off_nmse);
  const DecodePlan &pl = L.plan;
  float *qrot = reinterpret_cast<float *>(dec + pl.off_qrot);
  float *qsum = reinterpret_cast<float *>(dec + pl.off_qsum);
  float *part = reinterpret_cast<float *>(dec + pl.off_part);
  uint64_t *counters = reinterpret_cast<uint64_t *>(dec + pl.off_cnt);
  const bool mfma = decode_mfma_supported(pl, 16);
  const RotDev ident{KVQ_ROT_IDENTITY, nullptr, nullptr};
  const int U = (mode == KVQ_SELECT_JOINT) ? 1 : H;
  const size_t stride_u = static_cast<size_t>(num_candidates) * num_clips * Nq;

  // Full-precision reference readout of the raw K, V (own plan and workspace region).
  {
    const DecodePlan &rp = L.ref_plan;
    uint8_t *rdec = ws + L.off_refdec;
    float *rq = reinterpret_cast<float *>(rdec + rp.off_qrot);
    float *rs = reinterpret_cast<float *>(rdec + rp.off_qsum);
    float *rpart = reinterpret_cast<float *>(rdec + rp.off_part);
    KVQ_TRY(launch_query_rotation(q, dtype, rp, ident, rq, rs, stream));
    KVQ_TRY(launch_reference_split(rp, k, v, dtype, num_tokens, rq, rpart, stream));
    KVQ_TRY(launch_combine(rp, rpart, ident, o_ref, nullptr, stream));
  }
  float *gram = reinterpret_cast<float *>(ws + L.off_gram);
  double *den = reinterpret_cast<double *>(ws + L.off_den);
  KVQ_TRY(launch_nmse_prepare(o_ref, w_o, dtype, Nq, Hq, H, d_model, mode, gram, den, stream));
  KVQ_TRY(launch_fill_i32(seq_len, static_cast<int32_t>(num_tokens), 1, stream));
  for (int r = 0; r < num_candidates; ++r) {
    const RotDev rot = to_dev(candidates[r]);
    // matrix-core path: queries rotated inside the decode launch
    if (!mfma) KVQ_TRY(launch_query_rotation(q, dtype, pl, rot, qrot, qsum, stream));
    // the candidate's caches of every clip ratio in one pass (one rotation)
    KVQ_TRY(launch_quantize_clips(k, v, dtype, num_tokens, H, nullptr, rot, rot, key_mean, clips, clips, num_clips,
                                  pages, L.num_pages, 16, L.cache_bytes, stream));
    for (int i = 0; i < num_clips; ++i) {
      uint8_t *pages_i = pages + static_cast<size_t>(i) * L.cache_bytes;
      float *o_hat = o_hat_all + (static_cast<size_t>(r) * num_clips + i) * Nq * Hq * D;
      if (mfma) {
        KVQ_TRY(launch_decode_mfma(pl, q, dtype, rot, rot, pages_i, L.num_pages, 16, nullptr,
                                   static_cast<int>(L.num_pages), seq_len, part, counters, o_hat, nullptr, stream));
      } else {
        KVQ_TRY(launch_decode_split(pl, pages_i, L.num_pages, 16, nullptr, static_cast<int>(L.num_pages), seq_len,
                                    qrot, qsum, part, stream));
        KVQ_TRY(launch_combine(pl, part, rot, o_hat, nullptr, stream));
      }
    }
  }
  // post-W_O NMSE of every variant in one launch
  KVQ_TRY(launch_nmse_terms(o_hat_all, o_ref, gram, den, Nq, Hq, H, mode, num_candidates * num_clips, nmse_q, stride_u,
                            stream));
  KVQ_TRY(launch_select(nmse_q, U, num_candidates, num_clips, Nq, out_nmse, out_best, stream));
  return KVQ_OK;
}

const char *kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK:
      return "KVQ_OK";
    case KVQ_ERR_INVALID_ARGUMENT:
      return "KVQ_ERR_INVALID_ARGUMENT";
    case KVQ_ERR_UNSUPPORTED:
      return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE:
      return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_HIP:
      return "KVQ_ERR_HIP";
    default:
      return "KVQ_UNKNOWN_STATUS";
  }
}

int kvq_version(void) { return KVQ_VERSION; }

}  // extern "C"
