// windows.hip -- BF16 sink and recent windows: the window write.
//
// [OptR] = "Output-Aware Rotation for INT2 KV-Cache Quantization", §5
// (implementation details: 64 sink and 256 recent tokens stay in BF16) and
// §4 (sink and recent tokens skip INT2 quantization; values stay unchanged
// in BF16).  A token at position p < num_sink goes to the sink, any later
// token to recent slot p % num_recent, so the slot of position p is reused by
// position p + num_recent, when p has left the recent window (with the
// sequences' lengths given, only the positions that end the write inside the
// recent window are written, so a write of many positions is deterministic).
#include "kvq_internal.h"

namespace kvq {
namespace {

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

struct WinWriteArgs {
  const void *k, *v;  // [n][H][128], dtype
  int64_t n;
  int H;
  const int32_t *seq_idx, *positions;
  const int32_t *seq_lens;  // [num_seqs] lengths after the write, or null
  int num_seqs;
  uint16_t *sk, *sv, *rk, *rv;
  int S, W;
};

// one thread per 8 consecutive elements of one (token, head): 16 per head
template <int DT>
__global__ __launch_bounds__(256) void window_write_kernel(WinWriteArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(a.H) * 16;
  if (idx >= a.n * per_tok) return;
  const int64_t i = idx / per_tok;
  const int rem = static_cast<int>(idx - i * per_tok);  // head * 16 + piece
  const int b = a.seq_idx[i], p = a.positions[i];
  if (b < 0 || b >= a.num_seqs || p < 0 || (a.seq_lens && p >= a.seq_lens[b])) return;
  uint16_t *dk, *dv;
  size_t dst;
  if (p < a.S) {
    dk = a.sk;
    dv = a.sv;
    dst = (static_cast<size_t>(b) * a.S + p) * a.H * D + 8 * static_cast<size_t>(rem);
  } else if (a.W > 0 && (!a.seq_lens || p >= a.seq_lens[b] - a.W)) {
    dk = a.rk;
    dv = a.rv;
    dst = (static_cast<size_t>(b) * a.W + p % a.W) * a.H * D + 8 * static_cast<size_t>(rem);
  } else {
    return;
  }
  const size_t src = static_cast<size_t>(i) * a.H * D + 8 * static_cast<size_t>(rem);
  uint4 ok, ov;
  if constexpr (DT == KVQ_BF16) {
    ok = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + src);
    ov = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v) + src);
  } else {
    const float4 *kp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.k) + src);
    const float4 *vp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.v) + src);
    const float4 k0 = kp[0], k1 = kp[1], v0 = vp[0], v1 = vp[1];
    ok = uint4{bf16_rne(k0.x) | (bf16_rne(k0.y) << 16), bf16_rne(k0.z) | (bf16_rne(k0.w) << 16),
               bf16_rne(k1.x) | (bf16_rne(k1.y) << 16), bf16_rne(k1.z) | (bf16_rne(k1.w) << 16)};
    ov = uint4{bf16_rne(v0.x) | (bf16_rne(v0.y) << 16), bf16_rne(v0.z) | (bf16_rne(v0.w) << 16),
               bf16_rne(v1.x) | (bf16_rne(v1.y) << 16), bf16_rne(v1.z) | (bf16_rne(v1.w) << 16)};
  }
  *reinterpret_cast<uint4 *>(dk + dst) = ok;
  *reinterpret_cast<uint4 *>(dv + dst) = ov;
}

}  // namespace

hipError_t launch_window_write(const void *k, const void *v, int dtype, int64_t num_tokens, int H,
                               const int32_t *seq_idx, const int32_t *positions, const int32_t *seq_lens,
                               int num_seqs, uint16_t *sink_k,
                               uint16_t *sink_v, uint16_t *recent_k, uint16_t *recent_v, int num_sink,
                               int num_recent, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  WinWriteArgs a{k, v, num_tokens, H, seq_idx, positions, seq_lens, num_seqs, sink_k, sink_v, recent_k, recent_v,
                 num_sink, num_recent};
  const int64_t threads = num_tokens * H * 16;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (dtype == KVQ_F32)
    hipLaunchKernelGGL(window_write_kernel<KVQ_F32>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(window_write_kernel<KVQ_BF16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
