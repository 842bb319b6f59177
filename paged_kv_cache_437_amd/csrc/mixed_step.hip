// Prefill and decode of one step in a single launch (“深入 Nano-vLLM 推理引擎”, "Prefill and
// Decode" and the scheduler headings: a step's batch holds sequences in both phases).
// The grid is the decode pass's workgroups followed by the prefill's work items; a
// workgroup runs one or the other whole (decode_kernel.h, prefill_kernel.h), so the
// HBM-bound decode and the MFMA-bound prefill share the CUs instead of running one
// after the other.  The decode's merge kernel follows as its own launch.
#include "decode_kernel.h"
#include "prefill_kernel.h"

namespace pkv {

// GP: the decode pass's q heads per stream (G rounded down to a power of two, the
// rest in further streams); PGP: the prefill pass's q heads per work item, which must
// cover all G of a kv head (G rounded up to a power of two).
template <int D, int GP, int PGP, int MH, bool ROT>
__global__ __launch_bounds__(256, 2) void mixed_attention_bf16_kernel(
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache, int Hq, int Hkv,
    int G, int bs_log2, float scale_log2, const float* __restrict__ cos_sin, int max_position,
    int n_decode_wg,
    // decode
    const uint16_t* __restrict__ dq, uint16_t* __restrict__ dout,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ d_tables,
    int d_stride, int d_batch, int n_hg, int num_workers, int64_t* __restrict__ ws_prefix,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o,
    // prefill
    const uint16_t* __restrict__ pq, uint16_t* __restrict__ pout,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ p_tables, int p_stride, int p_batch, int max_tiles) {
  if (static_cast<int>(blockIdx.x) < n_decode_wg)
    decode_workgroup<D, GP, MH, true, ROT>(blockIdx.x, dq, dout, k_cache, v_cache, context_lens,
                                           d_tables, d_stride, d_batch, Hq, Hkv, G, n_hg,
                                           bs_log2, scale_log2, num_workers, ws_prefix, ws_ml,
                                           ws_o, cos_sin, max_position);
  else
    prefill_workgroup<D, PGP, true, ROT>(blockIdx.x - n_decode_wg, pq, pout, k_cache, v_cache,
                                        cu_q, cu_k, p_tables, p_stride, Hq, Hkv, G, bs_log2,
                                        scale_log2, p_batch, max_tiles, cos_sin, max_position);
}

hipError_t launch_mixed_attention_bf16(
    int head_dim, const void* k_cache, const void* v_cache, int num_q_heads, int num_kv_heads,
    int bs_log2, float scale, const void* q_prefill, void* out_prefill, int prefill_batch,
    int max_seqlen_q, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int32_t* prefill_tables, int prefill_stride, const void* q_decode, void* out_decode,
    int decode_batch, const int32_t* context_lens, const int32_t* decode_tables,
    int decode_stride, int num_workers, void* workspace, const float* cos_sin,
    int max_position, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int GP = heads_per_stream(G);
  const int PGP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;  // as the prefill kernel rounds
  const int MH = kv_heads_per_stream(head_dim, num_kv_heads, G);
  // the shapes built here: both passes take their whole-block paths and one grouping
  if (G > 8 || bs_log2 < 6 || (1 << bs_log2) < chunk_tokens(head_dim, MH) || prefill_batch <= 0 ||
      decode_batch <= 0 || max_seqlen_q <= 0)
    return hipErrorNotSupported;
  const int n_hg = (G + GP - 1) / GP;
  if ((num_kv_heads / MH) * n_hg > 65535) return hipErrorInvalidConfiguration;
  const int W = num_workers > 0 ? num_workers
                                : paged_decode_bf16_workers(head_dim, num_q_heads, num_kv_heads,
                                                            bs_log2);
  const DecodeWorkspace ws = carve_decode_workspace(workspace, decode_batch, W, MH * GP);
  // a multiple of 8 (the surplus workgroups have no worker and leave at once), so the
  // prefill's item w sits on the XCD that w mod 8 names
  const int n_decode_wg = ((W + 3) / 4 + kXcds - 1) / kXcds * kXcds;
  const int bm_tok = 128 / PGP;
  const int max_tiles = (max_seqlen_q + bm_tok - 1) / bm_tok;
  const int64_t slots = static_cast<int64_t>(prefill_batch) * num_kv_heads * max_tiles;
  if (slots + n_decode_wg > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(slots + n_decode_wg));
  const float scale_log2 = scale * kLog2e;
#define PKV_MIXED(D_, GP_, PGP_, MH_, ROT_)                                                    \
  hipExtLaunchKernelGGL((mixed_attention_bf16_kernel<D_, GP_, PGP_, MH_, ROT_>), grid,         \
                        dim3(256), 0, stream, timing_start(), timing_stop(), 0,                \
                        static_cast<const uint16_t*>(k_cache),                                 \
                        static_cast<const uint16_t*>(v_cache), num_q_heads, num_kv_heads, G,   \
                        bs_log2, scale_log2, cos_sin, max_position, n_decode_wg,               \
                        static_cast<const uint16_t*>(q_decode),                                \
                        static_cast<uint16_t*>(out_decode), context_lens, decode_tables,       \
                        decode_stride, decode_batch, n_hg, W, ws.prefix, ws.ml, ws.o,          \
                        static_cast<const uint16_t*>(q_prefill),                               \
                        static_cast<uint16_t*>(out_prefill), cu_seqlens_q, cu_seqlens_k,       \
                        prefill_tables, prefill_stride, prefill_batch, max_tiles)
#define PKV_MIXED_R(D_, GP_, PGP_, MH_)                   \
  if (cos_sin != nullptr) PKV_MIXED(D_, GP_, PGP_, MH_, true); \
  else PKV_MIXED(D_, GP_, PGP_, MH_, false);
  // (GP, PGP) pairs: G = 1 -> (1, 1), 2 -> (2, 2), 3 -> (2, 4), 4 -> (4, 4),
  // 5..7 -> (4, 8), 8 -> (8, 8)
#define PKV_MIXED_GP(D_, MH_)                                        \
  if (GP == 1) { PKV_MIXED_R(D_, 1, 1, MH_) }                        \
  else if (GP == 2 && PGP == 2) { PKV_MIXED_R(D_, 2, 2, MH_) }       \
  else if (GP == 2) { PKV_MIXED_R(D_, 2, 4, MH_) }                   \
  else if (GP == 4 && PGP == 4) { PKV_MIXED_R(D_, 4, 4, MH_) }       \
  else if (GP == 4) { PKV_MIXED_R(D_, 4, 8, MH_) }                   \
  else { PKV_MIXED_R(D_, 8, 8, MH_) }
  timing_begin("mixed_attention", stream);
  if (head_dim == 128) {
    switch (MH) {
      case 1: PKV_MIXED_GP(128, 1) break;
      case 2: PKV_MIXED_GP(128, 2) break;
      default: PKV_MIXED_GP(128, 4) break;
    }
  } else {
    switch (MH) {
      case 1: PKV_MIXED_GP(64, 1) break;
      case 2: PKV_MIXED_GP(64, 2) break;
      case 4: PKV_MIXED_GP(64, 4) break;
      default: PKV_MIXED_GP(64, 8) break;
    }
  }
  timing_end(stream);
#undef PKV_MIXED_GP
#undef PKV_MIXED_R
#undef PKV_MIXED
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(head_dim, GP, MH, ws, out_decode, context_lens, decode_batch,
                               num_q_heads, num_kv_heads, W, stream);
}

}  // namespace pkv
