// Paged varlen causal prefill, bf16 in / fp32 accumulate, on gfx950 MFMA: the kernel
// and its launchers.  The pass itself (what is computed, tiling, the LDS layout and
// the work order) is in prefill_kernel.h.
#include "prefill_kernel.h"

namespace pkv {

template <int D, int GP, bool BIG_BLOCK, bool ROT>
__global__ __launch_bounds__(256, 2) void paged_prefill_bf16_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ cu_seqlens_k,
    const int32_t* __restrict__ block_tables, int table_stride, int Hq, int Hkv, int G,
    int bs_log2, float scale_log2, int batch, int max_tiles, const float* __restrict__ cos_sin,
    int max_position) {
  prefill_workgroup<D, GP, BIG_BLOCK, ROT>(blockIdx.x, q, out, k_cache, v_cache, cu_seqlens_q,
                                           cu_seqlens_k, block_tables, table_stride, Hq, Hkv,
                                           G, bs_log2, scale_log2, batch, max_tiles, cos_sin,
                                           max_position);
}

template <int D, int GP>
static void launch_prefill(dim3 grid, hipStream_t stream, const void* q, void* out,
                           const void* kc, const void* vc, const int32_t* cu_q,
                           const int32_t* cu_k, const int32_t* tables, int stride, int Hq,
                           int Hkv, int G, int bs_log2, float scale_log2, int batch,
                           int max_tiles, const float* cos_sin, int max_position) {
  // blocks of at least 64 tokens hold a whole 64-key tile
  auto kernel = cos_sin != nullptr
                    ? (bs_log2 >= 6 ? paged_prefill_bf16_kernel<D, GP, true, true>
                                    : paged_prefill_bf16_kernel<D, GP, false, true>)
                    : (bs_log2 >= 6 ? paged_prefill_bf16_kernel<D, GP, true, false>
                                    : paged_prefill_bf16_kernel<D, GP, false, false>);
  hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, timing_start(), timing_stop(), 0,
                        static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                        static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), cu_q,
                        cu_k, tables, stride, Hq, Hkv, G, bs_log2, scale_log2, batch, max_tiles,
                        cos_sin, max_position);
}

hipError_t launch_paged_prefill_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                     const void* v_cache, int num_q_heads, int num_kv_heads,
                                     int bs_log2, int batch, int max_seqlen_q,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     const int32_t* block_tables, int table_stride, float scale,
                                     const float* cos_sin, int max_position, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  if (G > 128) return hipErrorInvalidConfiguration;
  const int GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : G <= 16 ? 16 : G <= 32
                 ? 32 : G <= 64 ? 64 : 128;
  const int bm_tok = 128 / GP;
  const int max_tiles = (max_seqlen_q + bm_tok - 1) / bm_tok;
  // one workgroup per (sequence, kv head, q tile) at most; the real items come first
  const int64_t slots = static_cast<int64_t>(batch) * num_kv_heads * max_tiles;
  if (slots > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(slots));
  const float scale_log2 = scale * kLog2e;
#define PKV_PF(D_, GP_)                                                                       \
  launch_prefill<D_, GP_>(grid, stream, q, out, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, \
                          block_tables, table_stride, num_q_heads, num_kv_heads, G, bs_log2,  \
                          scale_log2, batch, max_tiles, cos_sin, max_position)
#define PKV_PF_GP(D_)                                  \
  switch (GP) {                                        \
    case 1: PKV_PF(D_, 1); break;                      \
    case 2: PKV_PF(D_, 2); break;                      \
    case 4: PKV_PF(D_, 4); break;                      \
    case 8: PKV_PF(D_, 8); break;                      \
    case 16: PKV_PF(D_, 16); break;                    \
    case 32: PKV_PF(D_, 32); break;                    \
    case 64: PKV_PF(D_, 64); break;                    \
    default: PKV_PF(D_, 128); break;                   \
  }
  timing_begin("paged_prefill_mfma", stream);
  if (head_dim == 128) {
    PKV_PF_GP(128)
  } else {
    PKV_PF_GP(64)
  }
  timing_end(stream);
#undef PKV_PF_GP
#undef PKV_PF
  return hipGetLastError();
}

}  // namespace pkv
