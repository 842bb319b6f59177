// Paged decode attention, bf16 in / fp32 accumulate, for gfx950: the kernel and its
// launchers.  The pass itself (what is computed, the work division, the loads) is in
// decode_kernel.h.
#include "decode_kernel.h"

namespace pkv {

// (at least two waves per SIMD: the eight-head groups would otherwise take a few
// registers past 256 and run one wave per SIMD)
template <int D, int GP, int MH, bool ONE_BLOCK, bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
paged_decode_bf16_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, int batch, int Hq, int Hkv, int G, int n_hg, int bs_log2,
    float scale_log2, int num_workers, int64_t* __restrict__ ws_prefix,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o, const float* __restrict__ cos_sin,
    int max_position) {
  decode_workgroup<D, GP, MH, ONE_BLOCK, ROT>(
      blockIdx.x, q, out, k_cache, v_cache, context_lens, block_tables, table_stride, batch, Hq,
      Hkv, G, n_hg, bs_log2, scale_log2, num_workers, ws_prefix, ws_ml, ws_o, cos_sin,
      max_position);
}

// The same pass appending the step's new token of each sequence itself (chunks in one
// block, no rotary): the cache rows of the new tokens are written by the kernel, and the
// token's K and V enter the attention from k_new / v_new.
template <int D, int GP, int MH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
paged_decode_append_bf16_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, int batch, int Hq, int Hkv, int G, int n_hg, int bs_log2,
    float scale_log2, int num_workers, int64_t* __restrict__ ws_prefix,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o, DecodeAppend app) {
  decode_workgroup<D, GP, MH, true, false, true>(
      blockIdx.x, q, out, k_cache, v_cache, context_lens, block_tables, table_stride, batch, Hq,
      Hkv, G, n_hg, bs_log2, scale_log2, num_workers, ws_prefix, ws_ml, ws_o, nullptr, 0, app);
}

namespace {

template <int D, int GP, int MH>
hipError_t launch_decode_append(const void* q, void* out, const void* k_cache,
                                const void* v_cache, int num_q_heads, int num_kv_heads,
                                int bs_log2, int batch, const int32_t* context_lens,
                                const int32_t* block_tables, int table_stride, float scale,
                                int num_workers, void* workspace, const DecodeAppend& app,
                                hipStream_t stream) {
  if ((1 << bs_log2) < chunk_tokens(D, MH)) return hipErrorNotSupported;
  const int G = num_q_heads / num_kv_heads;
  const int n_hg = (G + GP - 1) / GP;
  const int S = (num_kv_heads / MH) * n_hg;
  if (S > 65535) return hipErrorInvalidConfiguration;
  const int W = num_workers > 0 ? num_workers : auto_decode_workers(GP);
  const DecodeWorkspace ws = carve_decode_workspace(workspace, batch, W, MH * GP);
  const float scale_log2 = scale * kLog2e;
  timing_begin("paged_decode_append", stream);
  hipExtLaunchKernelGGL((paged_decode_append_bf16_kernel<D, GP, MH>), dim3((W + 3) / 4), dim3(256),
                        0, stream, timing_start(), timing_stop(), 0,
                        static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                        static_cast<const uint16_t*>(k_cache),
                        static_cast<const uint16_t*>(v_cache), context_lens, block_tables,
                        table_stride, batch, num_q_heads, num_kv_heads, G, n_hg, bs_log2,
                        scale_log2, W, ws.prefix, ws.ml, ws.o, app);
  timing_end(stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(D, GP, MH, ws, out, context_lens, batch, num_q_heads,
                               num_kv_heads, W, stream);
}

template <int D, int GP, int MH, bool ONE_BLOCK>
hipError_t launch_decode(const void* q, void* out, const void* k_cache, const void* v_cache,
                         int num_q_heads, int num_kv_heads, int bs_log2, int batch,
                         const int32_t* context_lens, const int32_t* block_tables,
                         int table_stride, float scale, int num_workers, void* workspace,
                         const float* cos_sin, int max_position, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int n_hg = (G + GP - 1) / GP;
  const int S = (num_kv_heads / MH) * n_hg;
  if (S > 65535) return hipErrorInvalidConfiguration;
  const int W = num_workers > 0 ? num_workers : auto_decode_workers(GP);
  const DecodeWorkspace ws = carve_decode_workspace(workspace, batch, W, MH * GP);
  const float scale_log2 = scale * kLog2e;
  timing_begin("paged_decode", stream);
  auto kernel = cos_sin != nullptr ? paged_decode_bf16_kernel<D, GP, MH, ONE_BLOCK, true>
                                   : paged_decode_bf16_kernel<D, GP, MH, ONE_BLOCK, false>;
  hipExtLaunchKernelGGL(kernel, dim3((W + 3) / 4), dim3(256), 0, stream, timing_start(),
                        timing_stop(), 0, static_cast<const uint16_t*>(q),
                        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(k_cache),
                        static_cast<const uint16_t*>(v_cache), context_lens, block_tables,
                        table_stride, batch, num_q_heads, num_kv_heads, G, n_hg, bs_log2,
                        scale_log2, W, ws.prefix, ws.ml, ws.o, cos_sin, max_position);
  timing_end(stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(D, GP, MH, ws, out, context_lens, batch, num_q_heads,
                               num_kv_heads, W, stream);
}

template <int D, int GP, int MH>
hipError_t launch_decode_bs(const void* q, void* out, const void* k_cache, const void* v_cache,
                            int num_q_heads, int num_kv_heads, int bs_log2, int batch,
                            const int32_t* context_lens, const int32_t* block_tables,
                            int table_stride, float scale, int num_workers, void* workspace,
                            const float* cos_sin, int max_position, hipStream_t stream) {
  // ONE_BLOCK: every chunk lies in one block (block_size >= the chunk)
  if ((1 << bs_log2) >= chunk_tokens(D, MH))
    return launch_decode<D, GP, MH, true>(q, out, k_cache, v_cache, num_q_heads, num_kv_heads,
                                          bs_log2, batch, context_lens, block_tables,
                                          table_stride, scale, num_workers, workspace, cos_sin,
                                          max_position, stream);
  return launch_decode<D, GP, MH, false>(q, out, k_cache, v_cache, num_q_heads, num_kv_heads,
                                         bs_log2, batch, context_lens, block_tables,
                                         table_stride, scale, num_workers, workspace, cos_sin,
                                         max_position, stream);
}

template <int D, int MH>
hipError_t launch_decode_gp(int GP, const void* q, void* out, const void* k_cache,
                            const void* v_cache, int num_q_heads, int num_kv_heads, int bs_log2,
                            int batch, const int32_t* context_lens, const int32_t* block_tables,
                            int table_stride, float scale, int num_workers, void* workspace,
                            const float* cos_sin, int max_position, hipStream_t stream) {
#define PKV_DEC(GP_)                                                                         \
  return launch_decode_bs<D, GP_, MH>(q, out, k_cache, v_cache, num_q_heads, num_kv_heads, \
                                      bs_log2, batch, context_lens, block_tables,          \
                                      table_stride, scale, num_workers, workspace, cos_sin, \
                                      max_position, stream)
  switch (GP) {
    case 1: PKV_DEC(1);
    case 2: PKV_DEC(2);
    case 4: PKV_DEC(4);
    default: PKV_DEC(8);
  }
#undef PKV_DEC
}

}  // namespace

int paged_decode_bf16_workers(int head_dim, int num_q_heads, int num_kv_heads, int bs_log2) {
  (void)head_dim;
  (void)num_kv_heads;
  (void)bs_log2;
  return auto_decode_workers(heads_per_stream(num_q_heads / num_kv_heads));
}

size_t paged_decode_bf16_workspace(int head_dim, int num_q_heads, int num_kv_heads, int batch,
                                   int num_workers) {
  const int GP = heads_per_stream(num_q_heads / num_kv_heads);
  const int MH = kv_heads_per_stream(head_dim, num_kv_heads, num_q_heads / num_kv_heads);
  return decode_workspace_bytes(batch, num_workers > 0 ? num_workers : auto_decode_workers(GP),
                                MH * GP, head_dim);
}

hipError_t launch_paged_decode_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                    const void* v_cache, int num_q_heads, int num_kv_heads,
                                    int bs_log2, int batch, const int32_t* context_lens,
                                    const int32_t* block_tables, int table_stride, float scale,
                                    int num_workers, void* workspace, const float* cos_sin,
                                    int max_position, hipStream_t stream) {
  const int GP = heads_per_stream(num_q_heads / num_kv_heads);
  const int MH = kv_heads_per_stream(head_dim, num_kv_heads, num_q_heads / num_kv_heads);
#define PKV_DEC(D_, MH_)                                                                      \
  return launch_decode_gp<D_, MH_>(GP, q, out, k_cache, v_cache, num_q_heads, num_kv_heads, \
                                   bs_log2, batch, context_lens, block_tables, table_stride, \
                                   scale, num_workers, workspace, cos_sin, max_position,     \
                                   stream)
  if (head_dim == 128) {
    switch (MH) {
      case 1: PKV_DEC(128, 1);
      case 2: PKV_DEC(128, 2);
      default: PKV_DEC(128, 4);
    }
  }
  switch (MH) {
    case 1: PKV_DEC(64, 1);
    case 2: PKV_DEC(64, 2);
    case 4: PKV_DEC(64, 4);
    default: PKV_DEC(64, 8);
  }
#undef PKV_DEC
}

hipError_t launch_paged_decode_append_bf16(int head_dim, const void* q, void* out,
                                           const void* k_cache, const void* v_cache,
                                           int num_q_heads, int num_kv_heads, int bs_log2,
                                           int batch, const int32_t* context_lens,
                                           const int32_t* block_tables, int table_stride,
                                           float scale, int num_workers, void* workspace,
                                           const void* k_new, const void* v_new,
                                           const int32_t* slot_mapping, hipStream_t stream) {
  // one q head per kv head only: with grouped heads the appending kernel measured slower
  // than the KV write and the plain decode together
  if (num_q_heads != num_kv_heads) return hipErrorNotSupported;
  const int MH = kv_heads_per_stream(head_dim, num_kv_heads, 1);
  DecodeAppend app;
  app.k_new = static_cast<const uint16_t*>(k_new);
  app.v_new = static_cast<const uint16_t*>(v_new);
  app.slots = slot_mapping;
#define PKV_DEC(D_, MH_)                                                                      \
  return launch_decode_append<D_, 1, MH_>(q, out, k_cache, v_cache, num_q_heads, num_kv_heads, \
                                          bs_log2, batch, context_lens, block_tables,          \
                                          table_stride, scale, num_workers, workspace, app,    \
                                          stream)
  // with one q head per kv head a stream holds at most 512 bytes of kv-head rows
  if (head_dim == 128) {
    if (MH == 1) PKV_DEC(128, 1);
    PKV_DEC(128, 2);
  }
  switch (MH) {
    case 1: PKV_DEC(64, 1);
    case 2: PKV_DEC(64, 2);
    default: PKV_DEC(64, 4);
  }
#undef PKV_DEC
}

}  // namespace pkv
