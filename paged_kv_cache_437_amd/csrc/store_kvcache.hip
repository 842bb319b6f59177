// KV write through a slot mapping (“深入 Nano-vLLM 推理引擎”, "Control plane
// vs. data plane": the data plane only copies rows into the slots the control plane
// chose; a reused block is overwritten, never cleared first).
//
// One workgroup per token; its K and V rows (Hkv * D elements each, a multiple of 16
// bytes) are copied with 16-byte loads and stores.  The copy is bit-exact: rows move
// as raw bytes whatever the element type.  Slot -1 is a padding row and writes nothing.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

__global__ __launch_bounds__(256) void store_kvcache_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, const uint4* __restrict__ k,
    const uint4* __restrict__ v, const int32_t* __restrict__ slot_mapping, int chunks_per_row) {
  const int t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t src = static_cast<int64_t>(t) * chunks_per_row;
  const int64_t dst = static_cast<int64_t>(slot) * chunks_per_row;
  for (int c = threadIdx.x; c < chunks_per_row; c += blockDim.x) {
    const uint4 kk = k[src + c];
    const uint4 vv = v[src + c];
    k_cache[dst + c] = kk;
    v_cache[dst + c] = vv;
  }
}

hipError_t launch_store_kvcache(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                int32_t row_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int chunks = row_bytes / 16;
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  timing_begin("store_kvcache", stream);
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache),
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping,
                     chunks);
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace pkv
