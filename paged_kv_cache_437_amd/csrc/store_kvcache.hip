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

// The same write with K rotated at its token's position (rotary position embedding,
// half-split pairing; see pkv_store_kvcache_rotary).  Thread w of the token's
// workgroup takes 16 bytes of one head's first half-row, element i0 on, with their
// partners at i0 + D/2, and the cosines / sines of row `position` of the table; V rows
// are copied bit for bit.  Positions outside the table read its nearest row.
template <typename T, int D>
__global__ __launch_bounds__(256) void store_kvcache_rotary_kernel(
    T* __restrict__ k_cache, uint4* __restrict__ v_cache, const T* __restrict__ k,
    const uint4* __restrict__ v, const int32_t* __restrict__ slot_mapping,
    const int32_t* __restrict__ positions, const float* __restrict__ cos_sin, int max_position,
    int Hkv) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16 bytes
  constexpr int HC = D / 2 / EPC;      // 16-byte pieces per half row
  const int t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int pos = min(max(positions[t], 0), max_position - 1);
  const float* cs = cos_sin + static_cast<int64_t>(pos) * D;
  const int64_t src = static_cast<int64_t>(t) * Hkv * D;
  const int64_t dst = static_cast<int64_t>(slot) * Hkv * D;
  for (int w = threadIdx.x; w < Hkv * HC; w += blockDim.x) {
    const int hh = w / HC;
    const int i0 = (w - hh * HC) * EPC;
    const T* kr = k + src + hh * D + i0;
    T* kw = k_cache + dst + hh * D + i0;
    float c[EPC], s[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      c[e] = cs[i0 + e];
      s[e] = cs[D / 2 + i0 + e];
    }
    if constexpr (sizeof(T) == 2) {
      uint4 xv = *reinterpret_cast<const uint4*>(kr);
      uint4 yv = *reinterpret_cast<const uint4*>(kr + D / 2);
      uint32_t x[4] = {xv.x, xv.y, xv.z, xv.w}, y[4] = {yv.x, yv.y, yv.z, yv.w};
      rope8_bf16(x, y, c, s);
      *reinterpret_cast<uint4*>(kw) = make_uint4(x[0], x[1], x[2], x[3]);
      *reinterpret_cast<uint4*>(kw + D / 2) = make_uint4(y[0], y[1], y[2], y[3]);
    } else {
      const float4 x = *reinterpret_cast<const float4*>(kr);
      const float4 y = *reinterpret_cast<const float4*>(kr + D / 2);
      *reinterpret_cast<float4*>(kw) = make_float4(x.x * c[0] - y.x * s[0], x.y * c[1] - y.y * s[1],
                                                   x.z * c[2] - y.z * s[2], x.w * c[3] - y.w * s[3]);
      *reinterpret_cast<float4*>(kw + D / 2) =
          make_float4(y.x * c[0] + x.x * s[0], y.y * c[1] + x.y * s[1], y.z * c[2] + x.z * s[2],
                      y.w * c[3] + x.w * s[3]);
    }
  }
  const int chunks = Hkv * D * static_cast<int>(sizeof(T)) / 16;
  const int64_t src16 = static_cast<int64_t>(t) * chunks;
  const int64_t dst16 = static_cast<int64_t>(slot) * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) v_cache[dst16 + c] = v[src16 + c];
}

hipError_t launch_store_kvcache_rotary(bool bf16, int head_dim, void* k_cache, void* v_cache,
                                       const void* k, const void* v,
                                       const int32_t* slot_mapping, const int32_t* positions,
                                       int32_t num_tokens, int num_kv_heads,
                                       const float* cos_sin, int max_position,
                                       hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int row_chunks = num_kv_heads * head_dim * (bf16 ? 2 : 4) / 16;
  const int threads = row_chunks >= 256 ? 256 : ((row_chunks + 63) / 64) * 64;
  timing_begin("store_kvcache_rotary", stream);
#define PKV_STORE_ROT(T, D)                                                                    \
  hipExtLaunchKernelGGL((store_kvcache_rotary_kernel<T, D>), dim3(num_tokens), dim3(threads),  \
                        0, stream, timing_start(), timing_stop(), 0, static_cast<T*>(k_cache), \
                        static_cast<uint4*>(v_cache), static_cast<const T*>(k),                \
                        static_cast<const uint4*>(v), slot_mapping, positions, cos_sin,        \
                        max_position, num_kv_heads)
  if (bf16) {
    if (head_dim == 64) PKV_STORE_ROT(uint16_t, 64); else PKV_STORE_ROT(uint16_t, 128);
  } else {
    if (head_dim == 64) PKV_STORE_ROT(float, 64); else PKV_STORE_ROT(float, 128);
  }
#undef PKV_STORE_ROT
  timing_end(stream);
  return hipGetLastError();
}

hipError_t launch_store_kvcache(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                int32_t row_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int chunks = row_bytes / 16;
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  timing_begin("store_kvcache", stream);
  hipExtLaunchKernelGGL(store_kvcache_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                        timing_start(), timing_stop(), 0, static_cast<uint4*>(k_cache),
                        static_cast<uint4*>(v_cache), static_cast<const uint4*>(k),
                        static_cast<const uint4*>(v), slot_mapping, chunks);
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace pkv
