// Generic paged attention on the vector ALU: one wavefront per (query row, q head).
//
// What it computes is the plain definition (“深入 Nano-vLLM 推理引擎”,
// "Prefill and Decode" and "Preparing for computation"): for sequence b, query i of
// its Lq new tokens sits at position Lk - Lq + i and attends, with a softmax of
// scale * q.k, to keys 0 .. Lk - Lq + i read through the block table.  Decode is the
// one-query case over context_lens[b] keys.
//
// Lanes own keys for the scores (64 keys per step, online softmax across steps, after
// Milakov & Gimelshein's online normaliser) and own head_dim elements for the
// P.V accumulation.  Every K/V load is guarded by the key's validity, so table
// entries past the sequence's last block and stale rows are never read.  fp32
// accumulation throughout, one rounding of the output.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

template <typename T, int D>
__global__ __launch_bounds__(256) void attention_generic_kernel(
    const T* __restrict__ q, T* __restrict__ out, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, int Hq, int Hkv, int bs_log2,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ cu_seqlens_k,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, float scale_log2, const float* __restrict__ cos_sin, int max_position) {
  constexpr int E = D / 64;  // head_dim elements per lane in the P.V phase
  __shared__ float q_lds[4][D];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  const int h = blockIdx.z;

  int q_begin, Lq, Lk;
  if (context_lens != nullptr) {
    q_begin = b;
    Lq = 1;
    Lk = context_lens[b];
  } else {
    q_begin = cu_seqlens_q[b];
    Lq = cu_seqlens_q[b + 1] - q_begin;
    Lk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
  }
  const int i = blockIdx.x * 4 + wave;
  if (i >= Lq) return;  // the whole wave leaves; no workgroup barrier follows
  const int last_key = Lk - Lq + i;
  const int kvh = h / (Hq / Hkv);
  const int32_t* table = block_tables + static_cast<int64_t>(b) * table_stride;

  const T* q_row = q + (static_cast<int64_t>(q_begin + i) * Hq + h) * D;
#pragma unroll
  for (int e = 0; e < E; ++e) q_lds[wave][lane * E + e] = Elem<T>::load(q_row + lane * E + e);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (cos_sin != nullptr) {
    // rotary position embedding of the query at its position (half-split pairs: lane j
    // rotates elements j and j + D/2), in fp32
    const float* cs = cos_sin + static_cast<int64_t>(min(max(last_key, 0), max_position - 1)) * D;
    float x = 0.f, y = 0.f;
    if (lane < D / 2) {
      x = q_lds[wave][lane];
      y = q_lds[wave][lane + D / 2];
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < D / 2) {
      const float c = cs[lane], sn = cs[D / 2 + lane];
      q_lds[wave][lane] = x * c - y * sn;
      q_lds[wave][lane + D / 2] = y * c + x * sn;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  float m = -INFINITY;  // running max of the log2-domain scores
  float l = 0.f;        // running sum of exp2(score - m)
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;

  for (int j0 = 0; j0 <= last_key; j0 += 64) {
    const int j = j0 + lane;
    const bool valid = j <= last_key;
    int64_t row = 0;
    float s = -INFINITY;
    if (valid) {
      row = token_row(table[j >> bs_log2], j, bs_log2, Hkv, kvh, D);
      const T* kr = k_cache + row;
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) acc += q_lds[wave][d] * Elem<T>::load(kr + d);
      s = acc * scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(s));  // finite: key j0 is always valid
    const float p = valid ? exp2f(s - m_new) : 0.f;
    const float alpha = exp2f(m - m_new);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
    const int n_valid = min(64, last_key - j0 + 1);
    for (int t = 0; t < n_valid; ++t) {
      const float pt = __shfl(p, t, 64);
      const int64_t rt = __shfl(row, t, 64);
      const T* vr = v_cache + rt + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += pt * Elem<T>::load(vr + e);
    }
    m = m_new;
  }

  T* o_row = out + (static_cast<int64_t>(q_begin + i) * Hq + h) * D + lane * E;
  const float inv_l = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) Elem<T>::store(o_row + e, o[e] * inv_l);
}

template <typename T, int D>
static void launch_one(const void* q, void* out, const void* kc, const void* vc, int Hq, int Hkv,
                       int bs_log2, int batch, int max_q_rows, const int32_t* cu_q,
                       const int32_t* cu_k, const int32_t* ctx, const int32_t* tables,
                       int stride, float scale_log2, const float* cos_sin, int max_position,
                       hipStream_t stream) {
  dim3 grid((max_q_rows + 3) / 4, batch, Hq);
  timing_begin(ctx != nullptr ? "attention_generic_decode" : "attention_generic_prefill", stream);
  hipExtLaunchKernelGGL((attention_generic_kernel<T, D>), grid, dim3(256), 0, stream,
                        timing_start(), timing_stop(), 0, static_cast<const T*>(q),
                        static_cast<T*>(out), static_cast<const T*>(kc), static_cast<const T*>(vc),
                        Hq, Hkv, bs_log2, cu_q, cu_k, ctx, tables, stride, scale_log2, cos_sin,
                        max_position);
  timing_end(stream);
}

hipError_t launch_attention_generic(bool bf16, int head_dim, const void* q, void* out,
                                    const void* k_cache, const void* v_cache, int num_q_heads,
                                    int num_kv_heads, int bs_log2, int batch, int max_q_rows,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int table_stride, float scale, const float* cos_sin,
                                    int max_position, hipStream_t stream) {
  if (batch == 0 || max_q_rows == 0) return hipSuccess;
  const float scale_log2 = scale * kLog2e;
#define PKV_GENERIC(T, D)                                                                      \
  launch_one<T, D>(q, out, k_cache, v_cache, num_q_heads, num_kv_heads, bs_log2, batch,        \
                   max_q_rows, cu_seqlens_q, cu_seqlens_k, context_lens, block_tables,         \
                   table_stride, scale_log2, cos_sin, max_position, stream)
  if (bf16) {
    if (head_dim == 64) PKV_GENERIC(uint16_t, 64); else PKV_GENERIC(uint16_t, 128);
  } else {
    if (head_dim == 64) PKV_GENERIC(float, 64); else PKV_GENERIC(float, 128);
  }
#undef PKV_GENERIC
  return hipGetLastError();
}

}  // namespace pkv
