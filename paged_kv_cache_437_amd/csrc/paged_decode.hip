// Paged decode attention, bf16 in / fp32 accumulate, for gfx950.
//
// What is computed (“深入 Nano-vLLM 推理引擎”, "Prefill and Decode": each
// decode step adds one token per sequence; "From Sequences to Blocks": a sequence's
// tokens live in the blocks its table lists): for sequence b and q head h,
//   out[b, h] = softmax_j(scale * q[b, h] . k_j) v_j   over j < context_lens[b],
// with k_j, v_j the rows of kv head h / (Hq / Hkv) found through block_tables[b].
//
// Work decomposition.  The context is cut into splits of `split_tokens` tokens (a
// multiple of 256 and hence of every supported block size), so the cut depends only
// on lengths.  One workgroup of 4 wavefronts handles (split, kv head, group of up to
// 8 q heads, sequence); it walks its split 256 tokens at a time, wave w taking tokens
// 64w .. 64w+63 of each 256.  Per wave and 64 tokens:
//   * K rows go straight from HBM into the B operand of v_mfma_f32_16x16x32_bf16
//     (lane: token lane%16, 8 head_dim elements), the A operand holding the group's
//     q rows (padded to 16), so the 16x16 score tiles cost four MFMAs per 16 tokens;
//     every q head of the group reuses each K row loaded.
//   * Online softmax in the log2 domain (scale * log2 e folded into one multiply):
//     row max across the 16 lanes of a tile row, exp2, per-lane partial sums.
//   * Probabilities go through a per-wave LDS tile to the P.V phase, where lanes own
//     (token, 8 head_dim elements) of V rows loaded with 16-byte loads and accumulate
//     on the vector ALU.
// All K/V loads are predicated on token < context_len, so neither table entries past
// the last used block nor the stale tail of the last block is ever read.
// The four waves' (max, sum, unnormalised out) merge exactly in LDS; a sequence with
// one split writes its output directly, otherwise the partial goes to the workspace
// and decode_combine merges the splits:  M = max_s m_s,
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  rounded once to bf16.
// No atomics: results are bit-identical across runs and block relabellings.
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1, 64));
  x = fmaxf(x, __shfl_xor(x, 2, 64));
  x = fmaxf(x, __shfl_xor(x, 4, 64));
  x = fmaxf(x, __shfl_xor(x, 8, 64));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
__device__ __forceinline__ float read_lane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int D, int GP>
__global__ __launch_bounds__(256, 2) void paged_decode_bf16_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, int Hq, int Hkv, int G, int n_hg, int bs_log2, int split_tokens,
    int max_splits, float scale_log2, float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(GP == 1 || GP == 2 || GP == 4 || GP == 8, "heads per workgroup");
  constexpr int KK = D / 32;     // MFMA k-steps over head_dim
  constexpr int DCH = D / 8;     // 16-byte chunks per row
  constexpr int TPI = 64 / DCH;  // tokens per V load instruction of a wave
  constexpr int VIT = 64 / TPI;  // V load instructions per wave per 64 tokens

  __shared__ __attribute__((aligned(16))) float p_lds[4][64][16];
  __shared__ __attribute__((aligned(16))) float o_lds[4][GP][D];
  __shared__ float m_lds[4][16];
  __shared__ float l_lds[4][16];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / n_hg;
  const int hg = blockIdx.y - kvh * n_hg;
  const int b = blockIdx.z;
  const int L = context_lens[b];
  const int n_splits = (L + split_tokens - 1) / split_tokens;
  if (split >= n_splits) return;  // uniform over the workgroup, before any barrier

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int row = lane & 15;  // MFMA: token column (B) / head row (A)
  const int grp = lane >> 4;  // MFMA: which 8-element slice of each 32-wide k-step
  const int h0 = kvh * G + hg * GP;
  const int nh = min(GP, G - hg * GP);
  const int32_t* table = block_tables + static_cast<int64_t>(b) * table_stride;
  const int bs_mask = (1 << bs_log2) - 1;

  // q rows of the group as the MFMA A operand; rows >= nh are zero
  bf16x8_t qa[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (row < nh)
      w = *reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(b) * Hq + h0 + row) * D +
                                            kk * 32 + grp * 8);
    qa[kk] = __builtin_bit_cast(bf16x8_t, w);
  }

  float m_r[4], l_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_r[r] = -INFINITY;
    l_r[r] = 0.f;
  }
  float o[GP][8];
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

  const int v_chunk = lane % DCH;
  const int v_sub = lane / DCH;
  const int split_end = min(L, (split + 1) * split_tokens);

  for (int c0 = split * split_tokens; c0 < split_end; c0 += 256) {
    const int base = c0 + 64 * wave;  // first token of this wave's 64
    if (base >= L) continue;          // nothing valid for this wave (no barrier inside)

    // ---- issue every K and V load of the 64 tokens
    u32x4_t kb[4][KK];
    u32x4_t vb[VIT];
    if (bs_log2 >= 6) {
      // a 64-aligned run of 64 tokens lies in one block: one table entry per wave
      const int64_t blk = table[base >> bs_log2];
      const int64_t first = ((blk << bs_log2) | (base & bs_mask)) * Hkv + kvh;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int tok = base + 16 * t4 + row;
        const int64_t off = (first + static_cast<int64_t>(16 * t4 + row) * Hkv) * D + grp * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          u32x4_t w = {0u, 0u, 0u, 0u};
          if (tok < L) w = *reinterpret_cast<const u32x4_t*>(k_cache + off + kk * 32);
          kb[t4][kk] = w;
        }
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int tl = it * TPI + v_sub;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (base + tl < L)
          w = *reinterpret_cast<const u32x4_t*>(
              v_cache + (first + static_cast<int64_t>(tl) * Hkv) * D + v_chunk * 8);
        vb[it] = w;
      }
    } else {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int tok = base + 16 * t4 + row;
        int64_t off = 0;
        if (tok < L) off = token_row(table[tok >> bs_log2], tok, bs_log2, Hkv, kvh, D) + grp * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          u32x4_t w = {0u, 0u, 0u, 0u};
          if (tok < L) w = *reinterpret_cast<const u32x4_t*>(k_cache + off + kk * 32);
          kb[t4][kk] = w;
        }
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int tok = base + it * TPI + v_sub;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (tok < L)
          w = *reinterpret_cast<const u32x4_t*>(
              v_cache + token_row(table[tok >> bs_log2], tok, bs_log2, Hkv, kvh, D) +
              v_chunk * 8);
        vb[it] = w;
      }
    }

    // ---- scores: S[head 4*grp + r][token 16*t4 + row] in acc[t4][r]
    f32x4_t acc[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      acc[t4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc[t4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qa[kk], __builtin_bit_cast(bf16x8_t, kb[t4][kk]), acc[t4], 0, 0, 0);
    }

    // ---- online softmax (log2 domain), per head row
    float alpha_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const float s = (base + 16 * t4 + row < L) ? acc[t4][r] * scale_log2 : -INFINITY;
        acc[t4][r] = s;
        mx = fmaxf(mx, s);
      }
      const float m_new = fmaxf(m_r[r], row16_max(mx));  // finite: token `base` is valid
      alpha_r[r] = exp2f(m_r[r] - m_new);
      float sum = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const float p = exp2f(acc[t4][r] - m_new);
        acc[t4][r] = p;
        sum += p;
      }
      l_r[r] = l_r[r] * alpha_r[r] + sum;
      m_r[r] = m_new;
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
      *reinterpret_cast<f32x4_t*>(&p_lds[wave][16 * t4 + row][4 * grp]) = acc[t4];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- rescale and accumulate P.V on the vector ALU
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float a = read_lane(alpha_r[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= a;
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int tl = it * TPI + v_sub;
      float p[GP];
      if constexpr (GP >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < GP; h4 += 4) {
          const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&p_lds[wave][tl][h4]);
          p[h4] = pv[0]; p[h4 + 1] = pv[1]; p[h4 + 2] = pv[2]; p[h4 + 3] = pv[3];
        }
      } else {
#pragma unroll
        for (int h = 0; h < GP; ++h) p[h] = p_lds[wave][tl][h];
      }
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_lo(vb[it][w]);
        v[2 * w + 1] = bf16_hi(vb[it][w]);
      }
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += p[h] * v[e];
    }
    // p_lds[wave] is rewritten next iteration: keep this wave's reads before those writes
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge lanes of the wave: sums over the token sub-groups of each chunk
#pragma unroll
  for (int h = 0; h < GP; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[h][e];
#pragma unroll
      for (int sft = DCH; sft < 64; sft <<= 1) x += __shfl_xor(x, sft, 64);
      o[h][e] = x;
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) l_r[r] = row16_sum(l_r[r]);
  if (row == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m_lds[wave][4 * grp + r] = m_r[r];
      l_lds[wave][4 * grp + r] = l_r[r];
    }
  }
  if (v_sub == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o_lds[wave][h][v_chunk * 8 + e] = o[h][e];
  }
  __syncthreads();

  // ---- merge the four waves exactly, then write the output or the split's partial
  for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_lds[w][h]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(m_lds[w][h] - M);  // 0 for a wave without tokens
      lsum += f * l_lds[w][h];
      osum += f * o_lds[w][h][d];
    }
    const int64_t hq = static_cast<int64_t>(b) * Hq + h0 + h;
    if (n_splits == 1) {
      out[hq * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(osum / lsum));
    } else {
      ws_o[(hq * max_splits + split) * D + d] = osum;
      if (d == 0) ws_ml[hq * max_splits + split] = make_float2(M, lsum);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml, uint16_t* __restrict__ out,
    const int32_t* __restrict__ context_lens, int Hq, int split_tokens, int max_splits) {
  const int b = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= Hq * D) return;
  const int L = context_lens[b];
  const int n = (L + split_tokens - 1) / split_tokens;
  if (n <= 1) return;  // written directly by the split kernel
  const int h = idx / D;
  const int d = idx - h * D;
  const int64_t hq = static_cast<int64_t>(b) * Hq + h;
  const float2* ml = ws_ml + hq * max_splits;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, ml[s].x);
  float lsum = 0.f, osum = 0.f;
  for (int s = 0; s < n; ++s) {
    const float f = exp2f(ml[s].x - M);
    lsum += f * ml[s].y;
    osum += f * ws_o[(hq * max_splits + s) * D + d];
  }
  out[hq * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(osum / lsum));
}

void decode_split_plan(int max_context_len, int num_splits, int* split_tokens,
                       int* max_splits) {
  const int chunks = (max_context_len + 255) / 256;
  const int per = num_splits > 0 ? (chunks + num_splits - 1) / num_splits : 1;
  *split_tokens = per * 256;
  *max_splits = (max_context_len + *split_tokens - 1) / *split_tokens;
}

template <int D, int GP>
static void launch_split(dim3 grid, hipStream_t stream, const uint16_t* q, uint16_t* out,
                         const uint16_t* kc, const uint16_t* vc, const int32_t* ctx,
                         const int32_t* tables, int stride, int Hq, int Hkv, int G, int n_hg,
                         int bs_log2, int split_tokens, int max_splits, float scale_log2,
                         float* ws_o, float2* ws_ml) {
  hipLaunchKernelGGL((paged_decode_bf16_kernel<D, GP>), grid, dim3(256), 0, stream, q, out, kc,
                     vc, ctx, tables, stride, Hq, Hkv, G, n_hg, bs_log2, split_tokens, max_splits,
                     scale_log2, ws_o, ws_ml);
}

hipError_t launch_paged_decode_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                    const void* v_cache, int num_q_heads, int num_kv_heads,
                                    int bs_log2, int batch, const int32_t* context_lens,
                                    const int32_t* block_tables, int table_stride, float scale,
                                    int split_tokens, int max_splits, void* workspace,
                                    hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int GP = G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1));
  const int n_hg = (G + GP - 1) / GP;
  if (num_kv_heads * n_hg > 65535) return hipErrorInvalidConfiguration;
  const float scale_log2 = scale * kLog2e;
  float* ws_o = static_cast<float*>(workspace);
  float2* ws_ml = nullptr;
  if (max_splits > 1)
    ws_ml = reinterpret_cast<float2*>(ws_o + static_cast<int64_t>(batch) * num_q_heads *
                                                 max_splits * head_dim);
  const dim3 grid(max_splits, num_kv_heads * n_hg, batch);
  auto qq = static_cast<const uint16_t*>(q);
  auto oo = static_cast<uint16_t*>(out);
  auto kc = static_cast<const uint16_t*>(k_cache);
  auto vc = static_cast<const uint16_t*>(v_cache);
#define PKV_SPLIT(D_, GP_)                                                                   \
  launch_split<D_, GP_>(grid, stream, qq, oo, kc, vc, context_lens, block_tables,            \
                        table_stride, num_q_heads, num_kv_heads, G, n_hg, bs_log2,           \
                        split_tokens, max_splits, scale_log2, ws_o, ws_ml)
  timing_begin("paged_decode_split", stream);
  if (head_dim == 128) {
    switch (GP) {
      case 1: PKV_SPLIT(128, 1); break;
      case 2: PKV_SPLIT(128, 2); break;
      case 4: PKV_SPLIT(128, 4); break;
      default: PKV_SPLIT(128, 8); break;
    }
  } else {
    switch (GP) {
      case 1: PKV_SPLIT(64, 1); break;
      case 2: PKV_SPLIT(64, 2); break;
      case 4: PKV_SPLIT(64, 4); break;
      default: PKV_SPLIT(64, 8); break;
    }
  }
#undef PKV_SPLIT
  timing_end(stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_splits <= 1) return e;
  const dim3 cgrid((num_q_heads * head_dim + 255) / 256, batch);
  timing_begin("paged_decode_combine", stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, cgrid, dim3(256), 0, stream, ws_o, ws_ml, oo,
                       context_lens, num_q_heads, split_tokens, max_splits);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, cgrid, dim3(256), 0, stream, ws_o, ws_ml, oo,
                       context_lens, num_q_heads, split_tokens, max_splits);
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace pkv
