// Merge of the decode partials (internal; the division of work is in
// decode_plan.h).  A stream cut between workers left one fp32 partial per worker:
// the running max m (log2 domain), the sum l of 2^(s - m) and the unnormalised
// output o.  The merge is exact in real arithmetic and runs in worker order, so the
// result does not depend on timing:  M = max_w m_w,
//   out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w,  rounded once to bf16.
// (“深入 Nano-vLLM 推理引擎”, "Prefill and Decode": the query of a decode step
// attends to the sequence's whole cached context; the cut is a work division.)
#include "decode_plan.h"
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

namespace {

constexpr int kMergeBatch = 8;  // partials loaded together

// Grid: (stream within sequence * HS + head, sequence), D threads: thread d merges
// element d of one head of one stream.  Stream j covers kv heads kvg*MH + hh
// (hh < MH, kvg = j / n_hg) and, of each, q heads hg*GP + g (g < GP, hg = j % n_hg);
// its partials hold HS = MH * GP heads, head h = hh*GP + g.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(
    const int64_t* __restrict__ ws_prefix, const float2* __restrict__ ws_ml,
    const float* __restrict__ ws_o, uint16_t* __restrict__ out,
    const int32_t* __restrict__ context_lens, int batch, int Hq, int G, int GP, int MH,
    int n_hg, int ch_log2, int num_workers) {
  const int HS = MH * GP;
  const int j = blockIdx.x / HS;
  const int h = blockIdx.x - j * HS;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int kvg = j / n_hg;
  const int hg = j - kvg * n_hg;
  const int hh = h / GP;
  const int g = h - hh * GP;
  if (g >= min(GP, G - hg * GP)) return;  // q head past the group's heads
  // independent loads first
  const int L = context_lens[b];
  const int64_t C = ws_prefix[batch];
  const int64_t first = ws_prefix[b];
  const int nch = chunks_of(L, ch_log2);
  if (nch == 0) return;
  const int64_t W = num_workers;
  const int64_t cs = first + static_cast<int64_t>(j) * nch;  // the stream's chunks
  const int64_t ce = cs + nch - 1;
  const int64_t wa = worker_of(cs, C, W);
  const int64_t wb = worker_of(ce, C, W);
  if (wa == wb) return;  // finished by one worker

  // The stream's workers, up to D per pass: each thread finds one worker's partial
  // slot (-1 for a worker with no chunks), then every thread merges them in worker
  // order.
  __shared__ int64_t s_slot[D];
  float M = -INFINITY, lsum = 0.f, osum = 0.f;
  for (int64_t base = wa; base <= wb; base += D) {
    const int n = static_cast<int>(min(static_cast<int64_t>(D), wb - base + 1));
    __syncthreads();  // the previous pass has read s_slot
    if (d < n) {
      const int64_t w = base + d;
      const int64_t s0 = worker_start(w, C, W);
      const int64_t s1 = worker_start(w + 1, C, W);
      // the stream's segment is the worker's first unless the worker began before it
      s_slot[d] = s0 == s1 ? -1 : 2 * w + (w == wa && s0 < cs ? 1 : 0);
    }
    __syncthreads();
    for (int p0 = 0; p0 < n; p0 += kMergeBatch) {
      float2 ml[kMergeBatch];
      float ov[kMergeBatch];
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) {
        ml[p] = make_float2(-INFINITY, 0.f);
        ov[p] = 0.f;
        const int64_t slot = p0 + p < n ? s_slot[p0 + p] : -1;
        if (slot < 0) continue;
        ml[p] = ws_ml[slot * HS + h];
        ov[p] = ws_o[(slot * HS + h) * D + d];
      }
      float Mn = M;
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) Mn = fmaxf(Mn, ml[p].x);
      const float f = exp2f(M - Mn);  // 0 on the first batch (M = -inf)
      lsum *= f;
      osum *= f;
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) {
        const float x = exp2f(ml[p].x - Mn);  // 0 for the empty entries
        lsum += x * ml[p].y;
        osum += x * ov[p];
      }
      M = Mn;
    }
  }
  const int64_t row = static_cast<int64_t>(b) * Hq + (kvg * MH + hh) * G + hg * GP + g;
  out[row * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(osum / lsum));
}

}  // namespace

hipError_t launch_decode_combine(int head_dim, int GP, int MH, const DecodeWorkspace& ws,
                                 void* out, const int32_t* context_lens, int batch,
                                 int num_q_heads, int num_kv_heads, int num_workers,
                                 hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int n_hg = (G + GP - 1) / GP;
  const int S = (num_kv_heads / MH) * n_hg;
  if (S > 65535) return hipErrorInvalidConfiguration;
  const int ch = chunk_tokens(head_dim, MH);
  int ch_log2 = 0;
  while ((1 << ch_log2) < ch) ++ch_log2;
  if (static_cast<int64_t>(S) * MH * GP > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(S * MH * GP, batch);
  uint16_t* o = static_cast<uint16_t*>(out);
  timing_begin("paged_decode_combine", stream);
  if (head_dim == 128)
    hipExtLaunchKernelGGL((decode_combine_kernel<128>), grid, dim3(128), 0, stream, timing_start(),
                          timing_stop(), 0, ws.prefix, ws.ml, ws.o, o, context_lens, batch,
                          num_q_heads, G, GP, MH, n_hg, ch_log2, num_workers);
  else
    hipExtLaunchKernelGGL((decode_combine_kernel<64>), grid, dim3(64), 0, stream, timing_start(),
                          timing_stop(), 0, ws.prefix, ws.ml, ws.o, o, context_lens, batch,
                          num_q_heads, G, GP, MH, n_hg, ch_log2, num_workers);
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace pkv
