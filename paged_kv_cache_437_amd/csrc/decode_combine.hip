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

// Grid: (stream within sequence, sequence); a block of 128 threads loops over the
// stream's (head, head_dim) outputs.
template <int D, int GP>
__global__ __launch_bounds__(128) void decode_combine_kernel(
    const int64_t* __restrict__ ws_prefix, const float2* __restrict__ ws_ml,
    const float* __restrict__ ws_o, uint16_t* __restrict__ out,
    const int32_t* __restrict__ context_lens, int batch, int Hq, int G, int n_hg,
    int num_workers) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  // independent loads first
  const int L = context_lens[b];
  const int64_t C = ws_prefix[batch];
  const int64_t first = ws_prefix[b];
  const int nch = chunks_of(L);
  if (nch == 0) return;
  const int64_t W = num_workers;
  const int64_t cs = first + static_cast<int64_t>(j) * nch;  // the stream's chunks
  const int64_t ce = cs + nch - 1;
  const int64_t wa = worker_of(cs, C, W);
  const int64_t wb = worker_of(ce, C, W);
  if (wa == wb) return;  // finished by one worker
  const int kvh = j / n_hg;
  const int hg = j - kvh * n_hg;
  const int nh = min(GP, G - hg * GP);
  const int64_t hq0 = static_cast<int64_t>(b) * Hq + kvh * G + hg * GP;

  for (int idx = threadIdx.x; idx < nh * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY, lsum = 0.f, osum = 0.f;
    int64_t next_start = worker_start(wa, C, W);
    for (int64_t w0 = wa; w0 <= wb; w0 += kMergeBatch) {
      float2 ml[kMergeBatch];
      float ov[kMergeBatch];
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) {
        const int64_t w = w0 + p;
        ml[p] = make_float2(-INFINITY, 0.f);
        ov[p] = 0.f;
        if (w > wb) continue;
        const int64_t start = next_start;
        next_start = worker_start(w + 1, C, W);
        if (w > wa && start == next_start) continue;  // a worker with no chunks
        // the stream's segment is the worker's first unless the worker began before it
        const int64_t slot = 2 * w + (w == wa && start < cs ? 1 : 0);
        ml[p] = ws_ml[slot * GP + h];
        ov[p] = ws_o[(slot * GP + h) * D + d];
      }
      float Mn = M;
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) Mn = fmaxf(Mn, ml[p].x);
      const float f = exp2f(M - Mn);  // 0 on the first batch (M = -inf)
      lsum *= f;
      osum *= f;
#pragma unroll
      for (int p = 0; p < kMergeBatch; ++p) {
        const float e = exp2f(ml[p].x - Mn);  // 0 for the empty entries
        lsum += e * ml[p].y;
        osum += e * ov[p];
      }
      M = Mn;
    }
    out[(hq0 + h) * D + d] = static_cast<uint16_t>(f32_to_bf16_bits(osum / lsum));
  }
}

}  // namespace

hipError_t launch_decode_combine(int head_dim, int GP, const DecodeWorkspace& ws, void* out,
                                 const int32_t* context_lens, int batch, int num_q_heads,
                                 int num_kv_heads, int num_workers, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int n_hg = (G + GP - 1) / GP;
  const int S = num_kv_heads * n_hg;
  if (S > 65535) return hipErrorInvalidConfiguration;
  const dim3 grid(S, batch);
  uint16_t* o = static_cast<uint16_t*>(out);
  timing_begin("paged_decode_combine", stream);
#define PKV_COMB(D_, GP_)                                                                      \
  hipLaunchKernelGGL((decode_combine_kernel<D_, GP_>), grid, dim3(128), 0, stream, ws.prefix, \
                     ws.ml, ws.o, o, context_lens, batch, num_q_heads, G, n_hg, num_workers)
  if (head_dim == 128) {
    switch (GP) {
      case 1: PKV_COMB(128, 1); break;
      case 2: PKV_COMB(128, 2); break;
      case 4: PKV_COMB(128, 4); break;
      default: PKV_COMB(128, 8); break;
    }
  } else {
    switch (GP) {
      case 1: PKV_COMB(64, 1); break;
      case 2: PKV_COMB(64, 2); break;
      case 4: PKV_COMB(64, 4); break;
      default: PKV_COMB(64, 8); break;
    }
  }
#undef PKV_COMB
  timing_end(stream);
  return hipGetLastError();
}

}  // namespace pkv
