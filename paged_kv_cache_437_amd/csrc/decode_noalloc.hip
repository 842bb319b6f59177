// pkv_paged_decode_noalloc: paged decode with the split-K workspace in a fixed device
// array of the library's own, for callers that cannot allocate (HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a stand-in, so
// each device's address is taken once, with that device current, through
// hipGetSymbolAddress and kept per device; only that address is ever handed to the
// kernels.  Calls on one device share its array: two calls in flight on one device at
// once (on different streams) race on it.  Nothing in it needs clearing between calls:
// the decode writes every entry of the workspace it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pkv.h"
#include "errors.h"

static constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB per device

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, its address taken on the first call there.
pkv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return pkv::report_error(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pkv::report_error(PKV_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev,
                             kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return pkv::report_error(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s",
                               dev, hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_noalloc(const pkv_cache* cache, const void* q, void* out,
                                               int32_t num_q_heads, int32_t batch,
                                               const int32_t* context_lens,
                                               int32_t max_context_len,
                                               const int32_t* block_tables,
                                               int32_t block_table_stride, float scale,
                                               int32_t num_workers, const pkv_rotary* rotary,
                                               hipStream_t stream) {
  const size_t need = pkv_paged_decode_workspace_size(cache, num_q_heads, batch,
                                                      max_context_len, num_workers);
  if (need > kScratchBytes)
    return pkv::report_error(PKV_ERR_WORKSPACE,
                             "decode needs %zu bytes of workspace; the fixed scratch of the "
                             "no-allocation entry point holds %zu (ask for fewer workers)",
                             need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const pkv_status st = scratch_address(&ws);
    if (st != PKV_OK) return st;
  }
  const size_t ws_bytes = ws != nullptr ? kScratchBytes : 0;
  if (rotary != nullptr)
    return pkv_paged_decode_rotary(cache, q, out, num_q_heads, batch, context_lens,
                                   max_context_len, block_tables, block_table_stride, scale, ws,
                                   ws_bytes, num_workers, rotary, stream);
  return pkv_paged_decode(cache, q, out, num_q_heads, batch, context_lens, max_context_len,
                          block_tables, block_table_stride, scale, ws, ws_bytes, num_workers,
                          stream);
}
