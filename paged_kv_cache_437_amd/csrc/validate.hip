// Contract checks of the metadata arrays the data-plane calls read: pkv_validate_* and
// the PKV_DEBUG gate in front of every data-plane call.
//
// The control plane chooses every block id and slot on the host and the data plane
// only copies into and reads from them (“深入 Nano-vLLM 推理引擎”, "Control plane vs. data
// plane"); the kernels therefore trust the arrays they are given, and a bad slot or
// length becomes an access outside the pool.  These checks name such arrays before any
// kernel touches the caches.  One predicate per contract, written once for both sides:
// the host check runs it over host arrays on the calling thread, the device check runs
// it in a kernel over device arrays and reports through a status word of the library's
// own (a __device__ variable, one per GPU), so neither side allocates anything.  Every
// read either side makes is bounded by the sizes the call passes, whatever the arrays
// hold.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "../../include/pkv.h"
#include "errors.h"
#include "validate.h"

namespace pkv {
namespace {

struct StoreArgs {
  const int32_t* slots;
  int32_t n;
  int64_t num_slots;  // num_blocks * block_size
};

struct SeqArgs {
  // prefill (cu_q != nullptr) or decode (ctx != nullptr)
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* ctx;
  int32_t batch;
  int32_t max_q;  // max_seqlen_q (prefill)
  int32_t max_k;  // max_seqlen_k (prefill) or max_context_len (decode)
  const int32_t* tables;
  int32_t stride;
  int32_t num_blocks;
  int32_t bs_log2;
};

// ---- the predicates (host and device) ----

__host__ __device__ inline uint32_t slot_violation(int32_t s, int64_t num_slots) {
  return (s != -1 && (s < 0 || s >= num_slots)) ? PKV_BAD_SLOT : 0u;
}

// Sequence b's lengths and table row.  The table entries read are those of the used
// blocks, capped at the row's stride, so the reads stay inside the table whatever the
// lengths say.
__host__ __device__ inline uint32_t sequence_violation(const SeqArgs& a, int b) {
  uint32_t v = 0;
  int64_t L;  // keys the sequence reads
  if (a.cu_q != nullptr) {
    if (b == 0 && (a.cu_q[0] != 0 || a.cu_k[0] != 0)) v |= PKV_BAD_SEQLENS;
    const int64_t lq = static_cast<int64_t>(a.cu_q[b + 1]) - a.cu_q[b];
    const int64_t lk = static_cast<int64_t>(a.cu_k[b + 1]) - a.cu_k[b];
    if (lq < 0 || lk < 0 || lk < lq || (lq > 0 && lk < 1) || lq > a.max_q || lk > a.max_k)
      v |= PKV_BAD_SEQLENS;
    L = lq > 0 ? lk : 0;  // a sequence with no queries reads nothing
  } else {
    L = a.ctx[b];
    if (L < 1 || L > a.max_k) v |= PKV_BAD_CONTEXT;
  }
  if (L <= 0) return v;
  const int64_t used = ((L - 1) >> a.bs_log2) + 1;
  if (used > a.stride) v |= PKV_BAD_STRIDE;
  const int64_t n = used < a.stride ? used : a.stride;
  const int32_t* row = a.tables + static_cast<int64_t>(b) * a.stride;
  for (int64_t j = 0; j < n; ++j)
    if (row[j] < 0 || row[j] >= a.num_blocks) {
      v |= PKV_BAD_TABLE;
      break;
    }
  return v;
}

// ---- device side ----

__global__ void clear_status_kernel(uint32_t* status) { status[0] = 0u; }

// Slots: range of each, and duplicates among the valid ones (token t against every
// u < t, in tiles of 256 staged through LDS: quadratic, which a debugging pass can
// afford at the sizes of one step).
__global__ __launch_bounds__(256) void validate_store_kernel(StoreArgs a, uint32_t* status) {
  __shared__ int32_t tile[256];
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int32_t s = t < a.n ? a.slots[t] : -1;
  uint32_t v = t < a.n ? slot_violation(s, a.num_slots) : 0u;
  const bool check_dup = t < a.n && s >= 0 && s < a.num_slots;
  for (int64_t u0 = 0; u0 <= static_cast<int64_t>(blockIdx.x) * 256; u0 += 256) {
    __syncthreads();
    const int64_t u = u0 + threadIdx.x;
    tile[threadIdx.x] = u < a.n ? a.slots[u] : -1;
    __syncthreads();
    if (check_dup) {
      const int64_t lim = min(static_cast<int64_t>(256), t - u0);  // entries u < t
      for (int64_t i = 0; i < lim; ++i)
        if (tile[i] == s) {
          v |= PKV_DUP_SLOT;
          break;
        }
    }
  }
  if (v != 0u) atomicOr(status, v);
}

__global__ __launch_bounds__(256) void validate_seq_kernel(SeqArgs a, uint32_t* status) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.batch) return;
  const uint32_t v = sequence_violation(a, b);
  if (v != 0u) atomicOr(status, v);
}

// the library's status word, one per device
__device__ uint32_t g_validate_status[1];

std::mutex g_status_mu;
uint32_t* g_status_ptr[64] = {};

hipError_t status_word(uint32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_status_mu);
  if (g_status_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_validate_status));
    if (e != hipSuccess) return e;
    g_status_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_status_ptr[dev];
  return hipSuccess;
}

// Runs `launch(status)` between a clear of the status word and its read-back, and waits.
template <typename F>
hipError_t run_device_check(F launch, hipStream_t stream, uint32_t* found) {
  uint32_t* status = nullptr;
  hipError_t e = status_word(&status);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  launch(status);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  uint32_t host = 0;
  if ((e = hipMemcpyAsync(&host, status, sizeof(host), hipMemcpyDeviceToHost, stream)) !=
      hipSuccess)
    return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  *found = host;
  return hipSuccess;
}

// ---- host side ----

uint32_t host_store(const StoreArgs& a) {
  uint32_t v = 0;
  std::vector<int32_t> valid;
  valid.reserve(a.n);
  for (int32_t t = 0; t < a.n; ++t) {
    const uint32_t x = slot_violation(a.slots[t], a.num_slots);
    v |= x;
    if (x == 0u && a.slots[t] >= 0) valid.push_back(a.slots[t]);
  }
  std::sort(valid.begin(), valid.end());
  if (std::adjacent_find(valid.begin(), valid.end()) != valid.end()) v |= PKV_DUP_SLOT;
  return v;
}

uint32_t host_seq(const SeqArgs& a) {
  uint32_t v = 0;
  for (int b = 0; b < a.batch; ++b) v |= sequence_violation(a, b);
  return v;
}

int log2_of(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

pkv_status describe(uint32_t v, uint32_t* out) {
  if (out != nullptr) *out = v;
  if (v == 0u) return report_ok();
  char msg[384];
  int n = std::snprintf(msg, sizeof(msg), "metadata contract violated:");
  const struct {
    uint32_t bit;
    const char* what;
  } names[] = {
      {PKV_BAD_SLOT, " slot outside [0, num_blocks*block_size) and not -1;"},
      {PKV_DUP_SLOT, " a slot written twice in one call;"},
      {PKV_BAD_TABLE, " a used block-table entry outside [0, num_blocks);"},
      {PKV_BAD_SEQLENS, " cu_seqlens not from 0 / decreasing, Lk < Lq, Lk = 0 with Lq > 0, "
                        "or a length above its max;"},
      {PKV_BAD_CONTEXT, " a context length < 1 or above max_context_len;"},
      {PKV_BAD_STRIDE, " ceil(length / block_size) > block_table_stride;"},
  };
  for (const auto& x : names)
    if ((v & x.bit) != 0u && n < static_cast<int>(sizeof(msg)))
      n += std::snprintf(msg + n, sizeof(msg) - n, "%s", x.what);
  return report_error(PKV_ERR_INVALID, "%s", msg);
}

std::atomic<int> g_debug{-1};  // -1: not read from the environment yet

pkv_status check_cache_desc(const pkv_cache* c) {
  if (c == nullptr) return report_error(PKV_ERR_INVALID, "cache descriptor is NULL");
  if (c->num_blocks <= 0 || c->block_size < 1 || c->block_size > 256 ||
      (c->block_size & (c->block_size - 1)) != 0)
    return report_error(PKV_ERR_INVALID, "num_blocks %d / block_size %d", c->num_blocks,
                        c->block_size);
  return PKV_OK;
}

}  // namespace

bool debug_checks_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char* env = std::getenv("PKV_DEBUG");
    d = (env != nullptr && env[0] != '\0' && !(env[0] == '0' && env[1] == '\0')) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, d);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d == 1;
}

}  // namespace pkv

using namespace pkv;

extern "C" {

pkv_status pkv_debug_enable(int32_t on) {
  g_debug.store(on != 0 ? 1 : 0);
  return PKV_OK;
}

int32_t pkv_debug_enabled(void) { return debug_checks_on() ? 1 : 0; }

pkv_status pkv_validate_store(const pkv_cache* cache, const int32_t* slot_mapping,
                              int32_t num_tokens, int32_t arrays_on_host, uint32_t* violations,
                              hipStream_t stream) {
  pkv_status st = check_cache_desc(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return report_error(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (num_tokens > 0 && slot_mapping == nullptr)
    return report_error(PKV_ERR_INVALID, "slot_mapping is NULL");
  if (violations != nullptr) *violations = 0;
  if (num_tokens == 0) return report_ok();
  const StoreArgs a{slot_mapping, num_tokens,
                    static_cast<int64_t>(cache->num_blocks) * cache->block_size};
  if (arrays_on_host) return describe(host_store(a), violations);
  uint32_t found = 0;
  const hipError_t e = run_device_check(
      [&](uint32_t* status) {
        hipLaunchKernelGGL(validate_store_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0,
                           stream, a, status);
      },
      stream, &found);
  if (e != hipSuccess)
    return report_error(PKV_ERR_HIP, "validate_store: %s", hipGetErrorString(e));
  return describe(found, violations);
}

static pkv_status validate_seqs(const pkv_cache* cache, const SeqArgs& a, int32_t on_host,
                                uint32_t* violations, hipStream_t stream) {
  if (a.batch == 0) return report_ok();
  if (on_host) return describe(host_seq(a), violations);
  uint32_t found = 0;
  const hipError_t e = run_device_check(
      [&](uint32_t* status) {
        hipLaunchKernelGGL(validate_seq_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, stream,
                           a, status);
      },
      stream, &found);
  if (e != hipSuccess) return report_error(PKV_ERR_HIP, "validate: %s", hipGetErrorString(e));
  (void)cache;
  return describe(found, violations);
}

pkv_status pkv_validate_prefill(const pkv_cache* cache, int32_t batch,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t arrays_on_host, uint32_t* violations,
                                hipStream_t stream) {
  pkv_status st = check_cache_desc(cache);
  if (st != PKV_OK) return st;
  if (batch < 0 || block_table_stride < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return report_error(PKV_ERR_INVALID, "negative batch / stride / max_seqlen");
  if (violations != nullptr) *violations = 0;
  if (batch > 0 && (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
                    (block_tables == nullptr && block_table_stride > 0)))
    return report_error(PKV_ERR_INVALID, "cu_seqlens_q/k or block_tables is NULL");
  const SeqArgs a{cu_seqlens_q, cu_seqlens_k, nullptr, batch, max_seqlen_q, max_seqlen_k,
                  block_tables, block_table_stride, cache->num_blocks,
                  log2_of(cache->block_size)};
  return validate_seqs(cache, a, arrays_on_host, violations, stream);
}

pkv_status pkv_validate_decode(const pkv_cache* cache, int32_t batch,
                               const int32_t* context_lens, int32_t max_context_len,
                               const int32_t* block_tables, int32_t block_table_stride,
                               int32_t arrays_on_host, uint32_t* violations,
                               hipStream_t stream) {
  pkv_status st = check_cache_desc(cache);
  if (st != PKV_OK) return st;
  if (batch < 0 || block_table_stride < 0 || max_context_len < 0)
    return report_error(PKV_ERR_INVALID, "negative batch / stride / max_context_len");
  if (violations != nullptr) *violations = 0;
  if (batch > 0 && (context_lens == nullptr || (block_tables == nullptr && block_table_stride > 0)))
    return report_error(PKV_ERR_INVALID, "context_lens or block_tables is NULL");
  const SeqArgs a{nullptr, nullptr, context_lens, batch, 0, max_context_len,
                  block_tables, block_table_stride, cache->num_blocks,
                  log2_of(cache->block_size)};
  return validate_seqs(cache, a, arrays_on_host, violations, stream);
}

}  // extern "C"
