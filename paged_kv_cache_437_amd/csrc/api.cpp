// C ABI of libpkv (declared in include/pkv.h): host-side validation and dispatch.
// Nothing here touches the device before every host argument has been checked.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "../../include/pkv.h"
#include "errors.h"
#include "launch.h"
#include "validate.h"

namespace {

thread_local char g_last_error[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pkv_status ok() {
  g_last_error[0] = '\0';
  return PKV_OK;
}

}  // namespace

namespace pkv {

pkv_status report_error(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pkv_status report_ok() { return ok(); }

}  // namespace pkv

namespace {

int log2_exact(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return (1 << r) == x ? r : -1;
}

pkv_status check_cache(const pkv_cache* c) {
  if (c == nullptr) return fail(PKV_ERR_INVALID, "cache descriptor is NULL");
  if (c->k_cache == nullptr || c->v_cache == nullptr)
    return fail(PKV_ERR_INVALID, "k_cache / v_cache is NULL");
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID, "num_blocks and num_kv_heads must be positive");
  if (c->dtype != PKV_F32 && c->dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not PKV_F32 or PKV_BF16", c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", c->head_dim);
  if (c->block_size < 1 || c->block_size > 256 || log2_exact(c->block_size) < 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d (built: powers of two in [1, 256])",
                c->block_size);
  return PKV_OK;
}

pkv_status check_heads(const pkv_cache* c, int32_t num_q_heads) {
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, c->num_kv_heads);
  if (num_q_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d > 65535", num_q_heads);
  return PKV_OK;
}

pkv_status check_rotary(const pkv_cache* cache, const pkv_rotary* rot) {
  if (rot == nullptr) return fail(PKV_ERR_INVALID, "rotary descriptor is NULL");
  if (rot->cos_sin == nullptr) return fail(PKV_ERR_INVALID, "rotary cos_sin table is NULL");
  if (rot->max_position < 1)
    return fail(PKV_ERR_INVALID, "rotary max_position %d < 1", rot->max_position);
  (void)cache;
  return PKV_OK;
}

pkv_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

size_t elem_size(const pkv_cache* c) { return c->dtype == PKV_F32 ? 4 : 2; }

// upper bound on an explicit decode worker count (the automatic count is 1024 or 2048)
constexpr int32_t kMaxWorkers = 1 << 20;

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP launch error";
    case PKV_ERR_NO_BLOCKS: return "KV block pool exhausted";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error; }

int32_t pkv_version(void) { return 200; }

pkv_status pkv_store_kvcache_rotary(const pkv_cache* cache, const void* k, const void* v,
                                    const int32_t* slot_mapping, const int32_t* positions,
                                    int32_t num_tokens, const pkv_rotary* rotary,
                                    hipStream_t stream) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if ((st = check_rotary(cache, rotary)) != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (k == nullptr || v == nullptr || slot_mapping == nullptr || positions == nullptr)
    return fail(PKV_ERR_INVALID, "k, v, slot_mapping or positions is NULL");
  if (pkv::debug_checks_on() &&
      (st = pkv_validate_store(cache, slot_mapping, num_tokens, 0, nullptr, stream)) != PKV_OK)
    return st;
  return launched(pkv::launch_store_kvcache_rotary(
                      cache->dtype == PKV_BF16, cache->head_dim, cache->k_cache, cache->v_cache,
                      k, v, slot_mapping, positions, num_tokens, cache->num_kv_heads,
                      rotary->cos_sin, rotary->max_position, stream),
                  "store_kvcache_rotary");
}

pkv_status pkv_store_kvcache(const pkv_cache* cache, const void* k, const void* v,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             hipStream_t stream) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (k == nullptr || v == nullptr || slot_mapping == nullptr)
    return fail(PKV_ERR_INVALID, "k, v or slot_mapping is NULL");
  const size_t row_bytes = elem_size(cache) * cache->num_kv_heads * cache->head_dim;
  if (row_bytes > (1u << 30)) return fail(PKV_ERR_UNSUPPORTED, "row of %zu bytes", row_bytes);
  if (pkv::debug_checks_on() &&
      (st = pkv_validate_store(cache, slot_mapping, num_tokens, 0, nullptr, stream)) != PKV_OK)
    return st;
  return launched(pkv::launch_store_kvcache(cache->k_cache, cache->v_cache, k, v, slot_mapping,
                                            num_tokens, static_cast<int32_t>(row_bytes), stream),
                  "store_kvcache");
}

namespace {

pkv_status prefill_impl(const pkv_cache* cache, const void* q, void* out, int32_t num_q_heads,
                        int32_t batch, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, const int32_t* block_tables,
                        int32_t block_table_stride, float scale, const pkv_rotary* rot,
                        hipStream_t stream, bool dry = false) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != PKV_OK) return st;
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || block_table_stride < 0)
    return fail(PKV_ERR_INVALID, "negative batch / max_seqlen / stride");
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch == 0 || max_seqlen_q == 0) return ok();
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr ||
      block_tables == nullptr)
    return fail(PKV_ERR_INVALID, "q, out, cu_seqlens_q/k or block_tables is NULL");
  if (max_seqlen_k < max_seqlen_q)
    return fail(PKV_ERR_INVALID, "max_seqlen_k %d < max_seqlen_q %d", max_seqlen_k, max_seqlen_q);
  const int64_t need = (static_cast<int64_t>(max_seqlen_k) + cache->block_size - 1) /
                       cache->block_size;
  if (block_table_stride < need)
    return fail(PKV_ERR_INVALID, "block_table_stride %d < ceil(max_seqlen_k / block_size) %lld",
                block_table_stride, static_cast<long long>(need));
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PKV_ERR_INVALID, "scale %g must be finite and positive", scale);
  if (dry) return PKV_OK;
  if (pkv::debug_checks_on() &&
      (st = pkv_validate_prefill(cache, batch, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                 max_seqlen_k, block_tables, block_table_stride, 0, nullptr,
                                 stream)) != PKV_OK)
    return st;
  const int bs_log2 = log2_exact(cache->block_size);
  const float* cs = rot != nullptr ? rot->cos_sin : nullptr;
  const int max_pos = rot != nullptr ? rot->max_position : 0;
  if (cache->dtype == PKV_BF16)
    return launched(pkv::launch_paged_prefill_bf16(
                        cache->head_dim, q, out, cache->k_cache, cache->v_cache, num_q_heads,
                        cache->num_kv_heads, bs_log2, batch, max_seqlen_q, cu_seqlens_q,
                        cu_seqlens_k, block_tables, block_table_stride, scale, cs, max_pos,
                        stream),
                    "paged_prefill");
  return launched(pkv::launch_attention_generic(
                      false, cache->head_dim, q, out, cache->k_cache, cache->v_cache,
                      num_q_heads, cache->num_kv_heads, bs_log2, batch, max_seqlen_q,
                      cu_seqlens_q, cu_seqlens_k, nullptr, block_tables, block_table_stride,
                      scale, cs, max_pos, stream),
                  "paged_prefill");
}

}  // namespace

pkv_status pkv_paged_prefill(const pkv_cache* cache, const void* q, void* out,
                             int32_t num_q_heads, int32_t batch,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             const int32_t* block_tables, int32_t block_table_stride,
                             float scale, hipStream_t stream) {
  return prefill_impl(cache, q, out, num_q_heads, batch, cu_seqlens_q, cu_seqlens_k,
                      max_seqlen_q, max_seqlen_k, block_tables, block_table_stride, scale,
                      nullptr, stream);
}

pkv_status pkv_paged_prefill_rotary(const pkv_cache* cache, const void* q, void* out,
                                    int32_t num_q_heads, int32_t batch,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    float scale, const pkv_rotary* rotary, hipStream_t stream) {
  const pkv_status st = check_rotary(cache, rotary);
  if (st != PKV_OK) return st;
  return prefill_impl(cache, q, out, num_q_heads, batch, cu_seqlens_q, cu_seqlens_k,
                      max_seqlen_q, max_seqlen_k, block_tables, block_table_stride, scale,
                      rotary, stream);
}

size_t pkv_paged_decode_workspace_size(const pkv_cache* cache, int32_t num_q_heads,
                                       int32_t batch, int32_t max_context_len,
                                       int32_t num_workers) {
  if (cache == nullptr || num_q_heads <= 0 || batch <= 0 || max_context_len <= 0 ||
      num_workers < 0 || num_workers > kMaxWorkers || cache->num_kv_heads <= 0 ||
      num_q_heads % cache->num_kv_heads != 0 ||
      (cache->head_dim != 64 && cache->head_dim != 128))
    return 0;
  if (cache->dtype != PKV_BF16) return 0;  // the fp32 path needs none
  return pkv::paged_decode_bf16_workspace(cache->head_dim, num_q_heads, cache->num_kv_heads,
                                          batch, num_workers);
}

namespace {

pkv_status decode_impl(const pkv_cache* cache, const void* q, void* out, int32_t num_q_heads,
                       int32_t batch, const int32_t* context_lens, int32_t max_context_len,
                       const int32_t* block_tables, int32_t block_table_stride, float scale,
                       void* workspace, size_t workspace_bytes, int32_t num_workers,
                       const pkv_rotary* rot, hipStream_t stream, bool dry = false) {
  pkv_status st = check_cache(cache);
  if (st != PKV_OK) return st;
  if ((st = check_heads(cache, num_q_heads)) != PKV_OK) return st;
  if (batch < 0 || max_context_len < 0 || block_table_stride < 0 || num_workers < 0)
    return fail(PKV_ERR_INVALID, "negative batch / max_context_len / stride / num_workers");
  if (num_workers > kMaxWorkers)
    return fail(PKV_ERR_INVALID, "num_workers %d > %d", num_workers, kMaxWorkers);
  if (batch > 65535) return fail(PKV_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if (batch == 0) return ok();
  if (max_context_len == 0) return fail(PKV_ERR_INVALID, "max_context_len is 0");
  if (q == nullptr || out == nullptr || context_lens == nullptr || block_tables == nullptr)
    return fail(PKV_ERR_INVALID, "q, out, context_lens or block_tables is NULL");
  const int64_t need = (static_cast<int64_t>(max_context_len) + cache->block_size - 1) /
                       cache->block_size;
  if (block_table_stride < need)
    return fail(PKV_ERR_INVALID, "block_table_stride %d < ceil(max_context_len / block_size) %lld",
                block_table_stride, static_cast<long long>(need));
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PKV_ERR_INVALID, "scale %g must be finite and positive", scale);
  const size_t ws = pkv_paged_decode_workspace_size(cache, num_q_heads, batch, max_context_len,
                                                    num_workers);
  if (ws > 0 && (workspace == nullptr || workspace_bytes < ws))
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, ws);
  if (dry) return PKV_OK;
  if (pkv::debug_checks_on() &&
      (st = pkv_validate_decode(cache, batch, context_lens, max_context_len, block_tables,
                                block_table_stride, 0, nullptr, stream)) != PKV_OK)
    return st;
  const int bs_log2 = log2_exact(cache->block_size);
  const float* cs = rot != nullptr ? rot->cos_sin : nullptr;
  const int max_pos = rot != nullptr ? rot->max_position : 0;
  if (cache->dtype == PKV_BF16)
    return launched(pkv::launch_paged_decode_bf16(
                        cache->head_dim, q, out, cache->k_cache, cache->v_cache, num_q_heads,
                        cache->num_kv_heads, bs_log2, batch, context_lens, block_tables,
                        block_table_stride, scale, num_workers, workspace, cs, max_pos, stream),
                    "paged_decode");
  return launched(pkv::launch_attention_generic(
                      false, cache->head_dim, q, out, cache->k_cache, cache->v_cache,
                      num_q_heads, cache->num_kv_heads, bs_log2, batch, 1, nullptr, nullptr,
                      context_lens, block_tables, block_table_stride, scale, cs, max_pos,
                      stream),
                  "paged_decode");
}

}  // namespace

pkv_status pkv_paged_decode(const pkv_cache* cache, const void* q, void* out,
                            int32_t num_q_heads, int32_t batch,
                            const int32_t* context_lens, int32_t max_context_len,
                            const int32_t* block_tables, int32_t block_table_stride,
                            float scale, void* workspace, size_t workspace_bytes,
                            int32_t num_workers, hipStream_t stream) {
  return decode_impl(cache, q, out, num_q_heads, batch, context_lens, max_context_len,
                     block_tables, block_table_stride, scale, workspace, workspace_bytes,
                     num_workers, nullptr, stream);
}

pkv_status pkv_paged_decode_rotary(const pkv_cache* cache, const void* q, void* out,
                                   int32_t num_q_heads, int32_t batch,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   int32_t num_workers, const pkv_rotary* rotary,
                                   hipStream_t stream) {
  const pkv_status st = check_rotary(cache, rotary);
  if (st != PKV_OK) return st;
  return decode_impl(cache, q, out, num_q_heads, batch, context_lens, max_context_len,
                     block_tables, block_table_stride, scale, workspace, workspace_bytes,
                     num_workers, rotary, stream);
}

pkv_status pkv_paged_decode_append(const pkv_cache* cache, const void* q, const void* k_new,
                                   const void* v_new, void* out, int32_t num_q_heads,
                                   int32_t batch, const int32_t* slot_mapping,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   int32_t num_workers, hipStream_t stream) {
  pkv_status st = decode_impl(cache, q, out, num_q_heads, batch, context_lens, max_context_len,
                              block_tables, block_table_stride, scale, workspace,
                              workspace_bytes, num_workers, nullptr, stream, true);
  if (st != PKV_OK || batch == 0) return st;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr)
    return fail(PKV_ERR_INVALID, "k_new, v_new or slot_mapping is NULL");
  if (cache->dtype == PKV_BF16) {
    if (pkv::debug_checks_on() &&
        ((st = pkv_validate_store(cache, slot_mapping, batch, 0, nullptr, stream)) != PKV_OK ||
         (st = pkv_validate_decode(cache, batch, context_lens, max_context_len, block_tables,
                                   block_table_stride, 0, nullptr, stream)) != PKV_OK))
      return st;
    const hipError_t e = pkv::launch_paged_decode_append_bf16(
        cache->head_dim, q, out, cache->k_cache, cache->v_cache, num_q_heads,
        cache->num_kv_heads, log2_exact(cache->block_size), batch, context_lens, block_tables,
        block_table_stride, scale, num_workers, workspace, k_new, v_new, slot_mapping, stream);
    if (e != hipErrorNotSupported) return launched(e, "paged_decode_append");
  }
  // grouped heads, blocks shorter than a decode chunk, or an fp32 cache: the two kernels
  // in turn
  if ((st = pkv_store_kvcache(cache, k_new, v_new, slot_mapping, batch, stream)) != PKV_OK)
    return st;
  return pkv_paged_decode(cache, q, out, num_q_heads, batch, context_lens, max_context_len,
                          block_tables, block_table_stride, scale, workspace, workspace_bytes,
                          num_workers, stream);
}

}  // extern "C"

pkv_status pkv_mixed_attention(const pkv_cache* cache, int32_t num_q_heads, float scale,
                               const void* q_prefill, void* out_prefill, int32_t prefill_batch,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               const int32_t* prefill_tables, int32_t prefill_table_stride,
                               const void* q_decode, void* out_decode, int32_t decode_batch,
                               const int32_t* context_lens, int32_t max_context_len,
                               const int32_t* decode_tables, int32_t decode_table_stride,
                               void* workspace, size_t workspace_bytes, int32_t num_workers,
                               const pkv_rotary* rotary, hipStream_t stream) {
  pkv_status st;
  if (rotary != nullptr && (st = check_rotary(cache, rotary)) != PKV_OK) return st;
  if ((st = prefill_impl(cache, q_prefill, out_prefill, num_q_heads, prefill_batch,
                         cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, prefill_tables,
                         prefill_table_stride, scale, rotary, stream, true)) != PKV_OK)
    return st;
  if ((st = decode_impl(cache, q_decode, out_decode, num_q_heads, decode_batch, context_lens,
                        max_context_len, decode_tables, decode_table_stride, scale, workspace,
                        workspace_bytes, num_workers, rotary, stream, true)) != PKV_OK)
    return st;
  if (cache->dtype == PKV_BF16 && prefill_batch > 0 && max_seqlen_q > 0 && decode_batch > 0) {
    if (pkv::debug_checks_on() &&
        ((st = pkv_validate_prefill(cache, prefill_batch, cu_seqlens_q, cu_seqlens_k,
                                    max_seqlen_q, max_seqlen_k, prefill_tables,
                                    prefill_table_stride, 0, nullptr, stream)) != PKV_OK ||
         (st = pkv_validate_decode(cache, decode_batch, context_lens, max_context_len,
                                   decode_tables, decode_table_stride, 0, nullptr, stream)) !=
             PKV_OK))
      return st;
    const hipError_t e = pkv::launch_mixed_attention_bf16(
        cache->head_dim, cache->k_cache, cache->v_cache, num_q_heads, cache->num_kv_heads,
        log2_exact(cache->block_size), scale, q_prefill, out_prefill, prefill_batch,
        max_seqlen_q, cu_seqlens_q, cu_seqlens_k, prefill_tables, prefill_table_stride, q_decode,
        out_decode, decode_batch, context_lens, decode_tables, decode_table_stride, num_workers,
        workspace, rotary != nullptr ? rotary->cos_sin : nullptr,
        rotary != nullptr ? rotary->max_position : 0, stream);
    if (e != hipErrorNotSupported) return launched(e, "mixed_attention");
  }
  // shapes the single launch does not cover (and steps with one phase only): the two
  // passes one after the other on the same stream
  if ((st = prefill_impl(cache, q_prefill, out_prefill, num_q_heads, prefill_batch,
                         cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, prefill_tables,
                         prefill_table_stride, scale, rotary, stream)) != PKV_OK)
    return st;
  return decode_impl(cache, q_decode, out_decode, num_q_heads, decode_batch, context_lens,
                     max_context_len, decode_tables, decode_table_stride, scale, workspace,
                     workspace_bytes, num_workers, rotary, stream);
}
