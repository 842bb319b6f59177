// Host-side launchers of the libpkv kernels (internal; the public API is include/pkv.h).
// Every launcher enqueues on `stream` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Row copy through a slot mapping; row_bytes = Hkv * D * element size (multiple of 16).
hipError_t launch_store_kvcache(void* k_cache, void* v_cache, const void* k, const void* v,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                int32_t row_bytes, hipStream_t stream);

// The same with K rotated at positions[t] on the way in (rotary table cos_sin,
// [max_position][head_dim] fp32); V copied.
hipError_t launch_store_kvcache_rotary(bool bf16, int head_dim, void* k_cache, void* v_cache,
                                       const void* k, const void* v,
                                       const int32_t* slot_mapping, const int32_t* positions,
                                       int32_t num_tokens, int num_kv_heads,
                                       const float* cos_sin, int max_position,
                                       hipStream_t stream);

// Generic attention: one wavefront per (query row, q head), vector ALU only.  Serves
// fp32 prefill and decode.  Decode when `context_lens` is non-null (one query per
// sequence), otherwise packed prefill over cu_seqlens_q / cu_seqlens_k.
hipError_t launch_attention_generic(bool bf16, int head_dim, const void* q, void* out,
                                    const void* k_cache, const void* v_cache, int num_q_heads,
                                    int num_kv_heads, int bs_log2, int batch, int max_q_rows,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int table_stride, float scale, const float* cos_sin,
                                    int max_position, hipStream_t stream);

// With cos_sin non-null, each query is rotated at position context_len - 1.
// bf16 paged decode: the streaming kernel over `num_workers` wavefront workers (0 =
// as many as the device holds resident) and the combine kernel for streams cut
// between workers.  The workspace holds, 256-byte aligned one after the other:
// int64 [batch+1] first chunk of each sequence, float2 [2W][GP] (max, sum) and
// float [2W][GP][head_dim] partial outputs, W the worker count and GP the q heads
// per stream; paged_decode_bf16_workspace gives its size.
size_t paged_decode_bf16_workspace(int head_dim, int num_q_heads, int num_kv_heads, int batch,
                                   int num_workers);
hipError_t launch_paged_decode_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                    const void* v_cache, int num_q_heads, int num_kv_heads,
                                    int bs_log2, int batch, const int32_t* context_lens,
                                    const int32_t* block_tables, int table_stride, float scale,
                                    int num_workers, void* workspace, const float* cos_sin,
                                    int max_position, hipStream_t stream);

// launch_paged_decode_bf16 (no rotary) that also appends the step's new token of each
// sequence: k_new / v_new [batch][num_kv_heads][head_dim] go into the cache at
// slot_mapping[b] (the slot of position context_lens[b] - 1; -1 skips the write), and the
// attention takes that token from k_new / v_new; cache and output bits are those of
// launch_store_kvcache followed by launch_paged_decode_bf16.  Returns
// hipErrorNotSupported for grouped heads (num_q_heads != num_kv_heads) or when a chunk
// would span blocks; the caller then launches both.
hipError_t launch_paged_decode_append_bf16(int head_dim, const void* q, void* out,
                                           const void* k_cache, const void* v_cache,
                                           int num_q_heads, int num_kv_heads, int bs_log2,
                                           int batch, const int32_t* context_lens,
                                           const int32_t* block_tables, int table_stride,
                                           float scale, int num_workers, void* workspace,
                                           const void* k_new, const void* v_new,
                                           const int32_t* slot_mapping, hipStream_t stream);

// The worker count the bf16 decode picks when asked for 0 (auto).
int paged_decode_bf16_workers(int head_dim, int num_q_heads, int num_kv_heads, int bs_log2);

// Prefill of some sequences and decode of others in one launch (bf16, block_size >= 64,
// at most 8 q heads per kv head), then the decode's merge kernel; the decode part is
// the same work division as launch_paged_decode_bf16 with the same worker count, so
// results are bit-identical to the two separate launches.  Returns
// hipErrorNotSupported for shapes outside that set (the caller launches separately).
hipError_t launch_mixed_attention_bf16(
    int head_dim, const void* k_cache, const void* v_cache, int num_q_heads, int num_kv_heads,
    int bs_log2, float scale, const void* q_prefill, void* out_prefill, int prefill_batch,
    int max_seqlen_q, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int32_t* prefill_tables, int prefill_stride, const void* q_decode, void* out_decode,
    int decode_batch, const int32_t* context_lens, const int32_t* decode_tables,
    int decode_stride, int num_workers, void* workspace, const float* cos_sin,
    int max_position, hipStream_t stream);

// bf16 varlen causal prefill on MFMA (one launch).  With cos_sin non-null, every query
// row is rotated at its position (rotary table [max_position][head_dim] fp32).
hipError_t launch_paged_prefill_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                     const void* v_cache, int num_q_heads, int num_kv_heads,
                                     int bs_log2, int batch, int max_seqlen_q,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     const int32_t* block_tables, int table_stride, float scale,
                                     const float* cos_sin, int max_position, hipStream_t stream);

}  // namespace pkv
