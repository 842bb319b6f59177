// The decode's division of work, shared by the streaming kernel and the merge
// kernel (internal).  A stream is (sequence, kv head, group of up to GP q heads of
// that kv head); it is cut into chunks of kDecodeChunk tokens.  All chunks of all
// streams, in (sequence, stream, position) order, form one list of C chunks; worker
// w (a wavefront) takes chunks [w*C/W, (w+1)*C/W).  A worker's first segment (its
// run of chunks of one stream) leaves its partial, if any, in slot 2w, any later one
// in slot 2w+1; a stream that all falls to one worker is written out directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kDecodeChunk = 16;       // tokens per chunk
constexpr int kMaxAutoWorkers = 4096;  // bound on the automatic worker count

// q heads per stream for Hq / Hkv = G: G rounded up to a power of two, at most 8
inline int heads_per_stream(int G) { return G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1)); }

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace: int64 [batch+1] first chunk of each sequence (the last entry is C),
// then float2 [2W][GP] (max, sum) and float [2W][GP][D] unnormalised outputs.
struct DecodeWorkspace {
  int64_t* prefix;
  float2* ml;
  float* o;
};
inline DecodeWorkspace carve_decode_workspace(void* ws, int batch, int W, int GP) {
  char* base = static_cast<char*>(ws);
  DecodeWorkspace d;
  d.prefix = reinterpret_cast<int64_t*>(base);
  base += align256(sizeof(int64_t) * (static_cast<size_t>(batch) + 1));
  d.ml = reinterpret_cast<float2*>(base);
  base += align256(sizeof(float2) * 2 * static_cast<size_t>(W) * GP);
  d.o = reinterpret_cast<float*>(base);
  return d;
}
inline size_t decode_workspace_bytes(int batch, int W, int GP, int D) {
  return align256(sizeof(int64_t) * (static_cast<size_t>(batch) + 1)) +
         align256(sizeof(float2) * 2 * static_cast<size_t>(W) * GP) +
         sizeof(float) * 2 * static_cast<size_t>(W) * GP * D;
}

// chunks of a sequence of length L
__device__ __forceinline__ int chunks_of(int L) {
  return (max(L, 0) + kDecodeChunk - 1) / kDecodeChunk;
}

// first chunk of worker w
__device__ __forceinline__ int64_t worker_start(int64_t w, int64_t C, int64_t W) {
  return w * C / W;
}

// worker owning chunk c (the largest w with worker_start(w) <= c)
__device__ __forceinline__ int64_t worker_of(int64_t c, int64_t C, int64_t W) {
  return ((c + 1) * W - 1) / C;
}

// Merge of the partials of the streams that were cut between workers.
hipError_t launch_decode_combine(int head_dim, int GP, const DecodeWorkspace& ws, void* out,
                                 const int32_t* context_lens, int batch, int num_q_heads,
                                 int num_kv_heads, int num_workers, hipStream_t stream);

}  // namespace pkv
