// The decode's division of work, shared by the streaming kernel and the merge
// kernel (internal).  A stream is (sequence, group of MH adjacent kv heads, group of
// up to GP q heads of each of those kv heads); it is cut into chunks of
// chunk_tokens(D, MH) tokens.  All chunks of all streams, in (sequence, stream,
// position) order, form one list of C chunks; worker w (a wavefront) takes chunks
// [w*C/W, (w+1)*C/W).  A worker's first segment (its run of chunks of one stream)
// leaves its partial, if any, in slot 2w, any later one in slot 2w+1; a stream that
// all falls to one worker is written out directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// The automatic worker count: a constant of the stream shape, never read from the
// device, so where streams are cut (and so the result bits) depends only on the
// lengths and the shape.  One wave per SIMD of a 256-CU part while a stream holds up
// to 4 q heads per kv head, two beyond: more concurrent streams read HBM less
// efficiently, so the smallest count that keeps the vector work hidden is the
// fastest (measured: at 4 q heads per kv head one wave per SIMD is 4-13% faster than
// two; at 8, two are 8% faster; 1536 or 2560 workers ran 10-20% slower than the
// multiples of 1024 around them).
inline int auto_decode_workers(int GP) { return GP <= 4 ? 1024 : 2048; }

// q heads per kv head in a stream for Hq / Hkv = G: G rounded up to a power of two,
// at most 8
inline int heads_per_stream(int G) { return G >= 8 ? 8 : (G >= 4 ? 4 : (G >= 2 ? 2 : 1)); }

// kv heads per stream: the largest power of two that divides Hkv and spans at most
// 512 contiguous bytes of a token's row (2 at head_dim 128, 4 at 64), or 1 KB from 8 q
// heads per kv head up.  Measured on the decode at head_dim 128: with one q head per
// kv head 512 bytes per token beat 256 and 1 KB (whose 4-token chunks cost more per
// byte; 1 KB was 8% slower); at 4 q heads per kv head 512 bytes and 1 KB tie; at 8,
// 1 KB is 8% faster (the wider stream halves the streams, each chunk's vector work
// being the same).
inline int kv_heads_per_stream(int D, int Hkv, int G) {
  const int limit = heads_per_stream(G) >= 8 ? 1024 : 512;
  int mh = 1;
  while (mh * 2 * D * 2 <= limit && Hkv % (mh * 2) == 0) mh *= 2;
  return mh;
}

// Tokens per chunk: four 1 KB load instructions of K (and four of V) per lane group,
// i.e. 8 KB of K and V per chunk
__host__ __device__ constexpr int chunk_tokens(int D, int MH) { return 2048 / (D * MH); }

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace: int64 [batch+1] first chunk of each sequence (the last entry is C),
// then float2 [2W][HS] (max, sum) and float [2W][HS][D] unnormalised outputs, HS =
// MH * GP heads per stream.
struct DecodeWorkspace {
  int64_t* prefix;
  float2* ml;
  float* o;
};
inline DecodeWorkspace carve_decode_workspace(void* ws, int batch, int W, int HS) {
  char* base = static_cast<char*>(ws);
  DecodeWorkspace d;
  d.prefix = reinterpret_cast<int64_t*>(base);
  base += align256(sizeof(int64_t) * (static_cast<size_t>(batch) + 1));
  d.ml = reinterpret_cast<float2*>(base);
  base += align256(sizeof(float2) * 2 * static_cast<size_t>(W) * HS);
  d.o = reinterpret_cast<float*>(base);
  return d;
}
inline size_t decode_workspace_bytes(int batch, int W, int HS, int D) {
  return align256(sizeof(int64_t) * (static_cast<size_t>(batch) + 1)) +
         align256(sizeof(float2) * 2 * static_cast<size_t>(W) * HS) +
         sizeof(float) * 2 * static_cast<size_t>(W) * HS * D;
}

// chunks of 2^ch_log2 tokens in a sequence of length L
__device__ __forceinline__ int chunks_of(int L, int ch_log2) {
  return (max(L, 0) + (1 << ch_log2) - 1) >> ch_log2;
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
hipError_t launch_decode_combine(int head_dim, int GP, int MH, const DecodeWorkspace& ws,
                                 void* out, const int32_t* context_lens, int batch,
                                 int num_q_heads, int num_kv_heads, int num_workers,
                                 hipStream_t stream);

}  // namespace pkv
