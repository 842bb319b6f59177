// Device-side helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 is the upper half of an IEEE binary32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Rotary position embedding on 8 bf16 elements x (first half of a head row) and
// their partners y (the same elements + head_dim/2), both as 16-byte words, with
// the cosines c and sines s of those elements: x' = x c - y s, y' = y c + x s in fp32,
// each rounded once to bf16 (round to nearest even).
__device__ __forceinline__ void rope8_bf16(uint32_t (&x)[4], uint32_t (&y)[4], const float* c,
                                           const float* s) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
    const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
    const float c0 = c[2 * w], c1 = c[2 * w + 1], s0 = s[2 * w], s1 = s[2 * w + 1];
    x[w] = pack_bf16x2(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
    y[w] = pack_bf16x2(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
  }
}

// Element <-> float for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  typedef float storage;
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  typedef uint16_t storage;
  static __device__ __forceinline__ float load(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
  static __device__ __forceinline__ void store(uint16_t* p, float x) {
    *p = static_cast<uint16_t>(f32_to_bf16_bits(x));
  }
};

// Reductions over a full 64-lane wavefront (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Sum of an int over a full wavefront, returned wavefront-uniform: DPP within each
// row of 16 lanes (quad swaps, half-row and row mirrors), then the four row sums.
__device__ __forceinline__ int wave_sum_uniform(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);  // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Inclusive prefix sum over the wavefront's 64 lanes with DPP moves only (no LDS round
// trips): within each row of 16 lanes by shifts of 1, 2, 4 and 8 (lanes shifted in from
// outside the row read 0), then the last lane of row 0 is added to row 1 and that of
// row 2 to row 3 (row_bcast:15), then the last lane of row 1 to rows 2 and 3
// (row_bcast:31).  Lanes outside the selected rows get the move's old value, 0.
__device__ __forceinline__ int wave_scan_inclusive(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Row of token `pos` of a sequence for kv head `kvh`, as an element offset into a
// [num_blocks][block_size][Hkv][D] cache.  64-bit: large pools exceed 2^31 elements.
__device__ __forceinline__ int64_t token_row(int32_t block, int pos, int bs_log2, int Hkv,
                                             int kvh, int D) {
  const int64_t slot = (static_cast<int64_t>(block) << bs_log2) | (pos & ((1 << bs_log2) - 1));
  return (slot * Hkv + kvh) * D;
}

}  // namespace pkv
