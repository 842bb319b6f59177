// The decode pass as a device function (internal), shared by the decode kernel and
// the mixed prefill + decode kernel.
//
// Paged decode attention, bf16 in / fp32 accumulate, for gfx950.
//
// What is computed (“深入 Nano-vLLM 推理引擎”, "Prefill and Decode": each
// decode step adds one token per sequence; "From Sequences to Blocks": a sequence's
// tokens live in the blocks its table lists): for sequence b and q head h,
//   out[b, h] = softmax_j(scale * q[b, h] . k_j) v_j   over j < context_lens[b],
// with k_j, v_j the rows of kv head h / (Hq / Hkv) found through block_tables[b].
//
// The pass is a stream over HBM: every K/V byte is read once, so the design is about
// keeping loads in flight without gaps, not about arithmetic.
//
// Work decomposition.  A "stream" is (sequence, group of MH adjacent kv heads, group
// of up to GP q heads of each of them); it is cut into chunks of CH tokens.  All
// chunks of all streams, in (sequence, stream, position) order, form one list of C
// chunks that is divided evenly among W independent wavefront workers (worker w
// takes chunks [w*C/W, (w+1)*C/W)).  Each worker walks its range with two register
// buffers: the K/V loads of chunk c+1 (and the block-table entry of chunk c+2) are
// issued before chunk c is computed, so HBM sees a continuous stream.  K/V are read
// with non-temporal loads: they are used once, and streaming them past the caches is
// what lets the read approach the HBM peak.  The cut depends only on lengths and W,
// never on block ids.
//
// Per chunk and worker, K and V are read alike: lane (sub, hh, piece) loads 16 bytes,
// piece `piece` of kv head hh in row `sub` of the instruction, so each load
// instruction covers whole head rows of MH adjacent heads: MH*2*D contiguous bytes of
// each token row it touches (MH is chosen for 512 bytes, the size measured to stream
// best).  Then, on the vector ALU:
//   * scores: per q head, the q piece . K piece (bf16 pair dot products, fp32
//     accumulation), summed over the head row's lanes with DPP moves; every grouped q
//     head reuses each K row loaded;
//   * online softmax in the log2 domain (scale * log2 e folded into one multiply):
//     max over the chunk's rows in-lane and, across the rows one instruction spreads
//     over lanes, with v_permlane16/32_swap; the reference max moves only when a chunk
//     exceeds it by more than 2^8; exp2, rounded to bf16; per-lane shares of the row
//     sum of those rounded values;
//   * P.V: each lane accumulates its rows' weighted V pieces as bf16 pair dot products
//     over two of its rows (fp32 accumulation); the lanes holding one head_dim piece of
//     a head are summed once, at the end of the segment.
// q changes only with the stream, so it is loaded once per segment.
// Rows past context_len are never read: the buffer loads' range check returns zeros
// for them (block_size >= CH), or they re-read the chunk's last valid row (smaller
// blocks), so neither the stale tail of the last block nor a table entry past it is
// ever touched; their scores are masked to -inf.
//
// A stream whose chunks all fall to one worker is finished by it and written as
// bf16.  A stream cut between workers leaves one fp32 partial (max, sum,
// unnormalised out) per worker in the workspace, and decode_combine merges them
// exactly, in worker order:  M = max_w m_w,
//   out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w,  rounded once to bf16.
// No atomics: results are bit-identical across runs and block relabellings.
#pragma once

#include "decode_plan.h"
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

// DPP lane move within rows of 16 lanes (all rows and banks enabled)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// The same move with bound_ctrl set (every lane of these row patterns has a source, so
// the value is the same): in `x + dpp_b(x)` the compiler folds the move into the add
// (v_add_f32_dpp), which it does not do for dpp().
template <int CTRL>
__device__ __forceinline__ float dpp_b(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ int64_t read_lane64(int64_t x, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), lane);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
// One DPP move of a 64-bit value (both halves moved alike; lanes without a source, or
// outside the selected rows, get 0).
template <int CTRL, int ROW_MASK, bool BC>
__device__ __forceinline__ int64_t dpp64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, ROW_MASK, 0xF, BC);
  const uint32_t hi =
      __builtin_amdgcn_update_dpp(0, static_cast<int>(x >> 32), CTRL, ROW_MASK, 0xF, BC);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
// Inclusive prefix sum over the wavefront's 64 lanes with DPP moves only (no LDS round
// trips): within each row of 16 lanes by shifts of 1, 2, 4 and 8, then row 0's last
// lane into row 1 and row 2's into row 3 (row_bcast:15), then row 1's last lane into
// rows 2 and 3 (row_bcast:31).  Lane 63 ends with the wavefront's total.
__device__ __forceinline__ int64_t wave_scan64(int64_t x) {
  x += dpp64<0x111, 0xF, true>(x);   // row_shr:1
  x += dpp64<0x112, 0xF, true>(x);   // row_shr:2
  x += dpp64<0x114, 0xF, true>(x);   // row_shr:4
  x += dpp64<0x118, 0xF, true>(x);   // row_shr:8
  x += dpp64<0x142, 0xA, false>(x);  // row_bcast:15
  x += dpp64<0x143, 0xC, false>(x);  // row_bcast:31
  return x;
}

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format, no
// swizzle), and the cache-policy bit of a non-temporal buffer load.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

// K/V rows are read once: non-temporal loads stream them past the caches.
__device__ __forceinline__ u32x4_t load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// Position of a worker in the chunk list; every field is wavefront-uniform.
struct Cursor {
  int b;    // sequence
  int L;    // its context length
  int nch;  // its chunks per stream
  int j;    // stream within the sequence: kv head group * n_hg + q head group
  int k;    // chunk within the stream
};

// Loads per lane per chunk, for K and for V alike (each one 16 bytes)
constexpr int kChunkLoads = 4;
static_assert(kChunkLoads % 2 == 0, "P.V pairs a lane's tokens");

// (1, 1) in bf16: v_dot2 with it adds a pair of bf16 values into an fp32 sum
constexpr bf16x2_t kPairOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
// lazy rescale: the running max moves only when a chunk exceeds it by more than 2^8
constexpr float kRescaleSlack = 8.f;

// One chunk's operands in registers: this lane's 16-byte pieces of K and V, one per
// load instruction.
struct KVBuf {
  u32x4_t k[kChunkLoads];
  u32x4_t v[kChunkLoads];
};

// The step's new token of every sequence, for a decode that appends it itself:
// k_new / v_new [batch][Hkv][D], and slots[b], the cache slot of position
// context_lens[b] - 1 (where a separate KV write would have put it; -1: not written).
struct DecodeAppend {
  const uint16_t* k_new = nullptr;
  const uint16_t* v_new = nullptr;
  const int32_t* slots = nullptr;
};

// q . k over one 16-byte piece (8 products as 4 bf16 pair dot products, fp32
// accumulation)
__device__ __forceinline__ float dot_piece(u32x4_t a, u32x4_t b) {
  const bf16x8_t x = __builtin_bit_cast(bf16x8_t, a);
  const bf16x8_t y = __builtin_bit_cast(bf16x8_t, b);
  float c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                            __builtin_shufflevector(y, y, 0, 1), 0.f, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                      __builtin_shufflevector(y, y, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                      __builtin_shufflevector(y, y, 4, 5), c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                         __builtin_shufflevector(y, y, 6, 7), c, false);
}

// Sum over the DCH lanes that hold one token's pieces (16 lanes = a DPP row at head_dim
// 128, 8 lanes = half a row at 64); every one of them gets the sum.  FUSED: each step
// one v_add_f32_dpp instead of a DPP move and an add (with the nops between them).
// Identical sums either way.  Fused, the decode with 8 or 16 q heads per kv head ran
// 14-16% faster, 1 or 2 within noise, and 4 (the large lognormal batch) 2-3% slower,
// all with bit-identical outputs; the kernels fuse from 8 q heads per stream up.
template <int DCH, bool FUSED>
__device__ __forceinline__ float piece_sum(float x) {
  if constexpr (FUSED) {
    x += dpp_b<0xB1>(x);
    x += dpp_b<0x4E>(x);
    x += dpp_b<0x141>(x);
    if constexpr (DCH == 16) x += dpp_b<0x140>(x);
  } else {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (DCH == 16) x += dpp<0x140>(x);  // row_mirror
  }
  return x;
}

// Max / sum over the lanes that differ only in the bits from STRIDE up (the rows a
// load instruction spreads over lanes STRIDE apart): DPP row_ror:8 (lanes l and
// l^8), v_permlane16_swap (l^16) and v_permlane32_swap (l^32); no LDS.  STRIDE = 64:
// nothing to reduce.
template <int STRIDE>
__device__ __forceinline__ float sub_max(float x) {
  if constexpr (STRIDE <= 8) x = fmaxf(x, dpp<0x128>(x));  // row_ror:8
  if constexpr (STRIDE <= 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if constexpr (STRIDE <= 32) {
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
  }
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float sub_sum(float x) {
  if constexpr (STRIDE <= 8) x += dpp<0x128>(x);  // row_ror:8
  if constexpr (STRIDE <= 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  if constexpr (STRIDE <= 32) {
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  }
  return x;
}

}  // namespace

// One workgroup (four wavefront workers, wg*4 .. wg*4+3) of the decode pass; the
// kernels that run it give it its index.
template <int D, int GP, int MH, bool ONE_BLOCK, bool ROT, bool APPEND = false>
__device__ __forceinline__ void decode_workgroup(
    int wg, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, int batch, int Hq, int Hkv, int G, int n_hg, int bs_log2,
    float scale_log2, int num_workers, int64_t* __restrict__ ws_prefix,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o, const float* __restrict__ cos_sin,
    int max_position, DecodeAppend app = {}) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(!APPEND || (ONE_BLOCK && !ROT), "appending decode: chunks in one block, no rotary");
  static_assert(GP == 1 || GP == 2 || GP == 4 || GP == 8, "q heads per kv head in a stream");
  constexpr int DCH = D / 8;         // 16-byte pieces per head row
  constexpr int HPI = 64 / DCH;      // head rows per load instruction
  static_assert(MH >= 1 && MH <= HPI && (MH & (MH - 1)) == 0, "kv heads per stream");
  constexpr int TPI = HPI / MH;      // tokens per load instruction
  constexpr int VIT = kChunkLoads;   // K (and V) loads per lane per chunk
  constexpr int CH = VIT * TPI;      // tokens per chunk
  static_assert(CH == chunk_tokens(D, MH), "chunk");
  constexpr int CH_LOG2 = CH == 32 ? 5 : CH == 16 ? 4 : CH == 8 ? 3 : 2;
  constexpr int SUB = DCH * MH;      // lane stride between the tokens of an instruction
  constexpr int HS = MH * GP;        // heads of a stream's partials
  typedef KVBuf Buf;

  // wave index through readfirstlane: the compiler then knows everything derived
  // from it (the worker's chunk range and cursor) is wavefront-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int worker = wg * 4 + wave;
  if (worker >= num_workers) return;  // wavefront-uniform; the kernel has no block barrier
  // lane = (sub * MH + hh) * DCH + piece: 16-byte piece `piece` (head_dim
  // [8*piece, 8*piece+8)) of kv head hh of the stream, token `sub` of the instruction
  const int piece = lane % DCH;
  const int hh = (lane / DCH) % MH;
  const int sub = lane / SUB;
  const int S = (Hkv / MH) * n_hg;
  const int bs_mask = (1 << bs_log2) - 1;
  const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;  // token stride in a block

  // ---- the chunk list: its length, then this worker's first sequence.  Worker 0
  // also records every sequence's first chunk for the combine kernel.
  int64_t tot = 0;
  for (int b0 = 0; b0 < batch; b0 += 64)
    if (b0 + lane < batch) tot += static_cast<int64_t>(chunks_of(context_lens[b0 + lane], CH_LOG2)) * S;
  const int64_t C = read_lane64(wave_scan64(tot), 63);
  const int64_t W = num_workers;
  const int64_t c_begin = worker * C / W;
  const int64_t c_end = (worker + 1) * C / W;
  int b_first = -1;
  int64_t p_first = 0;
  {
    int64_t carry = 0;
    for (int b0 = 0; b0 < batch; b0 += 64) {
      const int b = b0 + lane;
      const int64_t n = b < batch ? static_cast<int64_t>(chunks_of(context_lens[b], CH_LOG2)) * S : 0;
      const int64_t incl = wave_scan64(n);
      const int64_t excl = carry + incl - n;
      if (worker == 0 && b < batch) ws_prefix[b] = excl;
      if (b_first < 0) {
        const uint64_t hit = __ballot(n > 0 && excl <= c_begin && c_begin < excl + n);
        if (hit) {
          const int ln = __builtin_ctzll(hit);
          b_first = b0 + ln;
          p_first = read_lane64(excl, ln);
        }
      }
      carry += read_lane64(incl, 63);
      if (worker != 0 && b_first >= 0) break;
    }
    if (worker == 0 && lane == 0) ws_prefix[batch] = C;
  }
  if (c_begin >= c_end) return;

  Cursor cur;
  cur.b = b_first;
  cur.L = context_lens[b_first];
  cur.nch = chunks_of(cur.L, CH_LOG2);
  {
    const int64_t r = c_begin - p_first;
    cur.j = static_cast<int>(r / cur.nch);
    cur.k = static_cast<int>(r - static_cast<int64_t>(cur.j) * cur.nch);
  }
  auto advance = [&](Cursor& x) {
    if (++x.k == x.nch) {
      x.k = 0;
      if (++x.j == S) {
        x.j = 0;
        do {  // the list holds a later chunk, so a sequence with chunks follows
          ++x.b;
          x.L = context_lens[x.b];
          x.nch = chunks_of(x.L, CH_LOG2);
        } while (x.nch == 0);
      }
    }
  };
  // Block id of the chunk's rows.  With ONE_BLOCK the chunk lies in one block, so the
  // address is wavefront-uniform (a scalar load); otherwise lane t < CH gets the block
  // of row t (clamped to the context: table entries past the last used block are
  // never read).
  auto table_entry = [&](const Cursor& x) -> int {
    if constexpr (ONE_BLOCK)
      return block_tables[static_cast<int64_t>(x.b) * table_stride + ((x.k * CH) >> bs_log2)];
    const int tok = min(x.k * CH + (lane & (CH - 1)), x.L - 1);
    return block_tables[static_cast<int64_t>(x.b) * table_stride + (tok >> bs_log2)];
  };
  // Lane (sub, hh, piece) reads piece `piece` of kv head hh of the stream in rows
  // it*TPI + sub: each load instruction covers TPI rows of MH heads, 1 KB of
  // contiguous row bytes when MH = HPI.  Every load of a chunk is issued without a
  // condition, so the compiler's waits count them in order.  With ONE_BLOCK the chunk
  // lies in one block and K, V (and q) are read with buffer loads: a wavefront-uniform
  // descriptor (base = the stream's first head in the chunk's first row) plus the
  // loop-invariant 32-bit lane offsets `kv_off`, so issuing writes no vector register
  // but the load destinations (a vector temporary there would make the compiler wait
  // for loads still in flight).  The descriptor's size ends with the context's last
  // row: rows past it (the stale tail of the last block) come back as zeros without a
  // memory access.  Without ONE_BLOCK a chunk spans several blocks: rows past the
  // context re-read the chunk's last valid row (their weight is exactly 0).  A `live`
  // == false chunk (the one after a worker's last) repeats the worker's last chunk.
  uint32_t kv_off[VIT];
#pragma unroll
  for (int it = 0; it < VIT; ++it)
    kv_off[it] = static_cast<uint32_t>(it * TPI + sub) * row_bytes + hh * D * 2 + piece * 16;
  const uint32_t q_off = static_cast<uint32_t>(hh * G * D * 2 + piece * 16);
  // this lane's piece of kv head kv0 + hh in a row of k_new / v_new
  const uint32_t kn_off = static_cast<uint32_t>(hh * D * 2 + piece * 16);
  // this lane's pieces of the q rows of x's stream (kv head hh, q heads g < GP; rows
  // past the group's heads re-read its last one, and those heads are never written
  // out).  Loaded once per segment, in order between the loads of its first chunk
  // and those of the chunk after, so the wait for them is the wait for that chunk.
  u32x4_t qv[GP];
  u32x4_t kn, vn;  // appending decode: this lane's pieces of the stream's new token
  auto load_q = [&](const Cursor& x) {
    const int kvg = n_hg == 1 ? x.j : x.j / n_hg;
    const int hg = x.j - kvg * n_hg;
    const int nh = min(GP, G - hg * GP);
    const int qrow0 = kvg * MH * G + hg * GP;  // this lane's q rows: qrow0 + hh*G + g
    if constexpr (APPEND) {
      // the stream's new token (its kv heads' rows of k_new / v_new), with q: once per
      // segment, used by the stream's last chunk and written out at its end
      const int64_t nrow = (static_cast<int64_t>(x.b) * Hkv + kvg * MH) * D;
      const auto knr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(app.k_new + nrow),
                                                         0, MH * D * 2, kBufferWord3);
      const auto vnr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(app.v_new + nrow),
                                                         0, MH * D * 2, kBufferWord3);
      kn = __builtin_amdgcn_raw_buffer_load_b128(knr, kn_off, 0, 0);
      vn = __builtin_amdgcn_raw_buffer_load_b128(vnr, kn_off, 0, 0);
    }
    if constexpr (ONE_BLOCK) {
      const auto qr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(q + static_cast<int64_t>(x.b) * Hq * D), 0, Hq * D * 2,
          kBufferWord3);
#pragma unroll
      for (int g = 0; g < GP; ++g)
        qv[g] = __builtin_amdgcn_raw_buffer_load_b128(qr, q_off, (qrow0 + min(g, nh - 1)) * D * 2,
                                                      0);
    } else {
      const uint16_t* qb = q + (static_cast<int64_t>(x.b) * Hq + qrow0 + hh * G) * D + piece * 8;
#pragma unroll
      for (int g = 0; g < GP; ++g)
        qv[g] = *reinterpret_cast<const u32x4_t*>(qb + min(g, nh - 1) * D);
    }
    if constexpr (ROT) {
      // rotary position embedding of the query at the context's last position: this
      // lane's 8 elements pair with the lane DCH/2 away (the other half of the head
      // row); x' = x c - y s in the first half, y' = y c + x s in the second, in fp32
      const int pos = min(max(x.L - 1, 0), max_position - 1);
      const float* cs = cos_sin + static_cast<int64_t>(pos) * D + (piece & (DCH / 2 - 1)) * 8;
      const float sgn = piece < DCH / 2 ? -1.f : 1.f;
      float c[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c[e] = cs[e];
        sn[e] = sgn * cs[D / 2 + e];
      }
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t own = qv[g][w];
          const uint32_t other =
              static_cast<uint32_t>(__shfl_xor(static_cast<int>(own), DCH / 2, 64));
          qv[g][w] = pack_bf16x2(bf16_lo(own) * c[2 * w] + bf16_lo(other) * sn[2 * w],
                                 bf16_hi(own) * c[2 * w + 1] + bf16_hi(other) * sn[2 * w + 1]);
        }
    }
  };
  auto issue = [&](const Cursor& x, int te, Buf& buf, bool live) {
    const int kv0 = (n_hg == 1 ? x.j : x.j / n_hg) * MH;  // the stream's first kv head
    const int tok0 = x.k * CH;
    if constexpr (ONE_BLOCK) {
      (void)live;
      const int64_t blk = __builtin_amdgcn_readfirstlane(te);
      const int64_t first = ((blk << bs_log2) | (tok0 & bs_mask)) * Hkv + kv0;
      // an appending decode takes the stream's last row (the new token) from k_new /
      // v_new: the descriptor of its last chunk ends before that row
      const bool new_row = APPEND && x.k == x.nch - 1;
      const int bytes = (min(x.L - tok0, CH) - 1) * static_cast<int>(row_bytes) +
                        (new_row ? 0 : MH * D * 2);
      const auto kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(k_cache + first * D), 0, bytes, kBufferWord3);
      const auto vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(v_cache + first * D), 0, bytes, kBufferWord3);
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        buf.k[it] = __builtin_amdgcn_raw_buffer_load_b128(kr, kv_off[it], 0, kNonTemporal);
        buf.v[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, kv_off[it], 0, kNonTemporal);
      }
    } else {
      const int last = live ? min(x.L - tok0, CH) - 1 : 0;  // last row read
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int tl = min(it * TPI + sub, last);
        const int64_t off =
            token_row(__shfl(te, tl, 64), tok0 + tl, bs_log2, Hkv, kv0 + hh, D) + piece * 8;
        buf.k[it] = load_stream(k_cache + off);
        buf.v[it] = load_stream(v_cache + off);
      }
    }
  };

  // Running softmax state of the current segment, per q head g of this lane's kv head:
  // the max m (log2 domain, the same in every lane of the kv head), this lane's share
  // of the sum (its rows' weights; the lanes of one row hold equal shares) and of the
  // unnormalised output (its rows, head_dim [8*piece, 8*piece+8)).
  float m[GP], l[GP], o[GP][8];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }
  };
  reset();
  bool first_segment = true;  // the worker's first segment takes partial slot 2w
  int seg_k0 = cur.k;         // chunk at which the current segment started

  // one chunk into the running state (registers only: no memory access).  The
  // probabilities are rounded to bf16 once; P.V pairs this lane's tokens (same
  // head_dim elements, tokens it and it+1) into bf16 dot products, and the sum takes the
  // same rounded values.  The reference max a head's probabilities are taken against
  // moves only when a chunk's max exceeds it by more than 2^8 (log2 domain), so most
  // chunks skip the rescale of the running output; probabilities stay <= 2^8.
  auto accumulate = [&](const Cursor& x, const Buf& buf) {
    const int valid = x.L - x.k * CH;  // rows of the chunk inside the context
    bf16x2_t pk[GP][VIT / 2];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      // scores of this lane's rows: the piece's dot product summed over the row's lanes
      float s[VIT];
      float mx = -INFINITY;
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const float d = piece_sum<DCH, (GP >= 8)>(dot_piece(qv[h], buf.k[it]));
        s[it] = (it * TPI + sub < valid) ? d * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[it]);
      }
      // the chunk's row 0 is valid, so its max is finite
      mx = sub_max<SUB>(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m[h] + kRescaleSlack)) {  // wavefront-uniform
        const float m_new = fmaxf(m[h], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] *= alpha;
      }
#pragma unroll
      for (int t2 = 0; t2 < VIT / 2; ++t2) {
        pk[h][t2] = {static_cast<__bf16>(__builtin_amdgcn_exp2f(s[2 * t2] - m[h])),
                     static_cast<__bf16>(__builtin_amdgcn_exp2f(s[2 * t2 + 1] - m[h]))};
        l[h] = __builtin_amdgcn_fdot2_f32_bf16(pk[h][t2], kPairOnes, l[h], false);
      }
    }
    // P.V: element pairs (token it, token it+1) of each 32-bit word of V, by byte
    // permutes, against (p_it, p_it+1) of every head
#pragma unroll
    for (int t2 = 0; t2 < VIT / 2; ++t2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = buf.v[2 * t2][w], b = buf.v[2 * t2 + 1][w];
        const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b, a, 0x05040100u));
        const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(b, a, 0x07060302u));
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          o[h][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(lo, pk[h][t2], o[h][2 * w], false);
          o[h][2 * w + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, pk[h][t2], o[h][2 * w + 1], false);
        }
      }
    }
  };

  // End of a segment (x is its last chunk): the final output if the whole stream ran
  // on this worker, else the worker's partial for the combine kernel.
  auto finalize = [&](const Cursor& x) {
    const int kvg = n_hg == 1 ? x.j : x.j / n_hg;
    const int hg = x.j - kvg * n_hg;
    const int nh = min(GP, G - hg * GP);
    if constexpr (APPEND) {
      // the stream's last chunk ran here: its first q-head group writes the new token's
      // rows of these kv heads into the cache (no chunk of this launch reads them)
      if (x.k == x.nch - 1 && hg == 0) {
        const int32_t slot = app.slots[x.b];
        if (slot >= 0 && sub == 0) {
          const int64_t row = (static_cast<int64_t>(slot) * Hkv + kvg * MH + hh) * D + piece * 8;
          *reinterpret_cast<u32x4_t*>(const_cast<uint16_t*>(k_cache) + row) = kn;
          *reinterpret_cast<u32x4_t*>(const_cast<uint16_t*>(v_cache) + row) = vn;
        }
      }
    }
    // sum the shares of the lanes holding the same head and head_dim piece
    float l_h[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      l_h[h] = sub_sum<SUB>(l[h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = sub_sum<SUB>(o[h][e]);
    }
    if (seg_k0 == 0 && x.k == x.nch - 1) {
      // the whole stream ran here: final output
      if (sub == 0) {
        const int64_t row0 = static_cast<int64_t>(x.b) * Hq + (kvg * MH + hh) * G + hg * GP;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h >= nh) break;
          const float inv = 1.f / l_h[h];
          u32x4_t w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            w[e2] = pack_bf16x2(o[h][2 * e2] * inv, o[h][2 * e2 + 1] * inv);
          *reinterpret_cast<u32x4_t*>(out + (row0 + h) * D + piece * 8) = w;
        }
      }
    } else {
      const int64_t slot = 2 * static_cast<int64_t>(worker) + (first_segment ? 0 : 1);
      if (sub == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          float* dst = ws_o + (slot * HS + hh * GP + h) * D + piece * 8;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[h][0], o[h][1], o[h][2], o[h][3]};
          *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{o[h][4], o[h][5], o[h][6], o[h][7]};
        }
        if (piece == 0) {
#pragma unroll
          for (int h = 0; h < GP; ++h) ws_ml[slot * HS + hh * GP + h] = make_float2(m[h], l_h[h]);
        }
      }
    }
    reset();
    first_segment = false;
  };

  // ---- the pipelined walk: chunk i computes while chunk i+1 loads and the table
  // entry of chunk i+2 is fetched.  The chunk after the worker's last is a dummy.
  // The inner loop runs the chunks of one segment and holds no global store (a store
  // there would make the next chunk's register reuse wait for every load in flight);
  // segment ends are finalized in the outer loop.  32-bit counters: a 64-bit compare
  // of uniform values would borrow a vector register and wait the same way.
  const int n_chunks = static_cast<int>(c_end - c_begin);
  Buf bufA, bufB;
  int i = 0;
  Cursor nxt = cur;
  if (n_chunks > 1) advance(nxt);
  int te_nxt = table_entry(nxt);
  issue(cur, table_entry(cur), bufA, true);
  load_q(cur);
  bool has_next = false;
  Cursor nn = nxt;
  int te_nn = 0;
  // Process `cur` from X after issuing `nxt` into Y; true at a segment end (the
  // cursors then advance after the finalize).
  auto step = [&](Buf& X, Buf& Y) -> bool {
    has_next = i + 1 < n_chunks;
    nn = nxt;
    if (i + 2 < n_chunks) advance(nn);
    te_nn = table_entry(nn);
    issue(nxt, te_nxt, Y, has_next);
    // keep those loads here, ahead of the computation of the current chunk
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (APPEND) {
      // a stream's last chunk: the context's last row is the new token, whose pieces
      // come from k_new / v_new (the chunk's descriptor ends before that row).  X is
      // this half-step's own buffer, so the substitution is in place.
      if (cur.k == cur.nch - 1) {
        const int valid = cur.L - cur.k * CH;
#pragma unroll
        for (int it = 0; it < VIT; ++it)
          if (it * TPI + sub == valid - 1) {
            X.k[it] = kn;
            X.v[it] = vn;
          }
      }
    }
    accumulate(cur, X);
    if (!has_next || cur.k == cur.nch - 1) return true;
    ++i;
    cur = nxt;
    nxt = nn;
    te_nxt = te_nn;
    return false;
  };
  // The two half-steps appear once each; a segment that starts with its chunk in
  // bufB enters the loop at the second one.
  bool start_in_b = false;
  for (;;) {
    bool ended_in_a;
    for (;;) {
      if (!start_in_b && step(bufA, bufB)) {
        ended_in_a = true;
        break;
      }
      start_in_b = false;
      if (step(bufB, bufA)) {
        ended_in_a = false;
        break;
      }
    }
    finalize(cur);
    if (!has_next) break;
    start_in_b = ended_in_a;  // the next chunk sits in the other buffer
    ++i;
    cur = nxt;
    nxt = nn;
    te_nxt = te_nn;
    seg_k0 = 0;
    load_q(cur);  // a new segment is a new stream
  }
}

}  // namespace pkv
