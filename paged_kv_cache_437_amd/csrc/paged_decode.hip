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
// Work decomposition.  A "stream" is (sequence, kv head, group of up to GP q heads
// of that kv head); it is cut into chunks of CH tokens.  All chunks of all streams,
// in (sequence, stream, position) order, form one list of C chunks that is divided
// evenly among W independent wavefront workers (worker w takes chunks
// [w*C/W, (w+1)*C/W)), W being as many waves as the device holds resident.  Each
// worker walks its range with two register buffers: the K/V loads of chunk c+1 (and
// the block-table entry of chunk c+2) are issued before chunk c is computed, so HBM
// sees a continuous stream.  K/V are read with non-temporal loads: they are used
// once, and streaming them past the caches is what lets the read approach the HBM
// peak.  The cut depends only on lengths and W, never on block ids.
//
// Per chunk and worker:
//   * K rows go straight from HBM into the B operand of v_mfma_f32_16x16x32_bf16
//     (lane: token lane%16, 8 head_dim elements), the A operand holding the group's
//     q rows (padded to 16), so every grouped q head reuses each K row loaded;
//   * online softmax in the log2 domain (scale * log2 e folded into one multiply):
//     row max across the 16 lanes of a tile row, exp2, per-lane partial sums;
//   * probabilities go through a per-wave LDS tile to the P.V phase, where lanes
//     own (token, 8 head_dim elements) of V rows loaded with 16-byte loads and
//     accumulate on the vector ALU.
// All K/V loads are predicated on token < context_len, so neither table entries past
// the last used block nor the stale tail of the last block is ever read.
//
// A stream whose chunks all fall to one worker is finished by it and written as
// bf16.  A stream cut between workers leaves one fp32 partial (max, sum,
// unnormalised out) per worker in the workspace, and decode_combine merges them
// exactly, in worker order:  M = max_w m_w,
//   out = sum_w 2^(m_w - M) o_w / sum_w 2^(m_w - M) l_w,  rounded once to bf16.
// No atomics: results are bit-identical across runs and block relabellings.
#include <algorithm>
#include <atomic>

#include "decode_plan.h"
#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

// Reductions over the 16 lanes of a row with DPP lane moves (quad swaps, then the
// half-row and row mirrors): every lane of the row ends with the result.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  return x + dpp<0x140>(x);
}
__device__ __forceinline__ float read_lane(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ int64_t read_lane64(int64_t x, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(x), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(x >> 32), lane);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int64_t shfl_up64(int64_t x, int d) {
  const int lo = __shfl_up(static_cast<int>(x), d, 64);
  const int hi = __shfl_up(static_cast<int>(x >> 32), d, 64);
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int lo = __shfl_xor(static_cast<int>(x), o, 64);
    const int hi = __shfl_xor(static_cast<int>(x >> 32), o, 64);
    x += static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
  }
  return x;
}

// K/V rows are read once: non-temporal loads stream them past the caches.
__device__ __forceinline__ u32x4_t load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// Wavefront-uniform base plus a 32-bit per-lane byte offset: one address register
// per lane and the scalar-base form of the load.
__device__ __forceinline__ u32x4_t load_stream(const uint16_t* base, uint32_t byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(base) + byte_off));
}

// Position of a worker in the chunk list; every field is wavefront-uniform.
struct Cursor {
  int b;    // sequence
  int L;    // its context length
  int nch;  // its chunks per stream
  int j;    // stream within the sequence: kv head * n_hg + head group
  int k;    // chunk within the stream
};

// One chunk's operands in registers: K rows as MFMA B operands, V rows as 16-byte
// (token, 8 head_dim elements) pieces, and the stream's q rows as the A operand.
template <int D, int CH>
struct KVBuf {
  u32x4_t k[CH / 16][D / 32];
  u32x4_t v[CH * (D / 8) / 64];
  u32x4_t q[D / 32];
};

}  // namespace

template <int D, int GP, bool ONE_BLOCK>
__global__ __launch_bounds__(256) void paged_decode_bf16_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ block_tables,
    int table_stride, int batch, int Hq, int Hkv, int G, int n_hg, int bs_log2,
    float scale_log2, int num_workers, int64_t* __restrict__ ws_prefix,
    float2* __restrict__ ws_ml, float* __restrict__ ws_o) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(GP == 1 || GP == 2 || GP == 4 || GP == 8, "heads per stream");
  constexpr int CH = kDecodeChunk;
  static_assert(CH == 16 || CH == 32, "chunk");
  constexpr int KK = D / 32;           // MFMA k-steps over head_dim
  constexpr int DCH = D / 8;           // 16-byte pieces per row
  constexpr int TPI = 64 / DCH;        // tokens per V load instruction
  constexpr int VIT = CH / TPI;        // V loads per lane per chunk
  constexpr int T16 = CH / 16;         // 16-token score tiles per chunk
  constexpr int RR = GP < 4 ? GP : 4;  // head rows a lane keeps softmax state for
  typedef KVBuf<D, CH> Buf;

  __shared__ __attribute__((aligned(16))) float p_lds[4][CH][16];

  // wave index through readfirstlane: the compiler then knows everything derived
  // from it (the worker's chunk range and cursor) is wavefront-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int worker = blockIdx.x * 4 + wave;
  if (worker >= num_workers) return;  // wavefront-uniform; the kernel has no block barrier
  const int row = lane & 15;  // MFMA: token column (B) / head row (A)
  const int grp = lane >> 4;  // MFMA: 8-element slice of each 32-wide k-step
  const int v_chunk = lane % DCH;
  const int v_sub = lane / DCH;
  const int S = Hkv * n_hg;
  const int bs_mask = (1 << bs_log2) - 1;
  const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;  // token stride in a block

  // ---- the chunk list: its length, then this worker's first sequence.  Worker 0
  // also records every sequence's first chunk for the combine kernel.
  int64_t tot = 0;
  for (int b0 = 0; b0 < batch; b0 += 64)
    if (b0 + lane < batch) tot += static_cast<int64_t>(chunks_of(context_lens[b0 + lane])) * S;
  const int64_t C = read_lane64(wave_sum64(tot), 0);
  const int64_t W = num_workers;
  const int64_t c_begin = worker * C / W;
  const int64_t c_end = (worker + 1) * C / W;
  int b_first = -1;
  int64_t p_first = 0;
  {
    int64_t carry = 0;
    for (int b0 = 0; b0 < batch; b0 += 64) {
      const int b = b0 + lane;
      const int64_t n = b < batch ? static_cast<int64_t>(chunks_of(context_lens[b])) * S : 0;
      int64_t incl = n;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t t = shfl_up64(incl, o);
        if (lane >= o) incl += t;
      }
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
  cur.nch = chunks_of(cur.L);
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
          x.nch = chunks_of(x.L);
        } while (x.nch == 0);
      }
    }
  };
  // Block id of this lane's token of the chunk (a vector load, so its wait counts in
  // order with the K/V loads); with ONE_BLOCK every lane gets the same id.
  auto table_entry = [&](const Cursor& x) -> int {
    const int tok = min(x.k * CH + (lane & (CH - 1)), x.L - 1);
    return block_tables[static_cast<int64_t>(x.b) * table_stride + (tok >> bs_log2)];
  };
  // Every load of a chunk is issued without a condition, so the compiler's waits
  // count them in order: rows past the context re-read the chunk's last valid row
  // (real data, never stale memory; their scores are masked and their V rows get
  // weight 0), q rows past the stream's heads re-read its first row (zeroed when
  // used), and a `live` == false chunk (the one after a worker's last) reads one row.
  auto issue = [&](const Cursor& x, int te, Buf& buf, bool live) {
    const int kvh = n_hg == 1 ? x.j : x.j / n_hg;
    const int hg = x.j - kvh * n_hg;
    const int tok0 = x.k * CH;
    const int last = live ? min(x.L - tok0, CH) - 1 : 0;  // last row read
    {
      const uint16_t* qb = q + (static_cast<int64_t>(x.b) * Hq + kvh * G + hg * GP) * D;
      const int qrow = (live && row < min(GP, G - hg * GP)) ? row : 0;
      const uint32_t off = static_cast<uint32_t>(qrow * D + grp * 8) * 2;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        buf.q[kk] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(qb) + off +
                                                      kk * 64);
    }
    if constexpr (ONE_BLOCK) {
      // block_size >= CH: the chunk lies in one block, so a uniform base and 32-bit
      // lane offsets address it
      const int64_t blk = __builtin_amdgcn_readfirstlane(te);
      const int64_t first = ((blk << bs_log2) | (tok0 & bs_mask)) * Hkv + kvh;
      const uint16_t* kb = k_cache + first * D;
      const uint16_t* vb = v_cache + first * D;
#pragma unroll
      for (int t4 = 0; t4 < T16; ++t4) {
        const uint32_t off = static_cast<uint32_t>(min(16 * t4 + row, last)) * row_bytes + grp * 16;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) buf.k[t4][kk] = load_stream(kb, off + kk * 64);
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it)
        buf.v[it] = load_stream(
            vb, static_cast<uint32_t>(min(it * TPI + v_sub, last)) * row_bytes + v_chunk * 16);
    } else {
      // small blocks: lane t holds the block of token tok0 + t
#pragma unroll
      for (int t4 = 0; t4 < T16; ++t4) {
        const int tl = min(16 * t4 + row, last);
        const int64_t off =
            token_row(__shfl(te, tl, 64), tok0 + tl, bs_log2, Hkv, kvh, D) + grp * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) buf.k[t4][kk] = load_stream(k_cache + off + kk * 32);
      }
#pragma unroll
      for (int it = 0; it < VIT; ++it) {
        const int tl = min(it * TPI + v_sub, last);
        buf.v[it] = load_stream(
            v_cache + token_row(__shfl(te, tl, 64), tok0 + tl, bs_log2, Hkv, kvh, D) +
            v_chunk * 8);
      }
    }
  };

  // running softmax state of the current segment: rows r = head 4*grp + r
  float m_r[RR], l_r[RR];
  float o[GP][8];
  auto reset = [&]() {
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      m_r[r] = -INFINITY;
      l_r[r] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  };
  reset();
  bool first_segment = true;  // the worker's first segment takes partial slot 2w
  int seg_k0 = cur.k;         // chunk at which the current segment started

  // one chunk into the running state (no memory writes besides the wave's LDS tile)
  auto accumulate = [&](const Cursor& x, const Buf& buf) {
    const int valid = x.L - x.k * CH;  // tokens of the chunk inside the context
    const int kvh = n_hg == 1 ? x.j : x.j / n_hg;
    const int hg = x.j - kvh * n_hg;
    const int nh = min(GP, G - hg * GP);
    // ---- scores: S[head 4*grp + r][token 16*t4 + row] in acc[t4][r]
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    f32x4_t acc[T16];
#pragma unroll
    for (int t4 = 0; t4 < T16; ++t4) {
      acc[t4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        acc[t4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, row < nh ? buf.q[kk] : zero),
            __builtin_bit_cast(bf16x8_t, buf.k[t4][kk]), acc[t4], 0, 0, 0);
    }
    // ---- online softmax (log2 domain), per head row
    float alpha_r[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      float mx = -INFINITY;
#pragma unroll
      for (int t4 = 0; t4 < T16; ++t4) {
        const float s = (16 * t4 + row < valid) ? acc[t4][r] * scale_log2 : -INFINITY;
        acc[t4][r] = s;
        mx = fmaxf(mx, s);
      }
      const float m_new = fmaxf(m_r[r], row16_max(mx));  // finite: the chunk's row 0 is valid
      alpha_r[r] = __builtin_amdgcn_exp2f(m_r[r] - m_new);
      float sum = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < T16; ++t4) {
        const float p = __builtin_amdgcn_exp2f(acc[t4][r] - m_new);
        acc[t4][r] = p;
        sum += p;
      }
      l_r[r] = l_r[r] * alpha_r[r] + sum;
      m_r[r] = m_new;
    }
#pragma unroll
    for (int t4 = 0; t4 < T16; ++t4)
      *reinterpret_cast<f32x4_t*>(&p_lds[wave][16 * t4 + row][4 * grp]) = acc[t4];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- rescale and accumulate P.V on the vector ALU
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float a = read_lane(alpha_r[h & 3], 16 * (h >> 2));
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= a;
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int tl = it * TPI + v_sub;
      float p[GP];
      if constexpr (GP >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < GP; h4 += 4) {
          const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&p_lds[wave][tl][h4]);
          p[h4] = pv[0];
          p[h4 + 1] = pv[1];
          p[h4 + 2] = pv[2];
          p[h4 + 3] = pv[3];
        }
      } else {
#pragma unroll
        for (int h = 0; h < GP; ++h) p[h] = p_lds[wave][tl][h];
      }
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_lo(buf.v[it][w]);
        v[2 * w + 1] = bf16_hi(buf.v[it][w]);
      }
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += p[h] * v[e];
    }
    // p_lds[wave] is rewritten by the next chunk: keep these reads before those writes
    __builtin_amdgcn_wave_barrier();
  };

  // End of a segment (x is its last chunk): the final output if the whole stream ran
  // on this worker, else the worker's partial for the combine kernel.
  auto finalize = [&](const Cursor& x) {
    const int kvh = n_hg == 1 ? x.j : x.j / n_hg;
    const int hg = x.j - kvh * n_hg;
    const int nh = min(GP, G - hg * GP);
    // reduce over the lanes sharing a head_dim piece
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float t = o[h][e];
#pragma unroll
        for (int sft = DCH; sft < 64; sft <<= 1) t += __shfl_xor(t, sft, 64);
        o[h][e] = t;
      }
    float l_h[GP], m_h[GP];
#pragma unroll
    for (int r = 0; r < RR; ++r) l_r[r] = row16_sum(l_r[r]);
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      l_h[h] = read_lane(l_r[h & 3], 16 * (h >> 2));
      m_h[h] = read_lane(m_r[h & 3], 16 * (h >> 2));
    }
    const int64_t hq0 = static_cast<int64_t>(x.b) * Hq + kvh * G + hg * GP;
    if (seg_k0 == 0 && x.k == x.nch - 1) {
      // the whole stream ran here: final output
      if (v_sub == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h >= nh) break;
          const float inv = 1.f / l_h[h];
          u32x4_t w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            w[e2] = pack_bf16x2(o[h][2 * e2] * inv, o[h][2 * e2 + 1] * inv);
          *reinterpret_cast<u32x4_t*>(out + (hq0 + h) * D + v_chunk * 8) = w;
        }
      }
    } else {
      const int64_t slot = 2 * static_cast<int64_t>(worker) + (first_segment ? 0 : 1);
      if (v_sub == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          float* dst = ws_o + (slot * GP + h) * D + v_chunk * 8;
          *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[h][0], o[h][1], o[h][2], o[h][3]};
          *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{o[h][4], o[h][5], o[h][6], o[h][7]};
        }
      }
      if (lane < GP) {
        float mm = m_h[0], ll = l_h[0];
#pragma unroll
        for (int h = 1; h < GP; ++h)
          if (lane == h) {
            mm = m_h[h];
            ll = l_h[h];
          }
        ws_ml[slot * GP + lane] = make_float2(mm, ll);
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
  }
}

namespace {

template <int D, int GP, bool ONE_BLOCK>
int auto_workers() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int w = cached[dev].load(std::memory_order_relaxed);
  if (w > 0) return w;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&paged_decode_bf16_kernel<D, GP, ONE_BLOCK>), 256, 0) !=
          hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    cus = 256;
    per_cu = 2;
  }
  w = std::min(kMaxAutoWorkers, cus * per_cu * 4);
  cached[dev].store(w, std::memory_order_relaxed);
  return w;
}

template <int D, int GP, bool ONE_BLOCK>
hipError_t launch_decode(const void* q, void* out, const void* k_cache, const void* v_cache,
                         int num_q_heads, int num_kv_heads, int bs_log2, int batch,
                         const int32_t* context_lens, const int32_t* block_tables,
                         int table_stride, float scale, int num_workers, void* workspace,
                         hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int n_hg = (G + GP - 1) / GP;
  const int S = num_kv_heads * n_hg;
  if (S > 65535) return hipErrorInvalidConfiguration;
  const int W = num_workers > 0 ? num_workers : auto_workers<D, GP, ONE_BLOCK>();
  const DecodeWorkspace ws = carve_decode_workspace(workspace, batch, W, GP);
  const float scale_log2 = scale * kLog2e;
  timing_begin("paged_decode", stream);
  hipLaunchKernelGGL((paged_decode_bf16_kernel<D, GP, ONE_BLOCK>), dim3((W + 3) / 4), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                     static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache),
                     context_lens, block_tables, table_stride, batch, num_q_heads, num_kv_heads,
                     G, n_hg, bs_log2, scale_log2, W, ws.prefix, ws.ml, ws.o);
  timing_end(stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(D, GP, ws, out, context_lens, batch, num_q_heads, num_kv_heads, W,
                               stream);
}

}  // namespace

size_t paged_decode_bf16_workspace(int head_dim, int num_q_heads, int num_kv_heads, int batch,
                                   int num_workers) {
  const int GP = heads_per_stream(num_q_heads / num_kv_heads);
  return decode_workspace_bytes(batch, num_workers > 0 ? num_workers : kMaxAutoWorkers, GP,
                                head_dim);
}

hipError_t launch_paged_decode_bf16(int head_dim, const void* q, void* out, const void* k_cache,
                                    const void* v_cache, int num_q_heads, int num_kv_heads,
                                    int bs_log2, int batch, const int32_t* context_lens,
                                    const int32_t* block_tables, int table_stride, float scale,
                                    int num_workers, void* workspace, hipStream_t stream) {
  // ONE_BLOCK: every 16-token chunk lies in one block (block_size >= 16)
  const int GP = heads_per_stream(num_q_heads / num_kv_heads);
#define PKV_DEC(D_, GP_)                                                                    \
  return bs_log2 >= 4                                                                       \
             ? launch_decode<D_, GP_, true>(q, out, k_cache, v_cache, num_q_heads,          \
                                            num_kv_heads, bs_log2, batch, context_lens,      \
                                            block_tables, table_stride, scale, num_workers,  \
                                            workspace, stream)                               \
             : launch_decode<D_, GP_, false>(q, out, k_cache, v_cache, num_q_heads,         \
                                             num_kv_heads, bs_log2, batch, context_lens,     \
                                             block_tables, table_stride, scale, num_workers, \
                                             workspace, stream)
  if (head_dim == 128) {
    switch (GP) {
      case 1: PKV_DEC(128, 1);
      case 2: PKV_DEC(128, 2);
      case 4: PKV_DEC(128, 4);
      default: PKV_DEC(128, 8);
    }
  }
  switch (GP) {
    case 1: PKV_DEC(64, 1);
    case 2: PKV_DEC(64, 2);
    case 4: PKV_DEC(64, 4);
    default: PKV_DEC(64, 8);
  }
#undef PKV_DEC
}

}  // namespace pkv
