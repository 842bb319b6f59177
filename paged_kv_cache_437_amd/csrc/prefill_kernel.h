// The prefill pass as a device function (internal), shared by the prefill kernel and
// the mixed prefill + decode kernel.
//
// Paged varlen causal prefill, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// What is computed (“深入 Nano-vLLM 推理引擎”, "Preparing for computation":
// prefill packs sequences and addresses them by cumulative lengths; "Prefix Caching
// by hashing": a cached prefix is read from its shared blocks, not recomputed):
// sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 (Lq of them) and Lk keys read
// through block_tables[b]; query i sits at position Lk - Lq + i and
//   out = softmax_j(scale * q . k_j) v_j   over keys j <= Lk - Lq + i.
//
// Tiling.  A workgroup (4 wavefronts) owns 128 query rows = all the q heads of one
// kv head over a tile of 128/GP tokens (GP = q heads per kv head rounded up to a
// power of two), so every K/V tile staged in LDS serves all grouped heads.  Each
// wave owns 32 rows (one head, consecutive tokens when GP <= 4).  Per 64-key tile:
//   S^T (keys x rows) = K Q^T    with v_mfma_f32_32x32x16_bf16, A = K rows from LDS
//                                (16-byte reads), B = the wave's q rows held in VGPRs;
//   online softmax in the log2 domain: each lane owns one query row (16 of the 32
//                                keys of each 32-key block; the other 16 are in lane
//                                l^32), so a row max is a local max plus one swap;
//   O^T (d x rows) += V^T P^T    A = V^T built with ds_read_tr16_b64 from the
//                                row-major V tile, B = P converted to bf16 in place.
// The key order inside each MFMA k-step is the same permutation for both operands,
// so the P registers produced by the S^T MFMA feed the O^T MFMA without shuffles.
// K/V tiles are double buffered in LDS and land there straight from global memory
// (16-byte direct-to-LDS loads: no register staging, no LDS write instructions);
// tile j+1 is in flight while tile j is computed.  The tiles are unpadded, with a
// 16-byte chunk swizzle that keeps both operand reads free of bank conflicts.  Keys
// at or past Lk re-read the tile's last valid key (stale rows never enter; their
// scores are masked), table entries past the last used block are never read, and
// causal masking is applied only on tiles that cross the diagonal.  The output rows go
// out through LDS: a lane holds 16-byte pieces of one row spread over head_dim, so each
// wave stages its 32 rows in a free K/V buffer and stores them whole.
// Work order: workgroups take the (sequence, kv head, q tile) items by level, the q
// tile's distance from the end of the longest prompt, in groups of 4 levels, so the
// longest causal tiles start first, the shortest run last, and the tiles of one
// sequence that share a K/V prefix run together; the grid is sized for the longest
// sequence and the slots past the real
// items (shorter sequences have fewer tiles) come last and exit at once.  When the kv
// heads divide into eight groups, workgroup w takes its items from kv heads
// congruent to w mod 8 only: workgroups are dispatched to the eight XCDs in turn, so
// every K/V tile of a kv head is read through one XCD's L2, where the other q tiles
// of its sequence find it again.
#pragma once

#include "device.h"
#include "launch.h"
#include "timing.h"

namespace pkv {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// (1, 1) in bf16: v_dot2 with it adds a pair of bf16 values into an fp32 sum
constexpr bf16x2_t kOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

// The pointer is cast to the LDS address space directly (not through an integer), so
// the compiler sees the __shared__ object plus an offset and folds constant offsets
// into the instruction's immediate field instead of keeping one address per offset.
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)((const __attribute__((address_space(3))) char*)p));
}

// Bounds of a sequence: its first query row, its query and key counts, and the first
// entry of its block table.
struct SeqBounds {
  int q_begin, Lq, Lk, blk0;
};

// Workgroup -> work item.  Q tile j of a sequence (j from 0 at its first query) sits at
// level u = max_tiles - 1 - j, so the last (heaviest) tiles of the longest prompts come
// first and tile 0 of every prompt last: in a causal prompt the tiles of one level need
// the same number of K/V tiles, and the order is longest-first up to the group size.
// Levels are taken in groups of R: group Y holds levels Y R .. Y R + R - 1 of every
// sequence, groups in order, and inside a group the items go by (sequence, kv head,
// level), so the tiles of one sequence and kv head that share a group run side by side
// and read the same K/V prefix together.  Against groups of 16 ranks counted from each
// sequence's last tile (the earlier order), per launch: varlen prefill 4-8% faster,
// prefix-cached and long prompts within noise; outputs bit-identical.  With n_b q tiles
// in sequence b (levels max_tiles - n_b .. max_tiles - 1), the groups below Y hold
// P(Y R) = Hkv * sum_b clamp(Y R - (max_tiles - n_b), 0, n_b) items: a binary search on
// P finds the group, a wavefront scan the sequence.  Returns false for i past the list,
// else the item and its sequence's bounds.  Every value is wavefront-uniform.
template <int R>
__device__ bool prefill_item(int64_t i, int batch, int Hkv, int bm_tok, int max_tiles,
                             const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                             const int32_t* __restrict__ block_tables, int table_stride,
                             int& b_out, int& kvh_out, int& tile_out, SeqBounds& sb) {
  constexpr int NC = 4;  // chunks of 64 sequences whose tile counts stay in registers
  const int lane = threadIdx.x & 63;
  auto load_tiles = [&](int b) -> int {
    return b < batch ? (cu_q[b + 1] - cu_q[b] + bm_tok - 1) / bm_tok : 0;
  };
  // the first 64 sequences' bounds and first table entries are loaded with their tile
  // counts, so when the item's sequence is one of them its bounds need no load after
  // the search (one dependent round trip fewer before the item's first K/V tile)
  int cq0 = 0, cq1 = 0, ck0 = 0, ck1 = 0, tb0 = 0;
  if (lane < batch) {
    cq0 = cu_q[lane];
    cq1 = cu_q[lane + 1];
    ck0 = cu_k[lane];
    ck1 = cu_k[lane + 1];
    if (table_stride > 0) tb0 = block_tables[static_cast<int64_t>(lane) * table_stride];
  }
  // the other chunks' bounds: every load first (a lane past the batch reads the last
  // sequence's), then the counts, so the loads overlap instead of waiting in turn
  int qa[NC], qz[NC];
#pragma unroll
  for (int c = 1; c < NC; ++c) {
    qa[c] = qz[c] = 0;
    if (64 * c < batch) {  // wavefront-uniform
      const int bc = min(64 * c + lane, batch - 1);
      qa[c] = cu_q[bc];
      qz[c] = cu_q[bc + 1];
    }
  }
  int nreg[NC];
  nreg[0] = (cq1 - cq0 + bm_tok - 1) / bm_tok;  // 0 past the batch
#pragma unroll
  for (int c = 1; c < NC; ++c)
    nreg[c] = 64 * c + lane < batch ? (qz[c] - qa[c] + bm_tok - 1) / bm_tok : 0;
  auto tiles_of = [&](int c) -> int {  // this lane's sequence of chunk c
    if (c < NC) {
      int n = nreg[0];
#pragma unroll
      for (int cc = 1; cc < NC; ++cc)
        if (c == cc) n = nreg[cc];
      return n;
    }
    return load_tiles(64 * c + lane);
  };
  const int n_chunks = (batch + 63) / 64;
  // a sequence of n q tiles has min(max(y - (max_tiles - n), 0), n) of them below level y
  auto below = [&](int n, int y) { return min(max(y - (max_tiles - n), 0), n); };
  auto items_below = [&](int y) -> int64_t {  // P(y)
    int part = 0;
    for (int c = 0; c < n_chunks; ++c) part += below(tiles_of(c), y);
    return static_cast<int64_t>(wave_sum_uniform(part)) * Hkv;
  };
  if (i >= items_below(max_tiles)) return false;
  int lo = 0, hi = (max_tiles + R - 1) / R;  // P(lo R) <= i < P(hi R)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (items_below(mid * R) <= i) lo = mid; else hi = mid;
  }
  const int y0 = lo * R;
  int64_t r = i - items_below(y0);
  for (int c = 0; c < n_chunks; ++c) {
    const int n = tiles_of(c);
    const int cnt = below(n, y0 + R) - below(n, y0);  // this sequence's levels in the group
    const int w = cnt * Hkv;                 // and its items there
    const int incl = wave_scan_inclusive(w);  // inclusive scan over the wavefront
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (r < total) {
      // the first lane whose inclusive count passes r has w > 0: a real sequence
      const int ln = __builtin_ctzll(__ballot(incl > r));
      const int cnt_b = __builtin_amdgcn_readlane(cnt, ln);
      const int rr = static_cast<int>(r) - (__builtin_amdgcn_readlane(incl, ln) -
                                            __builtin_amdgcn_readlane(w, ln));
      kvh_out = rr / cnt_b;
      const int b = 64 * c + ln;
      b_out = b;
      const int n_b = __builtin_amdgcn_readlane(n, ln);
      tile_out = max_tiles - 1 - (max(y0, max_tiles - n_b) + (rr - kvh_out * cnt_b));
      if (c == 0) {
        sb.q_begin = __builtin_amdgcn_readlane(cq0, ln);
        sb.Lq = __builtin_amdgcn_readlane(cq1, ln) - sb.q_begin;
        sb.Lk = __builtin_amdgcn_readlane(ck1, ln) - __builtin_amdgcn_readlane(ck0, ln);
        sb.blk0 = __builtin_amdgcn_readlane(tb0, ln);
      } else {
        sb.q_begin = cu_q[b];
        sb.Lq = cu_q[b + 1] - sb.q_begin;
        sb.Lk = cu_k[b + 1] - cu_k[b];
        sb.blk0 = block_tables[static_cast<int64_t>(b) * table_stride];
      }
      return true;
    }
    r -= total;
  }
  return false;  // not reached for i inside the list
}

// 16-byte chunk swizzle of the unpadded LDS K/V tiles (64 banks of 4 bytes: a 256-byte
// bank line): logical chunk c of row r sits at physical chunk c ^ swz<D>(r).  It puts
// the 16 rows that the 16 lanes of one ds_read_b128 cycle read (the K operand, one
// logical chunk) on 16 distinct chunk slots of the bank line, and the 4 rows x 64 bytes
// that 32 lanes of one transposing-read cycle take (the V operand) on disjoint slots.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

typedef __attribute__((address_space(3))) char lds_char;

// 16 bytes per lane from global memory straight into LDS: lane l's 16 bytes land at
// LDS byte lds + 16 l (global_load_lds_dwordx4; the compiler sets the LDS base in m0
// itself).  Each wave orders these writes against the other waves' LDS reads
// explicitly: vmcnt(0) and a barrier before a tile is read, and a buffer is refilled
// only after every wave is done with it.
typedef __attribute__((address_space(1))) const void global_cvoid;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_char*)p));
}
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  __builtin_amdgcn_global_load_lds((global_cvoid*)(sbase + voff),
                                   (lds_void*)static_cast<uintptr_t>(lds), 16, 0, 0);
}
__device__ __forceinline__ void dma16_ptr(const void* p, uint32_t lds) {
  __builtin_amdgcn_global_load_lds((global_cvoid*)p, (lds_void*)static_cast<uintptr_t>(lds), 16,
                                   0, 0);
}

// One workgroup (one work item of the list) of the prefill pass; the kernels that run
// it give it its index.
constexpr int kXcds = 8;  // XCDs of the part; workgroups are dispatched to them in turn
constexpr int kLevelGroup = 4;  // q-tile levels per group of the work order

template <int D, int GP, bool BIG_BLOCK, bool ROT>
__device__ __forceinline__ void prefill_workgroup(
    int wg, const uint16_t* __restrict__ q, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ cu_seqlens_k,
    const int32_t* __restrict__ block_tables, int table_stride, int Hq, int Hkv, int G,
    int bs_log2, float scale_log2, int batch, int max_tiles, const float* __restrict__ cos_sin,
    int max_position) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int BM_TOK = 128 / GP;  // tokens per workgroup tile
  constexpr int BN = 64;            // keys per K/V tile
  constexpr int RB = D * 2;         // bytes per LDS row (unpadded)
  constexpr int TB = BN * RB;       // bytes per LDS tile
  constexpr int KS = D / 16;        // S^T MFMA k-steps over head_dim
  constexpr int DT = D / 32;        // O^T tiles of 32 head_dim rows
  constexpr int CPR = D / 8;        // 16-byte chunks per K/V row
  constexpr int RPL = 64 / CPR;     // rows per wavefront load instruction (1 KB)
  constexpr int LIT = BN / (4 * RPL);  // load instructions per wavefront per tile (K and V each)
  // Lazy rescaling: the running max a row's probabilities are taken against moves
  // only when a new score exceeds it by more than 2^8 (log2 domain), so most tiles
  // skip the rescale of the accumulators; probabilities stay <= 2^8.
  constexpr float kRescaleSlack = 8.f;

  // two K and two V tile buffers; the tile loop is unrolled by two so every LDS
  // address is a per-lane base plus an immediate
  __shared__ __attribute__((aligned(1024))) char k_lds0[TB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TB];
  __shared__ __attribute__((aligned(1024))) char kv_lds1[2 * TB];  // second K, then second V
  char* const k_lds1 = kv_lds1;
  char* const v_lds1 = kv_lds1 + TB;

  int b = 0, kvh = 0, tile = 0;
  SeqBounds sb;
  if (Hkv % kXcds == 0) {
    // the list restricted to kv heads kvh = wg % 8 + 8 m, m < Hkv / 8
    if (!prefill_item<kLevelGroup>(wg / kXcds, batch, Hkv / kXcds, BM_TOK, max_tiles,
                                   cu_seqlens_q, cu_seqlens_k, block_tables, table_stride, b,
                                   kvh, tile, sb))
      return;  // past the list: uniform over the workgroup, before any barrier
    kvh = wg % kXcds + kXcds * kvh;
  } else if (!prefill_item<kLevelGroup>(wg, batch, Hkv, BM_TOK, max_tiles, cu_seqlens_q,
                                        cu_seqlens_k, block_tables, table_stride, b, kvh, tile,
                                        sb)) {
    return;
  }
  const int q_begin = sb.q_begin;
  const int Lq = sb.Lq;
  const int Lk = sb.Lk;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int tok0 = tile * BM_TOK;
  const int32_t* table = block_tables + static_cast<int64_t>(b) * table_stride;
  const int bs_mask = (1 << bs_log2) - 1;
  const uint32_t row_bytes = static_cast<uint32_t>(Hkv) * D * 2;  // token stride in a block

  // this lane's query row (rows are head-major: 32 rows of a wave share a head when GP<=4)
  const int R = 32 * wave + l32;
  const int head = R / BM_TOK;
  const int tok = tok0 + (R - head * BM_TOK);
  const bool row_valid = head < G && tok < Lq;
  const int hq = kvh * G + head;
  const int diag = Lk - Lq + tok;  // last visible key of this row (any value is fine if invalid)

  // keys the workgroup needs: up to the diagonal of its last valid token
  const int tok_last = min(tok0 + BM_TOK, Lq) - 1;
  const int k_end = Lk - Lq + tok_last + 1;
  const int n_kv = (k_end + BN - 1) / BN;
  const int first_masked_tile = (Lk - Lq + tok0) / BN;  // tiles before it need no mask

  // ---- global -> LDS loads of one K/V tile, straight into LDS (no register staging).
  // Wavefront instruction i covers LDS rows (4i + wave) * RPL .. + RPL; lane l writes
  // physical chunk l % CPR of row (4i + wave) * RPL + l / CPR and so loads that row's
  // logical chunk (l % CPR) ^ swz(row).  Rows past the last valid key re-read it.
  int ld_row[LIT], ld_chunk[LIT];
#pragma unroll
  for (int i = 0; i < LIT; ++i) {
    ld_row[i] = (4 * i + wave) * RPL + lane / CPR;
    ld_chunk[i] = (lane % CPR) ^ swz<D>(ld_row[i]);
  }
  // block id of tile t (with BIG_BLOCK a 64-key tile lies in one block and every lane
  // gets the same id)
  auto tile_block = [&](int t) -> int {
    return table[min(t * BN + (lane & (BN - 1)), Lk - 1) >> bs_log2];
  };
  auto fetch = [&](int t, int te, char* kl, char* vl) {
    const int kv0 = t * BN;
    const int last = min(Lk - kv0, BN) - 1;
    if constexpr (BIG_BLOCK) {
      const int64_t blk = __builtin_amdgcn_readfirstlane(te);
      const int64_t first = (((blk << bs_log2) | (kv0 & bs_mask)) * Hkv + kvh) * D;
      const char* kb = reinterpret_cast<const char*>(k_cache + first);
      const char* vb = reinterpret_cast<const char*>(v_cache + first);
#pragma unroll
      for (int i = 0; i < LIT; ++i) {
        const uint32_t off =
            static_cast<uint32_t>(min(ld_row[i], last)) * row_bytes + ld_chunk[i] * 16;
        const int lo = (4 * i + wave) * RPL * RB;
        dma16(kb, off, lds_addr(kl + lo));
        dma16(vb, off, lds_addr(vl + lo));
      }
    } else {
      // every row's table entry first, so the loads go out together
      int blk[LIT];
#pragma unroll
      for (int i = 0; i < LIT; ++i) blk[i] = table[(kv0 + min(ld_row[i], last)) >> bs_log2];
#pragma unroll
      for (int i = 0; i < LIT; ++i) {
        const int key = kv0 + min(ld_row[i], last);
        const int64_t off = token_row(blk[i], key, bs_log2, Hkv, kvh, D) + ld_chunk[i] * 8;
        const int lo = (4 * i + wave) * RPL * RB;
        dma16_ptr(k_cache + off, lds_addr(kl + lo));
        dma16_ptr(v_cache + off, lds_addr(vl + lo));
      }
    }
  };

  constexpr int KR = ROT ? KS / 2 : 1;
  constexpr int TROW = D * 4;                              // bytes of one table row
  constexpr bool STAGE = ROT && BM_TOK * TROW <= 2 * TB;  // q tiles of <= 64 tokens
  // With the table staged and blocks of 64 or more keys, the table rows and q go out
  // first and tile 0 after them, so the rotation runs while tile 0 is in flight.
  constexpr bool ROT_AHEAD = STAGE && BIG_BLOCK;

  // tile 0 goes out before the q rows: with blocks of 64 or more keys its block is the
  // table's first entry, loaded with the sequence bounds rather than after them
  int te_next = BIG_BLOCK ? sb.blk0 : 0;
  if constexpr (!ROT_AHEAD) {
    fetch(0, te_next, k_lds0, v_lds0);
    if (BIG_BLOCK && n_kv > 1) te_next = tile_block(1);
  }

  // rotary: cosines and sines of this row's position for the elements this lane holds
  // in k-steps ks < KS/2.  When the item's rows of the table (one per token of its q
  // tile) fit in the second K/V buffers, which are free until tile 1 is fetched, the
  // workgroup lands them there once with coalesced direct-to-LDS loads and every lane
  // reads its values back (the q heads of a tile share the rows); each lane reading its
  // own row from global memory instead touches 32 rows per load instruction.  Row r's
  // 16-byte chunk c sits at chunk c ^ (r % 16), so 16 consecutive rows read one logical
  // chunk from distinct banks.
  f32x4_t rc[KR][2], rs[KR][2];
  auto stage_table = [&]() {
    constexpr int CPT = TROW / 16;          // 16-byte chunks per table row
    constexpr int RPI = 64 / CPT;           // rows per wavefront load instruction
    constexpr int NI = (BM_TOK + RPI - 1) / RPI;
    const int pos0 = Lk - Lq + tok0;        // position of the tile's first token
    for (int i = wave; i < NI; i += 4) {    // wavefront-uniform
      const int r = i * RPI + lane / CPT;
      const int c = (lane % CPT) ^ (r & 15);
      const int64_t pos = min(max(pos0 + r, 0), max_position - 1);
      dma16_ptr(cos_sin + pos * D + 4 * c, lds_addr(k_lds1 + i * RPI * TROW));
    }
  };
  if constexpr (STAGE && !ROT_AHEAD) {
    stage_table();
  } else if constexpr (ROT && !STAGE) {
    const float* cs =
        cos_sin + static_cast<int64_t>(min(max(diag, 0), max_position - 1)) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KR; ++ks)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        rc[ks][h2] = *reinterpret_cast<const f32x4_t*>(cs + ks * 16 + 4 * h2);
        rs[ks][h2] = *reinterpret_cast<const f32x4_t*>(cs + D / 2 + ks * 16 + 4 * h2);
      }
  }

  // q row as the S^T MFMA B operand: lane holds d = ks*16 + 8*hi .. +8
  bf16x8_t qb[KS];
  if constexpr (ROT_AHEAD) {
    // every lane loads a row of the sequence (a lane past it the nearest real row, zeroed
    // once the loads have landed), so no branch around the loads stalls the wave on them
    // before the table rows and tile 0 go out
    const int64_t qrow = static_cast<int64_t>(q_begin + min(tok, Lq - 1)) * Hq + kvh * G +
                         min(head, G - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(q + qrow * D + ks * 16 + 8 * hi));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (row_valid)
        w = *reinterpret_cast<const u32x4_t*>(
            q + (static_cast<int64_t>(q_begin + tok) * Hq + hq) * D + ks * 16 + 8 * hi);
      qb[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  if constexpr (ROT_AHEAD) {
    // q went out first, then the table rows, then tile 0 (the scheduling barriers keep
    // the compiler from moving loads across); the wait leaves tile 0's 2*LIT
    // direct-to-LDS loads in flight: vmcnt counts this wave's memory loads in issue
    // order, so at most 2*LIT outstanding means q and the table rows have landed.  The
    // barrier is the bare instruction: __syncthreads' release fence would wait for
    // tile 0 as well.  The empty asm keeps the compiler from moving the table's LDS
    // reads above it.
    __builtin_amdgcn_sched_barrier(0);
    stage_table();
    __builtin_amdgcn_sched_barrier(0);
    fetch(0, te_next, k_lds0, v_lds0);
    __builtin_amdgcn_sched_barrier(0);
    static_assert(2 * LIT <= 15, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (2 * LIT));  // vmcnt(2*LIT)
    __builtin_amdgcn_s_barrier();  // every wave's table rows have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (n_kv > 1) te_next = tile_block(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, qb[ks]);
      qb[ks] = __builtin_bit_cast(bf16x8_t, row_valid ? w : u32x4_t{0u, 0u, 0u, 0u});
    }
  } else if constexpr (STAGE) {
    // the table rows have landed (this wave's loads and everyone's, after the barrier)
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
  }
  if constexpr (STAGE) {
    const int r = R - head * BM_TOK;  // this lane's token within the tile
    // the second K buffer and the second V buffer are one LDS object, so row r is at
    // r * TROW from its start whichever buffer holds it (read through a per-lane choice
    // of two objects, the compiler made the table reads wait for tile 0's loads too)
    const char* row = k_lds1 + r * TROW;
#pragma unroll
    for (int ks = 0; ks < KR; ++ks)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int c = 4 * ks + 2 * hi + h2;  // chunk of elements ks*16 + 8*hi + 4*h2 ..
        rc[ks][h2] = *reinterpret_cast<const f32x4_t*>(row + 16 * (c ^ (r & 15)));
        rs[ks][h2] = *reinterpret_cast<const f32x4_t*>(row + 16 * ((c + D / 8) ^ (r & 15)));
      }
  }
  if constexpr (ROT) {
    // element d of k-step ks (d = ks*16 + 8*hi + e) pairs with d + D/2, which this lane
    // holds in k-step ks + KS/2; rows past the sequence hold zeros and stay zero
#pragma unroll
    for (int ks = 0; ks < KR; ++ks) {
      const float c[8] = {rc[ks][0][0], rc[ks][0][1], rc[ks][0][2], rc[ks][0][3],
                          rc[ks][1][0], rc[ks][1][1], rc[ks][1][2], rc[ks][1][3]};
      const float sn[8] = {rs[ks][0][0], rs[ks][0][1], rs[ks][0][2], rs[ks][0][3],
                           rs[ks][1][0], rs[ks][1][1], rs[ks][1][2], rs[ks][1][3]};
      const u32x4_t xv = __builtin_bit_cast(u32x4_t, qb[ks]);
      const u32x4_t yv = __builtin_bit_cast(u32x4_t, qb[ks + KS / 2]);
      uint32_t x[4] = {xv[0], xv[1], xv[2], xv[3]}, y[4] = {yv[0], yv[1], yv[2], yv[3]};
      rope8_bf16(x, y, c, sn);
      qb[ks] = __builtin_bit_cast(bf16x8_t, u32x4_t{x[0], x[1], x[2], x[3]});
      qb[ks + KS / 2] = __builtin_bit_cast(bf16x8_t, u32x4_t{y[0], y[1], y[2], y[3]});
    }
  }

  // LDS read addresses (bytes within a tile): the K operand of k-step ks for this lane's
  // key row l32 (+32 rows for the second 32-key block: immediate), and the V^T operand
  // of head_dim tile dt for key row key_in (+16 rows per k-step, +8 for the second
  // half: immediates)
  int kaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kaddr[ks] = l32 * RB + 16 * ((2 * ks + hi) ^ swz<D>(l32));
  const int g16 = lane >> 4;
  const int gl = lane & 15;
  const int key_in = 4 * hi + (gl >> 2);
  // (rows key_in and key_in + 8 of a k-step have different swizzles: two addresses)
  int vaddr[DT], vaddr8[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int c = 4 * dt + 2 * (g16 & 1) + ((gl >> 1) & 1);
    vaddr[dt] = key_in * RB + 16 * (c ^ swz<D>(key_in)) + 8 * (gl & 1);
    vaddr8[dt] = (key_in + 8) * RB + 16 * (c ^ swz<D>(key_in + 8)) + 8 * (gl & 1);
  }

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m = -INFINITY;
  float l = 0.f;


  auto step = [&](int t, const char* kl, const char* vl, char* kn, char* vn) {
    const bool has_next = t + 1 < n_kv;
    // tile t has landed in LDS (every wave's share) and every wave is done with t-1
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    // ---- S^T = K Q^T for 64 keys: s[sub][r] is key 32*sub + 8*(r/4) + 4*hi + r%4
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
    // the two 32-key blocks' MFMA chains alternate, and each k-step's two K operands
    // are read while the previous k-step's MFMAs run (the group barriers pin that order:
    // left to itself the scheduler waits on every read right before its MFMA)
    auto kread = [&](int sub, int ks) -> bf16x8_t {
      return __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const u32x4_t*>(kl + 32 * sub * RB + kaddr[ks]));
    };
    bf16x8_t ka[KS][2];
    ka[0][0] = kread(0, 0);
    ka[0][1] = kread(1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 0x100: LDS reads
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
        ka[ks + 1][0] = kread(0, ks + 1);
        ka[ks + 1][1] = kread(1, ks + 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][0], qb[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][1], qb[ks], s[1], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 0x008: MFMAs
    }

    // tile t+1 goes out once this tile's S^T MFMAs are issued: its address arithmetic
    // and load issue then run while those MFMAs execute, rather than ahead of them (2-5%
    // faster than issuing it right after the barrier)
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) {
      fetch(t + 1, te_next, kn, vn);
      if (BIG_BLOCK) te_next = tile_block(min(t + 2, n_kv - 1));
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- causal mask on diagonal tiles (keys past Lk are past every diagonal too)
    if (t >= first_masked_tile) {
      // key offset 32*sub + 8*(r/4) + 4*hi + r%4 is visible when it is <= diag - t*BN;
      // the lane's 4*hi moves to the right-hand side so every test is against a
      // constant (no per-lane offsets held in registers across the loop)
      const int lim = diag - t * BN - 4 * hi;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * sub + 8 * (r >> 2) + (r & 3) > lim) s[sub][r] = -INFINITY;
    }

    // ---- online softmax in the log2 domain; the row max is this lane's 32 keys and
    // lane^32's
    float mx = s[0][0];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sub][r]);
    {  // lanes l and l^32 hold the two halves of a row: v_permlane32_swap pairs them
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * scale_log2;
    }
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack)) {  // wavefront-uniform
      const float m_new = fmaxf(m, mx);  // finite: key 0 of tile 0 is visible to every row
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    bf16x8_t pb[4];  // P^T operand of k-step ks = 2*sub + half
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][8 * half + 2 * e2], scale_log2, -m));
          const float p1 = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s[sub][8 * half + 2 * e2 + 1], scale_log2, -m));
          const bf16x2_t pk = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
          w[e2] = __builtin_bit_cast(uint32_t, pk);
          // the sum takes the rounded probabilities the P.V product uses (the packed
          // pair goes to the dot product as its own value, not re-read out of w)
          l = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes, l, false);
        }
        pb[2 * sub + half] = __builtin_bit_cast(bf16x8_t, w);
      }

    // ---- O^T += V^T P^T: A = V^T via transposing LDS reads, keys in the same order as P
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const i16x4_t lo4 =
            lds_read_tr16(vl + ks * 16 * RB + vaddr[dt]);
        const i16x4_t hi4 =
            lds_read_tr16(vl + ks * 16 * RB + vaddr8[dt]);
        const u32x2_t lo = __builtin_bit_cast(u32x2_t, lo4);
        const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi4);
        const u32x4_t va = {lo[0], lo[1], hi2[0], hi2[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pb[ks],
                                                       o[dt], 0, 0, 0);
      }
    }
  };
  for (int t = 0; t < n_kv; t += 2) {
    step(t, k_lds0, v_lds0, k_lds1, v_lds1);
    if (t + 1 < n_kv) step(t + 1, k_lds1, v_lds1, k_lds0, v_lds0);
  }

  // ---- normalise and store: o[dt][r] is d = 32*dt + 8*(r/4) + 4*hi + r%4 of this row
  {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l),
                                                     false, false);
    l = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
  }
  {
    // staged in LDS, row-major with a 16-byte chunk swizzle (chunk c of row r at
    // c ^ (r % (D/8))), so the stores below write whole rows: one instruction covers
    // 64 / (D/8) rows of 2D contiguous bytes instead of 32 rows x 16 bytes.  The stores
    // are non-temporal: nothing here reads the output again, and the K/V tiles that the
    // other q tiles of a sequence re-read keep the L2 to themselves.  The K/V
    // buffers the last tile did not use are free: every wave has passed the barrier of
    // tile n_kv - 1, so it is done with tile n_kv - 2's buffers, and nothing was
    // fetched into them since.  Each wave takes its own 32 rows' share, so no barrier.
    constexpr int CPO = D / 8;        // 16-byte chunks per output row
    constexpr int RPO = 64 / CPO;     // rows per store instruction
    constexpr int WB = 32 * D * 2;    // bytes of a wave's 32 rows (half a K or V buffer)
    char* stage = (n_kv & 1) ? (wave < 2 ? k_lds1 : v_lds1) : (wave < 2 ? k_lds0 : v_lds0);
    stage += (wave & 1) * WB;
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        // d = 32*dt + 8*r4 + 4*hi .. +4: chunk 4*dt + r4 of the row, its half hi
        u32x2_t w;
        w[0] = pack_bf16x2(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv);
        w[1] = pack_bf16x2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(stage + l32 * (2 * D) +
                                    16 * ((4 * dt + r4) ^ (l32 & (CPO - 1))) + 8 * hi) = w;
      }
    const int cl = lane % CPO;
    u32x4_t rows[32 / RPO];  // every read first, so they overlap
#pragma unroll
    for (int i = 0; i < 32 / RPO; ++i) {
      const int rr = i * RPO + lane / CPO;
      rows[i] = *reinterpret_cast<const u32x4_t*>(stage + rr * (2 * D) +
                                                  16 * (cl ^ (rr & (CPO - 1))));
    }
#pragma unroll
    for (int i = 0; i < 32 / RPO; ++i) {
      const int rr = i * RPO + lane / CPO;  // row of the wave
      const u32x4_t v = rows[i];
      const int Rw = 32 * wave + rr;
      const int hd = Rw / BM_TOK;
      const int tk = tok0 + (Rw - hd * BM_TOK);
      if (hd < G && tk < Lq)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(
            out + (static_cast<int64_t>(q_begin + tk) * Hq + kvh * G + hd) * D + 8 * cl));
    }
  }
}

}  // namespace pkv
