// Host control plane: the block manager of include/pkv.h (pkv_bm_*).  Follows the
// BlockManager of “Nano-vLLM 引擎架构解析” section 3.2 "PagedAttention" (Block: id,
// reference count, token ids; a deque of free blocks whose head is handed out; reuse
// by prefix hash; blocks allocated on demand) and “深入 Nano-vLLM 推理引擎” headings
// "From Sequences to Blocks", "Prefix Caching by hashing", "Control plane vs. data
// plane" and "Handling resource exhaustion".  Plain C++: no device call.
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "errors.h"

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): offset basis and prime of the published definition
constexpr uint64_t kFnvBasis = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// hash of a full block chained on the previous block's hash
uint64_t block_hash(uint64_t prev, const int32_t* tokens, int n) {
  unsigned char buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(prev >> (8 * i));
  uint64_t h = fnv_bytes(kFnvBasis, buf, 8);
  for (int t = 0; t < n; ++t) {
    const uint32_t v = static_cast<uint32_t>(tokens[t]);
    const unsigned char b[4] = {static_cast<unsigned char>(v), static_cast<unsigned char>(v >> 8),
                                static_cast<unsigned char>(v >> 16),
                                static_cast<unsigned char>(v >> 24)};
    h = fnv_bytes(h, b, 4);
  }
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;  // registered in the hash map under `hash`
  uint64_t hash = 0;
  std::vector<int32_t> tokens;  // the block's token ids while hashed
};

struct Sequence {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;
  int32_t cached_tokens = 0;
  uint64_t last_hash = kFnvBasis;  // hash of the last full block while allocated
};

}  // namespace

struct pkv_block_manager {
  int32_t block_size = 0;
  std::vector<Block> blocks;
  std::deque<int32_t> free_blocks;
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_seq = 0;

  // The block a full block of these tokens (chained on prev) would reuse, or -1.
  int32_t lookup(uint64_t h, const int32_t* tokens) const {
    const auto it = by_hash.find(h);
    if (it == by_hash.end()) return -1;
    const Block& b = blocks[it->second];
    if (std::memcmp(b.tokens.data(), tokens, sizeof(int32_t) * block_size) != 0) return -1;
    return it->second;
  }

  // Head of the free deque, its old registration dropped.
  int32_t take_free() {
    const int32_t id = free_blocks.front();
    free_blocks.pop_front();
    Block& b = blocks[id];
    if (b.hashed) {
      const auto it = by_hash.find(b.hash);
      if (it != by_hash.end() && it->second == id) by_hash.erase(it);
      b.hashed = false;
      b.tokens.clear();
    }
    b.ref = 1;
    return id;
  }

  // A cached block taken back off the free deque (ref 0 -> 1).
  void revive(int32_t id) {
    for (auto it = free_blocks.begin(); it != free_blocks.end(); ++it)
      if (*it == id) {
        free_blocks.erase(it);
        break;
      }
    blocks[id].ref = 1;
  }

  void register_hash(int32_t id, uint64_t h, const int32_t* tokens) {
    Block& b = blocks[id];
    const auto it = by_hash.find(h);
    if (it != by_hash.end() && it->second != id) blocks[it->second].hashed = false;
    by_hash[h] = id;
    b.hashed = true;
    b.hash = h;
    b.tokens.assign(tokens, tokens + block_size);
  }

  // Plan of an allocation: how many leading full blocks hit, and how many free
  // blocks it takes (misses, the partial block, and hits on freed blocks).
  void plan(const Sequence& s, int32_t* hits, int64_t* takes) const {
    const int64_t n = static_cast<int64_t>(s.tokens.size());
    const int64_t nblk = (n + block_size - 1) / block_size;
    const int64_t full = n / block_size;
    uint64_t h = kFnvBasis;
    int32_t hit = 0;
    int64_t take = 0;
    bool miss = false;
    for (int64_t j = 0; j < full; ++j) {
      const int32_t* tok = s.tokens.data() + j * block_size;
      h = block_hash(h, tok, block_size);
      const int32_t id = miss ? -1 : lookup(h, tok);
      if (id < 0) {
        miss = true;
        ++take;
      } else {
        ++hit;
        if (blocks[id].ref == 0) ++take;
      }
    }
    take += nblk - full;  // the partial last block
    *hits = hit;
    *takes = take;
  }
};

namespace {

pkv_status get_seq(pkv_block_manager* bm, int64_t seq, Sequence** out) {
  if (bm == nullptr) return pkv::report_error(PKV_ERR_INVALID, "block manager is NULL");
  const auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end())
    return pkv::report_error(PKV_ERR_INVALID, "unknown sequence id %lld",
                             static_cast<long long>(seq));
  *out = &it->second;
  return PKV_OK;
}

pkv_status get_seq(const pkv_block_manager* bm, int64_t seq, const Sequence** out) {
  Sequence* s = nullptr;
  const pkv_status st = get_seq(const_cast<pkv_block_manager*>(bm), seq, &s);
  *out = s;
  return st;
}

void release(pkv_block_manager* bm, Sequence& s) {
  for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
    Block& b = bm->blocks[*it];
    if (--b.ref == 0) bm->free_blocks.push_back(*it);
  }
  s.table.clear();
  s.cached_tokens = 0;
  s.last_hash = kFnvBasis;
}

}  // namespace

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pkv_block_manager** out) {
  if (out == nullptr) return pkv::report_error(PKV_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1)
    return pkv::report_error(PKV_ERR_INVALID, "num_blocks %d and block_size %d must be >= 1",
                             num_blocks, block_size);
  if (free_order != nullptr) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return pkv::report_error(PKV_ERR_INVALID, "free_order is not a permutation of 0..%d",
                                 num_blocks - 1);
      seen[b] = 1;
    }
  }
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager;
  if (bm == nullptr) return pkv::report_error(PKV_ERR_INVALID, "host allocation failed");
  bm->block_size = block_size;
  bm->blocks.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i)
    bm->free_blocks.push_back(free_order != nullptr ? free_order[i] : i);
  *out = bm;
  return pkv::report_ok();
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_num_free(const pkv_block_manager* bm) {
  if (bm == nullptr) return pkv::report_error(PKV_ERR_INVALID, "block manager is NULL");
  return static_cast<int32_t>(bm->free_blocks.size());
}

int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
  if (bm == nullptr) return pkv::report_error(PKV_ERR_INVALID, "block manager is NULL");
  if (block < 0 || block >= static_cast<int32_t>(bm->blocks.size()))
    return pkv::report_error(PKV_ERR_INVALID, "block %d outside the pool", block);
  return bm->blocks[block].ref;
}

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, const int32_t* token_ids,
                               int32_t num_tokens, int64_t* seq_out) {
  if (bm == nullptr || token_ids == nullptr || seq_out == nullptr)
    return pkv::report_error(PKV_ERR_INVALID, "NULL argument");
  if (num_tokens < 1) return pkv::report_error(PKV_ERR_INVALID, "num_tokens %d < 1", num_tokens);
  Sequence s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  const int64_t id = bm->next_seq++;
  bm->seqs.emplace(id, std::move(s));
  *seq_out = id;
  return pkv::report_ok();
}

pkv_status pkv_bm_remove_sequence(pkv_block_manager* bm, int64_t seq) {
  Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  release(bm, *s);
  bm->seqs.erase(seq);
  return pkv::report_ok();
}

int32_t pkv_bm_can_allocate(const pkv_block_manager* bm, int64_t seq) {
  const Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  int32_t hits = 0;
  int64_t takes = 0;
  bm->plan(*s, &hits, &takes);
  return takes <= static_cast<int64_t>(bm->free_blocks.size()) ? 1 : 0;
}

pkv_status pkv_bm_allocate(pkv_block_manager* bm, int64_t seq) {
  Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  if (!s->table.empty())
    return pkv::report_error(PKV_ERR_INVALID, "sequence %lld already holds blocks",
                             static_cast<long long>(seq));
  int32_t hits = 0;
  int64_t takes = 0;
  bm->plan(*s, &hits, &takes);
  if (takes > static_cast<int64_t>(bm->free_blocks.size()))
    return pkv::report_error(PKV_ERR_NO_BLOCKS, "needs %lld free blocks, %zu free",
                             static_cast<long long>(takes), bm->free_blocks.size());
  const int32_t bs = bm->block_size;
  const int64_t n = static_cast<int64_t>(s->tokens.size());
  const int64_t full = n / bs;
  uint64_t h = kFnvBasis;
  for (int64_t j = 0; j < full; ++j) {
    const int32_t* tok = s->tokens.data() + j * bs;
    h = block_hash(h, tok, bs);
    if (j < hits) {
      const int32_t id = bm->lookup(h, tok);  // the plan's hit
      if (bm->blocks[id].ref == 0) bm->revive(id);
      else ++bm->blocks[id].ref;
      s->table.push_back(id);
    } else {
      const int32_t id = bm->take_free();
      bm->register_hash(id, h, tok);
      s->table.push_back(id);
    }
  }
  if (n > full * bs) s->table.push_back(bm->take_free());
  s->cached_tokens = hits * bs;
  s->last_hash = h;
  return pkv::report_ok();
}

int32_t pkv_bm_num_cached_tokens(const pkv_block_manager* bm, int64_t seq) {
  const Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  return s->cached_tokens;
}

int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq) {
  const Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  return static_cast<int32_t>(s->tokens.size());
}

int32_t pkv_bm_can_append(const pkv_block_manager* bm, int64_t seq) {
  const Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  const bool needs_block = s->tokens.size() % bm->block_size == 0;
  return (!needs_block || !bm->free_blocks.empty()) ? 1 : 0;
}

pkv_status pkv_bm_append_token(pkv_block_manager* bm, int64_t seq, int32_t token_id) {
  Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  const int32_t bs = bm->block_size;
  const int64_t n = static_cast<int64_t>(s->tokens.size());
  if (static_cast<int64_t>(s->table.size()) != (n + bs - 1) / bs)
    return pkv::report_error(PKV_ERR_INVALID, "sequence %lld is not allocated",
                             static_cast<long long>(seq));
  const bool needs_block = n % bs == 0;
  if (needs_block && bm->free_blocks.empty())
    return pkv::report_error(PKV_ERR_NO_BLOCKS, "no free block for sequence %lld",
                             static_cast<long long>(seq));
  if (needs_block) s->table.push_back(bm->take_free());
  s->tokens.push_back(token_id);
  if ((n + 1) % bs == 0) {  // the token filled its block: register the block's hash
    const int32_t* tok = s->tokens.data() + (n + 1 - bs);
    s->last_hash = block_hash(s->last_hash, tok, bs);
    bm->register_hash(s->table.back(), s->last_hash, tok);
  }
  return pkv::report_ok();
}

pkv_status pkv_bm_deallocate(pkv_block_manager* bm, int64_t seq) {
  Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  release(bm, *s);
  return pkv::report_ok();
}

int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* out,
                           int32_t capacity) {
  const Sequence* s = nullptr;
  if (const pkv_status st = get_seq(bm, seq, &s)) return st;
  if (capacity < 0 || (out == nullptr && capacity > 0))
    return pkv::report_error(PKV_ERR_INVALID, "bad output array (capacity %d)", capacity);
  const int32_t n = static_cast<int32_t>(s->table.size());
  for (int32_t i = 0; i < n && i < capacity; ++i) out[i] = s->table[i];
  return n;
}

}  // extern "C"
