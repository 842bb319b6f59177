/*
 * pkv.h - paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The data plane of a nano-vLLM-style engine: the KV write through a slot
 * mapping, causal prefill over sequences packed by cumulative lengths that reads
 * cached blocks through block tables, and decode over block tables with context
 * lengths.  Pages: “Nano-vLLM 引擎架构解析” section 3.2
 * "PagedAttention" (fixed pool of 256-token blocks, ref-counted ids, block reuse
 * by prefix hash) and “深入 Nano-vLLM 推理引擎” headings "From Sequences to Blocks",
 * "Prefix Caching by hashing", "Control plane vs. data plane" (block metadata
 * lives on the CPU, KV data on the GPU, freed blocks are not cleared),
 * "Prefill and Decode" and "Preparing for computation" (prefill packs sequences
 * by cumulative lengths; decode batches one token per sequence).
 *
 * Conventions for every call:
 *  - Every array pointer of the data-plane calls (store, prefill, decode) is a
 *    DEVICE pointer owned by the caller.  The library allocates no device memory,
 *    keeps no state between calls, never synchronises, and enqueues all its work
 *    on `stream`.  Calls are reentrant.  (Exceptions, each said where it is
 *    declared: the contract checks and debug mode synchronise and report through a
 *    status word the library holds per device.)  The block manager (pkv_bm_*) is
 *    host-only and takes host arrays.
 *  - Element type: q, k, v, both caches and out share one type (pkv_dtype).
 *    Metadata arrays are int32.
 *  - Cache layout (one layer): k_cache and v_cache are each
 *    [num_blocks][block_size][num_kv_heads][head_dim], contiguous.  Slot s is
 *    block s / block_size, offset s % block_size, i.e. row s of
 *    [num_blocks * block_size][num_kv_heads][head_dim].
 *  - Grouped heads: q head h reads kv head h / (num_q_heads / num_kv_heads).
 *  - Causal alignment: a sequence with Lq queries over Lk keys places query i
 *    at position Lk - Lq + i; it sees keys 0 .. Lk - Lq + i.
 *  - Host scalars are validated before any HIP call; a bad one returns an error
 *    status and touches nothing.  Device arrays are the caller's contract and
 *    are not read on the host (see each call); pkv_validate_* and debug mode
 *    (PKV_DEBUG) check them.  Results never depend on cache
 *    rows outside a sequence's (table, length): stale or NaN contents of freed
 *    blocks and of the unused tail of a sequence's last block cannot leak.
 *  - Supported: head_dim 64 or 128; block_size a power of two in [1, 256];
 *    num_q_heads a multiple of num_kv_heads.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent shapes */
  PKV_ERR_UNSUPPORTED = -2, /* head_dim, block_size or dtype outside what is built */
  PKV_ERR_WORKSPACE = -3,   /* decode workspace missing or too small */
  PKV_ERR_HIP = -4,         /* a kernel launch failed (hipGetLastError) */
  PKV_ERR_NO_BLOCKS = -5    /* block manager: too few free blocks (the scheduler preempts) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* One layer's KV pool.  The control plane owns block ids and reference counts;
 * the data plane sees ids only.  A block shared by several sequences (a cached
 * prefix) simply appears in several block tables. */
typedef struct {
  void* k_cache; /* [num_blocks][block_size][num_kv_heads][head_dim] */
  void* v_cache; /* same shape */
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_cache;

/* KV write (“深入 Nano-vLLM 推理引擎”, "Control plane vs. data plane": a reused block is simply
 * overwritten).  For t in [0, num_tokens): if slot_mapping[t] >= 0, row
 * slot_mapping[t] of each cache receives k[t] / v[t] bit for bit; slot -1 (a
 * padding row) writes nothing.
 *   k, v          [num_tokens][num_kv_heads][head_dim], contiguous
 *   slot_mapping  [num_tokens] int32
 * Contract: valid slots lie in [0, num_blocks * block_size) and are distinct
 * within one call (two writes to one slot would race).  num_tokens == 0 is a
 * no-op. */
pkv_status pkv_store_kvcache(const pkv_cache* cache, const void* k, const void* v,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             hipStream_t stream);

/* Rotary position embedding (RoPE), fused into the KV write and into the attention
 * calls' query prologue (“基于 nano-vLLM 学习大模型推理关键功能” §3.3 lists a rotary_embedding layer
 * among the model's layers; the formula is RoFormer's (Su et al., 2021), with the
 * half-split pairing: element i of a head row pairs with element i + head_dim/2).
 * For a row x at position p, with c_i = cos(p * theta_i), s_i = sin(p * theta_i):
 *   x'[i]              = x[i] * c_i - x[i + head_dim/2] * s_i
 *   x'[i + head_dim/2] = x[i + head_dim/2] * c_i + x[i] * s_i,   i < head_dim/2,
 * computed in fp32 and rounded once to the element type.  The table is the caller's:
 *   cos_sin       device fp32 [max_position][head_dim]; row p holds c_0 .. c_{D/2-1}
 *                 then s_0 .. s_{D/2-1} (theta_i = base^(-2i/head_dim) conventionally)
 *   max_position  rows of the table (>= 1); a position outside [0, max_position) is a
 *                 contract violation and reads the nearest row. */
typedef struct {
  const float* cos_sin;
  int32_t max_position;
} pkv_rotary;

/* pkv_store_kvcache with K rotated at its token's position on the way in (V is copied
 * bit for bit).
 *   positions  [num_tokens] int32 device array: the token's position in its sequence */
pkv_status pkv_store_kvcache_rotary(const pkv_cache* cache, const void* k, const void* v,
                                    const int32_t* slot_mapping, const int32_t* positions,
                                    int32_t num_tokens, const pkv_rotary* rotary,
                                    hipStream_t stream);

/* Varlen causal prefill (“深入 Nano-vLLM 推理引擎”, "Preparing for computation": sequences are
 * packed and addressed by cumulative lengths; "Prefix Caching": cached blocks
 * are read, not recomputed).  Sequence b owns query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and Lk = cu_seqlens_k[b+1] -
 * cu_seqlens_k[b] keys, read from the cache through block_tables[b]; K/V of all
 * Lk tokens (the new ones included) must already be written.
 *   q, out         [total_q][num_q_heads][head_dim], total_q = cu_seqlens_q[batch]
 *   cu_seqlens_q   [batch+1] int32, non-decreasing, starting at 0
 *   cu_seqlens_k   [batch+1] int32, non-decreasing, starting at 0
 *   max_seqlen_q   host upper bound on every Lq (sizes the grid)
 *   max_seqlen_k   host upper bound on every Lk
 *   block_tables   [batch][block_table_stride] int32; only entries
 *                  0 .. ceil(Lk / block_size)-1 of a row are read
 *   scale          multiplies q.k before the softmax (usually 1/sqrt(head_dim));
 *                  must be finite and > 0 (PKV_ERR_INVALID otherwise)
 * Contract: Lk >= Lq, Lk >= 1 when Lq > 0, ceil(Lk/block_size) <=
 * block_table_stride, used table entries in [0, num_blocks).  Rows of out
 * outside [0, total_q) are not written. */
pkv_status pkv_paged_prefill(const pkv_cache* cache, const void* q, void* out,
                             int32_t num_q_heads, int32_t batch,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             const int32_t* block_tables, int32_t block_table_stride,
                             float scale, hipStream_t stream);

/* pkv_paged_prefill with every query row rotated at its position (query i of a
 * sequence sits at Lk - Lq + i) before the scores; the cached keys are expected to be
 * rotated already (pkv_store_kvcache_rotary).  q itself is not modified. */
pkv_status pkv_paged_prefill_rotary(const pkv_cache* cache, const void* q, void* out,
                                    int32_t num_q_heads, int32_t batch,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    float scale, const pkv_rotary* rotary, hipStream_t stream);

/* Bytes of device workspace pkv_paged_decode needs for this shape; num_workers as
 * in pkv_paged_decode.  0 for the fp32 path (it needs none) and for invalid
 * arguments.  For bf16: 2*W*HS*(4*head_dim + 8) + 8*(batch + 1) bytes, rounded up
 * to 256-byte pieces, with W = num_workers (the automatic count when 0) and HS =
 * MH*GP heads per stream (see num_workers): GP = q heads per kv head rounded down to
 * a power of two, at most 8; MH = the largest power of two dividing num_kv_heads with
 * MH*head_dim*2 <= 512 bytes (1024 from GP 8 up) (about 2.1 MB at head_dim 128, 32 q /
 * 32 kv heads and the automatic W = 1024).  max_context_len does not change it.  The
 * worker count is an argument, unlike the survey's four-argument form, because the
 * workspace scales with it and a caller may choose it. */
size_t pkv_paged_decode_workspace_size(const pkv_cache* cache, int32_t num_q_heads,
                                       int32_t batch, int32_t max_context_len,
                                       int32_t num_workers);

/* Decode (“深入 Nano-vLLM 推理引擎”, "Prefill and Decode": one new token per sequence per step).
 * Sequence b's single query attends to its context_lens[b] cached tokens, the
 * new token's K/V (written beforehand) being the last.
 *   q, out          [batch][num_q_heads][head_dim]
 *   context_lens    [batch] int32, each in [1, max_context_len]
 *   max_context_len host upper bound on context_lens
 *   block_tables    [batch][block_table_stride] int32
 *   workspace       device scratch of at least
 *                   pkv_paged_decode_workspace_size(...) bytes (may be NULL when
 *                   that size is 0); contents on entry are ignored
 *   num_workers     bf16: a stream is (sequence, MH adjacent kv heads, up to GP q
 *                   heads of each); its K/V is cut into chunks of 2048/(head_dim*MH)
 *                   tokens, and the list of all chunks is divided evenly among this
 *                   many wavefront workers; a stream cut between workers is merged
 *                   exactly (log-sum-exp) by a second kernel.  0 = automatic:
 *                   1024 workers while GP <= 4, 2048 for GP 8 (a constant of the
 *                   shape, never read from the device); W in [1, 2^20] = exactly W
 *                   (1 = no cut at all).  Ignored by the fp32 path, which never cuts.
 * Where a context is cut depends only on the lengths, the shape and the worker count,
 * never on block ids or on the device, so results are bit-identical under any
 * relabelling of physical blocks and on any part. */
pkv_status pkv_paged_decode(const pkv_cache* cache, const void* q, void* out,
                            int32_t num_q_heads, int32_t batch,
                            const int32_t* context_lens, int32_t max_context_len,
                            const int32_t* block_tables, int32_t block_table_stride,
                            float scale, void* workspace, size_t workspace_bytes,
                            int32_t num_workers, hipStream_t stream);

/* pkv_paged_decode with each query rotated at its position, context_lens[b] - 1,
 * before the scores (keys rotated already; q not modified). */
pkv_status pkv_paged_decode_rotary(const pkv_cache* cache, const void* q, void* out,
                                   int32_t num_q_heads, int32_t batch,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   int32_t num_workers, const pkv_rotary* rotary,
                                   hipStream_t stream);

/* One decode step in one call: the KV write of each sequence's new token and the
 * decode over the context that now ends with it (“深入 Nano-vLLM 推理引擎”, "Prefill and
 * Decode": a decode step appends one token per sequence and attends over the whole
 * context).  k_new, v_new: [batch][num_kv_heads][head_dim] device arrays of the cache's
 * element type, the new token of each sequence; slot_mapping: int32 [batch] on the
 * device, the cache slot of position context_lens[b] - 1 of sequence b (the slot
 * pkv_store_kvcache would be given), -1 to skip the write.  The other arguments are
 * those of pkv_paged_decode.  The cache and out end bit-identical to pkv_store_kvcache
 * (k_new, v_new, slot_mapping, batch tokens) followed by pkv_paged_decode with the same
 * num_workers, provided slot_mapping[b] is that slot of block_tables[b] (with -1 the
 * cache row is left alone while the attention may still take the token from k_new /
 * v_new).  With bf16 caches, one q head per kv head and blocks of at least one decode
 * chunk (8 tokens at head_dim 128) the decode kernel writes the new rows itself and
 * takes the new token's K and V from k_new / v_new, saving the KV-write launch;
 * otherwise the two kernels run in turn.  Errors as in the two calls. */
pkv_status pkv_paged_decode_append(const pkv_cache* cache, const void* q, const void* k_new,
                                   const void* v_new, void* out, int32_t num_q_heads,
                                   int32_t batch, const int32_t* slot_mapping,
                                   const int32_t* context_lens, int32_t max_context_len,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   float scale, void* workspace, size_t workspace_bytes,
                                   int32_t num_workers, hipStream_t stream);

/* pkv_paged_decode (or pkv_paged_decode_rotary when rotary is not NULL) without a
 * workspace argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The split-K
 * workspace is a fixed 16 MiB device array of the library's own, one per GPU, held
 * until the process ends; this call allocates nothing.  Results are bit-identical to
 * pkv_paged_decode with the same num_workers.  A shape whose workspace
 * (pkv_paged_decode_workspace_size) exceeds 16 MiB returns PKV_ERR_WORKSPACE: the
 * automatic worker count fits for up to 4 q heads per kv head; with 8 or more ask for
 * fewer workers (e.g. 480 at head_dim 128).  Calls on one GPU share its array: calls in
 * flight on one GPU at once race.  Other arguments and errors as in pkv_paged_decode. */
pkv_status pkv_paged_decode_noalloc(const pkv_cache* cache, const void* q, void* out,
                                    int32_t num_q_heads, int32_t batch,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    float scale, int32_t num_workers, const pkv_rotary* rotary,
                                    hipStream_t stream);

/* One step's attention for a batch holding sequences in both phases (“深入 Nano-vLLM 推理引擎”,
 * "Prefill and Decode" and the scheduler headings: the running batch mixes prompts
 * being prefilled with sequences being decoded).  The prefill arguments are those of
 * pkv_paged_prefill (for the prefill sequences), the decode arguments those of
 * pkv_paged_decode (for the decode sequences, with its workspace and num_workers), and
 * rotary is NULL or as in the _rotary calls.  Results are bit-identical to the two
 * calls made one after the other.  For bf16 caches with block_size >= 64 and at most
 * 8 q heads per kv head both passes run in one kernel launch (workgroups of the
 * decode pass, then the prefill's work items, sharing the GPU) followed by the
 * decode's merge kernel; other shapes, and steps with one phase empty, run the two
 * passes one after the other.  Errors as in the two calls. */
pkv_status pkv_mixed_attention(const pkv_cache* cache, int32_t num_q_heads, float scale,
                               const void* q_prefill, void* out_prefill, int32_t prefill_batch,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               const int32_t* prefill_tables, int32_t prefill_table_stride,
                               const void* q_decode, void* out_decode, int32_t decode_batch,
                               const int32_t* context_lens, int32_t max_context_len,
                               const int32_t* decode_tables, int32_t decode_table_stride,
                               void* workspace, size_t workspace_bytes, int32_t num_workers,
                               const pkv_rotary* rotary, hipStream_t stream);

/* ---- Block manager: the host control plane that hands out block ids.
 * (“Nano-vLLM 引擎架构解析” section 3.2 "PagedAttention": a Block has an id, a
 * reference count and its token ids; the manager keeps a deque of free blocks and
 * hands out its head; blocks are reused by prefix hash and allocated on demand as a
 * sequence grows.  “深入 Nano-vLLM 推理引擎”: "From Sequences to Blocks" (a sequence is
 * cut into fixed-size blocks; two sequences never share a block's tokens), "Prefix
 * Caching by hashing" (a hash -> block id map; a new sequence whose block hash is
 * cached takes that block with one more reference), "Control plane vs. data plane"
 * (the manager lives in host memory; a freed block is only marked free, its GPU
 * contents are overwritten on reuse) and "Handling resource exhaustion" (when no
 * block is free the scheduler preempts a sequence).)
 *
 * Host memory only: no device call is made.  A manager is not thread-safe; use one
 * per control-plane thread.  Sequences are named by the ids pkv_bm_add_sequence
 * returns.
 *
 * Prefix cache.  Only full blocks are cached.  Block j of a sequence (tokens
 * j*block_size .. (j+1)*block_size - 1) has the hash h_j = FNV-1a-64 over the 8
 * bytes of h_{j-1} (h_{-1} = the FNV offset basis) followed by the block's token
 * ids (4 bytes each, little-endian), so equal hashes mean equal whole prefixes up
 * to a 2^-64 collision; a hit also compares the block's own token ids.  When a
 * sequence is allocated, its blocks are looked up from the first: every block up
 * to the first miss is a hit and is reused (one more reference; a cached block that
 * was freed but not yet handed out again is taken back off the free deque); every
 * block from the first miss on, and the last partial block, gets a new block from
 * the head of the free deque.  A new full block registers its hash at once (its
 * K/V are written by the same step's pkv_store_kvcache, before any prefill reads
 * them); a block handed out again loses its old registration, so a stale block is
 * never a hit.  Freed blocks go to the tail of the free deque, the sequence's last
 * block first. */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager over block ids 0 .. num_blocks-1, all free; the free deque holds them in
 * the order of free_order (a host array, a permutation of 0 .. num_blocks-1), or in
 * id order when free_order is NULL.  num_blocks >= 1, block_size >= 1.  *out
 * receives the handle (host memory). */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pkv_block_manager** out);
/* Frees the manager and everything it holds (NULL is a no-op). */
void pkv_bm_destroy(pkv_block_manager* bm);
/* Free blocks, or a negative pkv_status for a NULL manager. */
int32_t pkv_bm_num_free(const pkv_block_manager* bm);
/* Reference count of a block (0 = free), or a negative pkv_status. */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block);

/* Registers a sequence with its first num_tokens token ids (a host array, copied;
 * num_tokens >= 1); it holds no blocks yet.  *seq_out receives its id. */
pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, const int32_t* token_ids,
                               int32_t num_tokens, int64_t* seq_out);
/* Releases the sequence's blocks (if any) and forgets it. */
pkv_status pkv_bm_remove_sequence(pkv_block_manager* bm, int64_t seq);
/* 1 if pkv_bm_allocate would succeed now, 0 if not, negative pkv_status on error. */
int32_t pkv_bm_can_allocate(const pkv_block_manager* bm, int64_t seq);
/* Blocks for all of the sequence's tokens (prefill), prefix hits reused as above.
 * PKV_ERR_NO_BLOCKS if too few are free (nothing changes); PKV_ERR_INVALID if the
 * sequence already holds blocks. */
pkv_status pkv_bm_allocate(pkv_block_manager* bm, int64_t seq);
/* Leading tokens whose K/V were already cached at the last pkv_bm_allocate (a
 * multiple of block_size; these need no prefill), or a negative pkv_status. */
int32_t pkv_bm_num_cached_tokens(const pkv_block_manager* bm, int64_t seq);
/* Tokens the sequence holds, or a negative pkv_status. */
int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq);
/* 1 if pkv_bm_append_token would succeed now (a new block is needed only when the
 * token starts one), 0 if not, negative pkv_status on error. */
int32_t pkv_bm_can_append(const pkv_block_manager* bm, int64_t seq);
/* Decode: appends one token id to an allocated sequence, taking a new block when
 * the token starts one; a block that the token fills registers its hash.
 * PKV_ERR_NO_BLOCKS if a block is needed and none is free (nothing changes). */
pkv_status pkv_bm_append_token(pkv_block_manager* bm, int64_t seq, int32_t token_id);
/* Preemption or completion: drops one reference from each of the sequence's blocks
 * (a block at zero goes to the tail of the free deque, contents and hash kept); the
 * sequence keeps its tokens and can be allocated again. */
pkv_status pkv_bm_deallocate(pkv_block_manager* bm, int64_t seq);
/* Copies the sequence's block table (up to capacity entries) to the host array
 * out and returns its length, or a negative pkv_status.  out may be NULL with
 * capacity 0 to ask for the length. */
int32_t pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* out,
                           int32_t capacity);

/* ---- Contract checks of the metadata arrays (a debugging aid).
 * The data-plane calls trust their device arrays: block ids and slots are chosen on the
 * host by the control plane and the GPU only copies into and reads from them
 * (“深入 Nano-vLLM 推理引擎”, "Control plane vs. data plane"), so a bad slot or length would
 * become an access outside the pool.  These calls check the arrays one data-plane call
 * would read against its contract and report each kind of violation found as a bit:
 *   PKV_BAD_SLOT     a slot outside [0, num_blocks*block_size) other than -1
 *   PKV_DUP_SLOT     a valid slot that appears twice in one call (a write race)
 *   PKV_BAD_TABLE    a used block-table entry (entries 0 .. ceil(L/block_size)-1 of a
 *                    row, capped at the stride) outside [0, num_blocks)
 *   PKV_BAD_SEQLENS  cu_seqlens_q[0] or cu_seqlens_k[0] not 0, a negative length, Lk <
 *                    Lq, Lk = 0 with Lq > 0, Lq > max_seqlen_q or Lk > max_seqlen_k
 *   PKV_BAD_CONTEXT  a context length < 1 or > max_context_len
 *   PKV_BAD_STRIDE   ceil(L/block_size) > block_table_stride
 * arrays_on_host != 0: the arrays are host arrays, checked on the calling thread (stream
 * unused).  arrays_on_host == 0: they are device arrays, checked by a kernel on `stream`
 * that reports through a status word the library holds per device (no allocation); the
 * call then waits for the stream.  Two device checks in flight on one device at once
 * share that word and race.  Every read stays inside the sizes passed (num_tokens,
 * batch + 1 cumulative lengths, batch rows of block_table_stride entries), whatever
 * the arrays hold.  Returns PKV_OK when every contract holds, PKV_ERR_INVALID (with
 * pkv_last_error naming the violations) when one does not, another status if the check
 * itself could not run; *violations (may be NULL) receives the bits.
 * Debug mode: while pkv_debug_enabled() is 1 (initially when the environment variable
 * PKV_DEBUG is set and not "0"), every data-plane call first checks its device arrays
 * this way and returns the violation without launching anything. */
typedef enum {
  PKV_BAD_SLOT = 1,
  PKV_DUP_SLOT = 2,
  PKV_BAD_TABLE = 4,
  PKV_BAD_SEQLENS = 8,
  PKV_BAD_CONTEXT = 16,
  PKV_BAD_STRIDE = 32
} pkv_contract;

/* Arrays of pkv_store_kvcache (only num_blocks and block_size of `cache` are used). */
pkv_status pkv_validate_store(const pkv_cache* cache, const int32_t* slot_mapping,
                              int32_t num_tokens, int32_t arrays_on_host, uint32_t* violations,
                              hipStream_t stream);
/* Arrays of pkv_paged_prefill. */
pkv_status pkv_validate_prefill(const pkv_cache* cache, int32_t batch,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t arrays_on_host, uint32_t* violations,
                                hipStream_t stream);
/* Arrays of pkv_paged_decode. */
pkv_status pkv_validate_decode(const pkv_cache* cache, int32_t batch,
                               const int32_t* context_lens, int32_t max_context_len,
                               const int32_t* block_tables, int32_t block_table_stride,
                               int32_t arrays_on_host, uint32_t* violations,
                               hipStream_t stream);
/* Turns debug mode on (on != 0) or off for the whole process. */
pkv_status pkv_debug_enable(int32_t on);
/* 1 while debug mode is on, else 0. */
int32_t pkv_debug_enabled(void);

/* Kernel timing, off by default (tracing support for benchmarks).  While on,
 * every kernel the library launches is bracketed by two hipEvents recorded on
 * the stream it runs on.  pkv_timing_collect waits for the recorded events,
 * writes one entry per kernel name (up to `capacity`) and returns how many
 * kernel names there were, or a negative pkv_status on a HIP error; the
 * recorded events are consumed.  Host-side bookkeeping only: no device memory. */
typedef struct {
  char kernel[64];
  int64_t launches;
  double total_ms;
  double min_ms;
  double max_ms;
} pkv_kernel_timing;

pkv_status pkv_timing_enable(int32_t on);
int32_t pkv_timing_collect(pkv_kernel_timing* out, int32_t capacity);

/* The same recorded launches one by one, in launch order: waits for their events,
 * writes one entry per launch (up to `capacity`; the rest are dropped) and returns
 * how many launches there were, or a negative pkv_status on a HIP error.  The events
 * are consumed, as by pkv_timing_collect; call one or the other.  Lets a caller time
 * consecutive launches individually without synchronising between them. */
typedef struct {
  char kernel[64];
  double ms;
} pkv_kernel_sample;

int32_t pkv_timing_samples(pkv_kernel_sample* out, int32_t capacity);

/* Static text for a status code. */
const char* pkv_status_string(pkv_status status);

/* Details of the last error returned on the calling thread ("" if none). */
const char* pkv_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
