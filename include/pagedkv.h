/*
 * pagedkv.h -- C ABI of a PagedAttention decode library for AMD Instinct MI355X (gfx950).
 *
 * The problem (sources are the three pages this library follows):
 *   - A sequence's KV cache is split into fixed-size blocks that live anywhere in a physical
 *     pool; a per-sequence block table links logical blocks to physical ones (Qualiteg,
 *     "About PagedAttention for LLM serving", "Deepening Our Understanding ..." item 1-2 and
 *     "There are logical blocks and physical blocks, and the two are linked by a block
 *     table").
 *   - A special kernel removes padding: each sequence of the ragged batch uses exactly its own
 *     context length (same post, "In a Nutshell ..." item 2-1).
 *   - The attention operator must therefore be computed over non-contiguous KV-cache blocks
 *     (vAttention paper, section 3.1 "Requires re-writing the attention kernel"), here for
 *     one new query token per sequence (decode), with grouped-query attention.
 *   - Requests sharing a prefix share its KV blocks (Hacker News discussion of
 *     PagedAttention, replies on prefix sharing); a private copy of a shared block is made
 *     with pkv_copy_blocks before it diverges.
 *
 * Operation: out[i,h,:] = softmax(scale * q[i,h,:] . K_i^T) V_i, where K_i, V_i are the first
 * L_i = context_lens[i] logical positions of sequence i in kv head h / (H / Hkv). The pages
 * give no equation; this is the plain scaled-dot-product reading, every cached position
 * visible to the newest query. context_lens[i] counts the token written this step.
 *
 * Layouts (row-major, contiguous; T = the element type named by pkv_dtype):
 *   q, out         [B, H, D]        T
 *   k_cache        [N, Hkv, S, D]   T   -- token rows; a (block, kv head) tile is S*D contiguous
 *   v_cache        [N, Hkv, (S/VS)*D, VS]  T, VS = min(S, 32) -- column groups of VS positions,
 *                                       each a [D, VS] tile (head_dim rows): position t, dim d of
 *                                       a block at row (t / VS)*D + d, column t % VS; for
 *                                       S <= 32 simply [N, Hkv, D, S]. A (block, kv head) tile is
 *                                       S*D contiguous, like K
 *   key, value     [T_new, Hkv, D]  T   -- the new tokens of this step
 *   slot_mapping   [T_new]          int64, slot = block_id * S + position_in_block
 *   block_tables   [B, MB]          int32; entries at or past ceil(L_i / S) are never used
 *                                         (decode may read any entry of row i, in bounds)
 *   context_lens   [B]              int32
 *   block_mapping  [M, 2]           int64 (src, dst) pairs
 *   partition workspace (split-context mode, fp32):
 *     max_logits, exp_sums [B, H, NPmax];  tmp_out [B, H, NPmax, D]
 *     with NPmax = ceil(max_context_len / partition_size).
 *     For partition p of sequence i, head h: max_logits = max of the natural-log logits
 *     scale*q.k over the partition, exp_sums = sum exp(logit - max_logits), tmp_out = the
 *     partition's normalised output. Partitions p >= ceil(L_i / partition_size) are not
 *     written.
 *
 * Ownership and threading: every pointer argument marked "device" is caller-owned device
 * memory; the library allocates and frees nothing and keeps no state beyond its compiled
 * kernels. All compute calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream) and are reentrant.
 *
 * Errors: arguments are validated on the host before anything is enqueued; a failed check
 * returns PKV_ERR_INVALID_ARGUMENT or PKV_ERR_UNSUPPORTED and enqueues nothing. A failed
 * kernel launch returns PKV_ERR_HIP (pkv_last_hip_error gives the hipError_t). Errors during
 * execution surface at the caller's next synchronisation. pkv_last_error_message returns a
 * thread-local description of the last failure.
 *
 * Caller contract that is not checked (it would need a device-to-host copy): block ids are in
 * [0, N); L_i <= MB * S and L_i <= max_context_len; slots are distinct; copy pairs have
 * distinct destinations and no destination is also a source; the work list is as described
 * at pkv_paged_attention_decode. So that a broken contract can
 * never make a kernel touch memory outside the buffers: kernels clamp block ids into [0, N),
 * work items into [0, B * NP), L_i into [0, MB * S] (and the partition count into
 * [0, NPmax]) and skip slots outside [0, N * S); the results for the affected sequences are
 * then undefined.
 *
 * Supported shapes: D in {64, 128}; S in {16, 32, 64, 128, 256} (the range of block sizes that
 * item 1-2 of the Qualiteg post calls best: larger blocks bring fragmentation back); G = H / Hkv in {1, 2, 4, 8, 16} (fp32 and the VALU kernel: G <= 8);
 * partition_size 0 or a positive multiple of S.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARGUMENT = 1, /* a size, pointer or alignment is wrong */
  PKV_ERR_UNSUPPORTED = 2,      /* a valid shape this build has no kernel for */
  PKV_ERR_HIP = 3,              /* the HIP runtime refused a launch */
  PKV_ERR_NO_BLOCKS = 4         /* the block manager has too few free blocks */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Decode kernel family. AUTO picks MFMA for fp16/bf16 with G >= 4 (the query group makes the
 * per-block product a dense G x D by D x S matrix product) and the VALU kernel otherwise. */
typedef enum { PKV_KERNEL_AUTO = 0, PKV_KERNEL_VALU = 1, PKV_KERNEL_MFMA = 2 } pkv_kernel;

/* Write this step's new K/V rows into the pool: for each t < num_tokens with slot
 * s = slot_mapping[t] in [0, num_blocks * block_size):
 *   k_cache[s / S, h, s % S, :] = key[t, h, :];  v_cache[s / S, h, :, s % S] = value[t, h, :]
 * for every kv head h. Negative slots are skipped (a padding convention). Bit copies.
 * Source: the cache update of each generation step (Qualiteg post, the past_key_values loop
 * in "Deepening Our Understanding ..."), placed by slot into blocks (item 1-2).
 * key, value: device [T_new, Hkv, D]; k_cache, v_cache: device pools; slot_mapping: device
 * int64 [T_new]. 16-byte aligned key/value/k_cache/v_cache. num_tokens may be 0. */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                 void* v_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, pkv_dtype dtype,
                                 void* stream);

/* Paged decode attention (the operation at the top of this file) of one query token per
 * sequence. partition_size == 0: single pass, writes `out`; max_logits/exp_sums/tmp_out must
 * be NULL. partition_size > 0 (a multiple of block_size): split-context mode, writes the
 * partition workspace only; call pkv_paged_attention_reduce afterwards on the same stream.
 * Source: vAttention section 3.1 (attention over non-contiguous KV-cache blocks); Qualiteg
 * post items 1-2 and 2-1 (blocks, block table, no padding).
 * out, q: device [B, H, D]; k_cache, v_cache: device pools of num_blocks blocks;
 * block_tables: device int32 [B, MB], or NULL for the conventional contiguous reservation
 * (sequence i owns pool blocks i * MB .. i * MB + MB - 1, addressed without a table; needs
 * num_blocks >= B * MB) -- the layout paging replaces, kept to measure what the block table
 * costs the kernel; MFMA kernel only); context_lens: device int32 [B].
 * work_items / num_work_items: NULL (all B * NP units in index order), or a device int32 list of
 * num_work_items units u = i * NP + p (sequence i, range p; NP = 1 in single-pass mode, else
 * ceil(max_context_len / partition_size)) in the order they are to be dispatched. The list
 * must hold every unit that has work -- each sequence in single-pass mode, each (i, p) with
 * p < ceil(L_i / partition_size) in split mode -- exactly once; units left out are not
 * computed. Listing the largest units first (longest-processing-time-first) lets small units
 * fill in behind large ones instead of leaving a tail, and leaving out empty partitions keeps
 * them from occupying workgroup slots; the result does not depend on the order.
 * max_context_len: a host-side upper bound of every L_i (sizes the partition grid); scale:
 * the logit scale (usually 1/sqrt(D)). L_i = 0 gives a zero output row (single pass) or no
 * partials. */
pkv_status pkv_paged_attention_decode(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
    int32_t partition_size, float* max_logits, float* exp_sums, float* tmp_out, void* stream);

/* Options of pkv_paged_attention_decode_ex (a NULL options pointer means all defaults). */
enum {
  /* Load K/V with ordinary cached loads instead of the default non-temporal (streaming) ones.
   * Set it when block tables share physical blocks between sequences (a common prefix, Hacker
   * News discussion of PagedAttention, replies on shared prefixes): the shared tiles are then
   * served from the caches. */
  PKV_DECODE_CACHED_KV = 1u << 0
};
typedef struct {
  pkv_kernel kernel;     /* kernel family; PKV_KERNEL_MFMA needs fp16/bf16, VALU needs G <= 8 */
  uint32_t flags;        /* PKV_DECODE_* bits */
  /* NULL, or device [B, Hkv, D] T rows of each sequence's newest token (logical position
   * L_i - 1), 16-byte aligned: the call then also does the cache write of
   * pkv_reshape_and_cache for that token -- K row and V column stored at the slot
   * block_tables maps position L_i - 1 to -- and attends to it from these rows, reading the
   * pool only up to position L_i - 2. new_key and new_value are both NULL or both set. */
  const void* new_key;
  const void* new_value;
} pkv_decode_options;

/* pkv_paged_attention_decode with options (see pkv_decode_options). k_cache and v_cache are
 * written only when options->new_key is set. */
pkv_status pkv_paged_attention_decode_ex(
    const pkv_decode_options* options, void* out, const void* q, void* k_cache, void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    pkv_dtype dtype, int32_t partition_size, float* max_logits, float* exp_sums,
    float* tmp_out, void* stream);

/* Partition 0 of sequences that share its blocks, one pass over each shared tile for the
 * whole group. Requests that share a prompt prefix share its KV blocks (Hacker News discussion
 * of PagedAttention, replies on prefix sharing); grouped-query attention already reuses a
 * loaded tile for the G query heads of its kv head (vAttention section 3.1 names GQA), and
 * this reuses it across the sequences as well: the matrix-core product's 16 columns hold
 * G heads of each of up to 16 / G members.
 * groups: device int32 [num_groups][4], 16-byte aligned; row u lists the sequences of group u,
 * -1 for none; entries past min(4, 16 / G) must be -1 (the kernel does not read them, so a
 * sequence listed there would get no partition 0). Writes max_logits, exp_sums and
 * tmp_out of partition 0 (positions 0 .. partition_size - 1) of every member, exactly as
 * pkv_paged_attention_decode in split-context mode would. The step's other units (the
 * members' partitions p >= 1 and every partition of the other sequences) can run in the same
 * launch: work_items (device int32 [num_work_items], units i * NP + p, or NULL with
 * num_work_items 0) lists them, and new_key/new_value (both NULL or both set; only with a
 * work list) give the fused newest-position write, all exactly as pkv_paged_attention_decode
 * with partitions, PKV_DECODE_CACHED_KV and those options would run them. The caller then
 * merges with pkv_paged_attention_reduce. k_cache and v_cache are written only by the fused
 * write. fp16/bf16; other arguments as for pkv_paged_attention_decode.
 * Caller contract (not checked; PKV_VALIDATE=1 in the Python binding checks it): a sequence is
 * in at most one group; every member has L_i >= partition_size (L_i > partition_size with new
 * rows) and the same block ids in table entries 0 .. partition_size / S - 1 (the first
 * member's table row and length are the ones read); no listed unit is partition 0 of a
 * member, and the work list holds no unit twice. */
pkv_status pkv_paged_attention_decode_shared(
    const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* groups,
    int32_t num_groups, const int32_t* work_items, int32_t num_work_items,
    const void* new_key, const void* new_value, int32_t max_context_len, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, float scale, pkv_dtype dtype, int32_t partition_size,
    float* max_logits, float* exp_sums, float* tmp_out, void* stream);

/* Decode of groups of sequences that share their first shared_len positions, each group in
 * one pass that writes its members' outputs. Requests that share a prompt prefix share its KV
 * blocks (Hacker News discussion of PagedAttention, replies on prefix sharing); the matrix-core
 * product's 16 columns hold the G query heads of each of up to 16 / G members
 * (grouped-query attention, vAttention section 3.1), so a shared tile is read once per group
 * and feeds every member, and then each member's own positions (shared_len .. L_i - 1) are read
 * through its own table row and feed only its columns. The result is the operation at the top
 * of this file for every member, as pkv_paged_attention_decode in single-pass mode computes it
 * (same tolerance, different order of the fp32 additions).
 * out, q: device [B, H, D]; k_cache, v_cache, block_tables, context_lens: as for
 * pkv_paged_attention_decode. groups: device int32 [num_groups][4], 16-byte aligned; row u
 * lists the member sequences of group u (-1 for none; entries past 16 / G must be -1; the
 * first entry must be a member). shared_len: a multiple of block_size, at most
 * max_blocks_per_seq * block_size. new_key/new_value: NULL, or device [B, Hkv, D] rows of each
 * sequence's newest position (L_i - 1), written to its slot and attended to as in
 * pkv_paged_attention_decode_ex. Workgroups run in group order, so list the groups with the
 * most positions first. Only members' rows of out are written. fp16/bf16.
 * Caller contract (not checked; PKV_VALIDATE=1 in the Python binding checks it): a sequence is
 * in at most one group; every member's table agrees with its group's first member's over
 * entries 0 .. shared_len / S - 1; every member has L_i >= shared_len (L_i > shared_len with
 * new rows). */
pkv_status pkv_paged_attention_decode_grouped(
    void* out, const void* q, void* k_cache, void* v_cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* groups,
    int32_t num_groups, int32_t shared_len, const void* new_key, const void* new_value,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype, void* stream);

/* Bytes of the library-owned partition workspace of pkv_paged_attention_decode_static (each
 * device the library runs on holds its own copy until the process ends). */
#define PKV_STATIC_WORKSPACE_BYTES ((size_t)80 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: split-context decode followed by the merge, exactly
 * pkv_paged_attention_decode with partition_size > 0 and then pkv_paged_attention_reduce into
 * `out`, with the partition workspace (max_logits | exp_sums | tmp_out, each part 256-byte
 * aligned) in a static device array of PKV_STATIC_WORKSPACE_BYTES instead of caller memory.
 * It calls no hipMalloc or hipFree; the first call on a device looks up that device's array.
 * Arguments as for pkv_paged_attention_decode (kernel family AUTO, no options); partition_size
 * must be > 0. A shape whose workspace (2 * round_up(4 * B * H * NP, 256) + 4 * B * H * NP * D
 * bytes, NP = ceil(max_context_len / partition_size)) exceeds PKV_STATIC_WORKSPACE_BYTES is
 * rejected with PKV_ERR_INVALID_ARGUMENT before anything is enqueued (the long-context batch of
 * 32 sequences, 64 heads, D 128 up to 32768 positions fits at partitions of 512).
 * All calls on one device share its array, and no part of it needs to start at zero: calls
 * that overlap on one device (on different streams or host threads) race and give undefined
 * results; calls queued on one stream are ordered. */
pkv_status pkv_paged_attention_decode_static(
    void* out, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* work_items, int32_t num_work_items, int32_t max_context_len,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
    int32_t partition_size, void* stream);

/* Merge split-context partitions: for each (i, h) with n = ceil(L_i / partition_size)
 * partitions, M = max_p max_logits, w_p = exp_sums_p * exp(max_logits_p - M),
 * out = sum_p w_p tmp_out_p / sum_p w_p (a zero row when n = 0). The merge is an exact
 * rewriting of the softmax sum; the pages do not describe it.
 * out: device [B, H, D] T; workspace as written by pkv_paged_attention_decode with the same
 * partition_size and max_num_partitions = NPmax. */
pkv_status pkv_paged_attention_reduce(void* out, const float* max_logits,
                                      const float* exp_sums, const float* tmp_out,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t head_dim,
                                      int32_t partition_size, int32_t max_num_partitions,
                                      pkv_dtype dtype, void* stream);

/* Copy-on-write of shared blocks: for each layer l < num_layers and pair (src, dst) of
 * block_mapping, block dst of k_caches[l] and v_caches[l] becomes a bit copy of block src
 * (all Hkv * S * D elements of each). Source: prefix sharing (Hacker News discussion of
 * PagedAttention, replies on shared prefixes).
 * k_caches, v_caches: HOST arrays of num_layers device pool pointers (16-byte aligned);
 * block_mapping: device int64 [num_pairs, 2]; pairs whose src or dst is outside
 * [0, num_blocks) are skipped. */
pkv_status pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                           const int64_t* block_mapping, int32_t num_pairs,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, pkv_dtype dtype, void* stream);

/* Conversion of a V pool between token rows and the column-group layout this library reads
 * (see Layouts above): for every block b < num_blocks, kv head h, position t < S, dim d,
 *   v_cache[b, h, (t / VS) * D + d, t % VS] = v_rows[b, h, t, d]      (from_rows)
 *   v_rows[b, h, t, d] = v_cache[b, h, (t / VS) * D + d, t % VS]      (to_rows)
 * Bit copies. For callers whose V pool is laid out like K ([N, Hkv, S, D] token rows, the
 * blocks of the Qualiteg post's item 1-2): convert once, then decode, prefill and the cache
 * writes run on the column-group pool; to_rows exports it back.
 * v_rows, v_cache: device pools of num_blocks blocks, 16-byte aligned. The two may be the same
 * buffer (converted in place, group by group) or disjoint; any other overlap is rejected.
 * num_blocks may be 0. */
pkv_status pkv_v_cache_from_rows(const void* v_rows, void* v_cache, int32_t num_blocks,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 pkv_dtype dtype, void* stream);
pkv_status pkv_v_cache_to_rows(const void* v_cache, void* v_rows, int32_t num_blocks,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pkv_dtype dtype, void* stream);

/* Bytes of the split-context workspace: 4 * B * H * NPmax * (D + 2); 0 when
 * partition_size <= 0 (or any size is not positive), SIZE_MAX when the product does not fit in
 * size_t. Carve it as max_logits | exp_sums | tmp_out in that order. */
size_t pkv_partition_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                     int32_t max_context_len, int32_t partition_size);

/* Paged prefill attention: causal attention of each sequence's new tokens over its paged
 * cache. Sequence i has Q_i = query_start[i + 1] - query_start[i] new tokens, rows
 * query_start[i] .. query_start[i + 1] - 1 of q and out, at positions L_i - Q_i .. L_i - 1
 * (L_i = context_lens[i]; their K/V must already be in the cache, e.g. written with
 * pkv_reshape_and_cache). The token at position p, head h gets
 *   out = softmax(scale * q . K_i[0..p]^T) V_i[0..p]   over kv head h / (H / Hkv).
 * Source: the first forward pass over the prompt that fills the cache before one-token
 * generation (Qualiteg post, the past_key_values loop in "Deepening Our Understanding ...");
 * a chunk on top of an existing cache is the same computation; blocks and block table as for
 * decode (items 1-2, 2-1; vAttention section 3.1).
 * q, out: device [T, H, D] (T = num_tokens = query_start[B]); k_cache, v_cache, block_tables,
 * context_lens: as for decode; query_start: device int32 [B + 1], non-decreasing from 0;
 * max_query_len: a host bound of every Q_i. Work is split into units (sequence i, tile t of
 * pkv_prefill_tile_tokens query tokens), u = i * NT + t with NT = ceil(max_query_len / tile);
 * work_items / num_work_items: NULL (all B * NT units in index order; tiles past Q_i do
 * nothing) or a device int32 list of the units to run in dispatch order (each unit with tokens
 * exactly once; most positions first shortens the tail). fp16/bf16 only; D in {64, 128};
 * S in {16, 32, 64, 128, 256}; G in {1, 2, 4, 8, 16}. Caller contract (not checked):
 * Q_i <= L_i <= MB * S.
 * Rows are written only for real tokens. */
pkv_status pkv_paged_attention_prefill(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       const int32_t* query_start, int32_t max_query_len,
                                       const int32_t* work_items, int32_t num_work_items,
                                       int32_t num_seqs, int32_t num_tokens, int32_t num_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t num_blocks, float scale,
                                       pkv_dtype dtype, void* stream);
/* Query tokens per prefill work unit for this head shape (128 / G; 0 if unsupported). */
int32_t pkv_prefill_tile_tokens(int32_t num_heads, int32_t num_kv_heads);

/* ---- Host block manager ----
 *
 * The bookkeeping paging needs on the host (Qualiteg post: blocks taken "as needed" and
 * released, item 1-3; logical blocks mapped to physical ones by the block table; per-iteration
 * scheduling that swaps requests in and out, item 2-2; Hacker News discussion: prefix sharing
 * with copy-on-write). Physical blocks [0, num_blocks) of the device pool carry reference
 * counts; a sequence is an ordered list of blocks and a token count. Sharing (fork) adds
 * references; appending a token into a block that other sequences still hold first moves the
 * sequence to a private copy (the caller copies the block with pkv_copy_blocks); freeing drops
 * references and returns blocks that reach zero. Swapping moves a sequence's blocks to a host
 * pool of num_host_blocks (the caller copies them with pkv_swap_blocks) and back. Host-only, no
 * GPU work; not thread-safe per manager. Sequence ids are caller-chosen non-negative int64. */
typedef struct pkv_block_manager pkv_block_manager;

pkv_status pkv_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size,
                         pkv_block_manager** bm);
void pkv_bm_destroy(pkv_block_manager* bm);
int32_t pkv_bm_free_blocks(const pkv_block_manager* bm);       /* device blocks not in use */
int32_t pkv_bm_free_host_blocks(const pkv_block_manager* bm);
/* A new sequence holding num_tokens positions (its prompt): ceil(num_tokens / S) fresh
 * blocks. PKV_ERR_NO_BLOCKS (nothing changed) if they are not all free. */
pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq, int32_t num_tokens);
/* child becomes a copy of parent that shares all of its blocks (one more reference each). */
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
/* Room for one more token of seq: returns its slot (block * S + offset). If the token opens a
 * new block, a fresh block is appended. If it falls into a block that is shared, the sequence
 * gets a fresh private block in its place and *copy_src / *copy_dst name the block to copy
 * (else both are -1); the copy must happen before the token is written. PKV_ERR_NO_BLOCKS
 * (nothing changed) if a needed block is not free. */
pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int64_t* slot, int32_t* copy_src,
                         int32_t* copy_dst);
/* Drop seq: every block loses one reference; blocks reaching zero are free again. */
pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq);
int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq);  /* -1 if unknown */
int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block);  /* -1 if out of range */
/* Block tables of n sequences (host int32 [n, max_blocks], -1 past each sequence's blocks)
 * and their token counts (host int32 [n]). PKV_ERR_INVALID_ARGUMENT if a sequence is unknown,
 * swapped out, or holds more than max_blocks blocks. */
pkv_status pkv_bm_tables(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                         int32_t max_blocks, int32_t* tables, int32_t* context_lens);
/* Swap seq out to host blocks: fills pairs (host int32 [2 * nb], nb = its block count) with
 * (device block, host block) and releases its device references (a shared block stays on the
 * device for its other holders, and this sequence gets a host copy of it).
 * *num_pairs = nb. PKV_ERR_NO_BLOCKS (nothing changed) without enough free host blocks. */
pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq, int32_t* pairs,
                           int32_t max_pairs, int32_t* num_pairs);
/* Swap seq back in: fresh device blocks; pairs = (host block, device block). */
pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq, int32_t* pairs, int32_t max_pairs,
                          int32_t* num_pairs);

/* Copy whole blocks between a device pool and a host pool (both K and V, one layer):
 * for each pair (src, dst) of host int32 pairs [2 * num_pairs], block dst of (dst_k, dst_v)
 * becomes a copy of block src of (src_k, src_v); every block is block_bytes long, and the
 * pools hold num_src_blocks / num_dst_blocks blocks (pairs outside them are refused before
 * anything is enqueued). to_device != 0: sources are host memory, destinations device
 * memory; else the reverse. Host pools should be pinned (hipHostMalloc) for the copies to be
 * asynchronous on `stream`. */
pkv_status pkv_swap_blocks(const void* src_k, const void* src_v, int32_t num_src_blocks,
                           void* dst_k, void* dst_v, int32_t num_dst_blocks,
                           const int32_t* pairs, int32_t num_pairs, size_t block_bytes,
                           int32_t to_device, void* stream);

/* ---- Virtually contiguous KV pool (the alternative to paging that vAttention proposes) ----
 *
 * The conventional layout gives each sequence one contiguous region sized for its maximum
 * length; paging replaces it with blocks and a block table (Qualiteg post, items 1-1..1-3).
 * vAttention's alternative keeps each sequence's KV contiguous in *virtual* memory and backs
 * it with physical pages only as it grows (vAttention paper, section 3: the issues of the
 * PagedAttention model, and its table of contents on virtual-memory demand paging). This
 * pool does that with HIP virtual memory: it reserves, for each of num_seqs sequences and
 * for K and V separately, address space for max_context_len positions in the contiguous
 * layout of pkv_paged_attention_decode without a block table (sequence i owns blocks
 * i * MB .. i * MB + MB - 1, MB = pkv_vmm_pool_blocks_per_seq), and maps physical pages of
 * page_bytes on demand. Decode then reads it through block_tables = NULL with
 * max_blocks_per_seq = MB and num_blocks = num_seqs * MB.
 *
 * Unlike every other entry point these calls allocate: they are the allocator. The pool
 * belongs to the device that is current at creation. Any access to a position that is not
 * mapped faults the GPU: map every position decode or a cache write may touch (the first
 * L_i positions of sequence i) before launching on the pool. Not thread-safe per pool. */
typedef struct pkv_vmm_pool pkv_vmm_pool;

/* Reserve the address space (nothing is mapped yet). page_bytes: physical page size, 0 for
 * the device's recommended granularity, else a multiple of its minimum granularity. MB is
 * rounded up so that every sequence's region is a whole number of pages. */
pkv_status pkv_vmm_pool_create(int32_t num_seqs, int32_t max_context_len, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, pkv_dtype dtype,
                               size_t page_bytes, pkv_vmm_pool** pool);
/* Back positions [0, num_positions) of sequence seq (K and V) with physical pages; grows
 * only (a smaller count than already mapped does nothing). */
pkv_status pkv_vmm_pool_map(pkv_vmm_pool* pool, int32_t seq, int32_t num_positions);
/* Unmap and free all of sequence seq's pages (the sequence finished). The caller must make
 * sure no queued GPU work still reads them. */
pkv_status pkv_vmm_pool_unmap(pkv_vmm_pool* pool, int32_t seq);
/* Copy the first num_blocks blocks of sequence seq between the pool and caller device memory
 * (k, v: device, num_blocks * Hkv * S * D elements each, in the decode layouts), on `stream`:
 * into the pool if to_pool != 0, out of it otherwise. Refuses blocks that are not mapped. */
pkv_status pkv_vmm_pool_copy(pkv_vmm_pool* pool, int32_t seq, int32_t num_blocks, void* k,
                             void* v, int32_t to_pool, void* stream);
/* Unmap everything and release the address space; NULL is ignored. */
void pkv_vmm_pool_destroy(pkv_vmm_pool* pool);
void* pkv_vmm_pool_k(const pkv_vmm_pool* pool);        /* device base of the K region */
void* pkv_vmm_pool_v(const pkv_vmm_pool* pool);        /* device base of the V region */
int32_t pkv_vmm_pool_blocks_per_seq(const pkv_vmm_pool* pool);
size_t pkv_vmm_pool_page_bytes(const pkv_vmm_pool* pool);
size_t pkv_vmm_pool_mapped_bytes(const pkv_vmm_pool* pool); /* K + V physically backed */

/* ---- Read-bandwidth probes (measurement only) ----
 *
 * A paged KV read fetches whole (block, kv head) tiles of S * D contiguous elements from
 * blocks anywhere in the pool (Qualiteg post, item 1-2; vAttention section 3.1: the kernel
 * reads non-contiguous KV-cache blocks). These kernels do those loads and nothing else, so
 * their bandwidth is the ceiling a paged decode can approach on this device. Neither reads
 * anything back to the host: time them with events on `stream`. sink: device, 4-byte
 * aligned, one word that is written only if the folded data equals a fixed pattern (it
 * keeps the loads from being optimised away). nontemporal != 0 uses the streaming cache
 * policy of the decode kernels' K/V loads. workgroups: grid size (256 threads each; a few
 * per compute unit fills the device). */
/* Read bytes (a positive multiple of 32768) of buf (device, 16-byte aligned) once, in 32 KiB
 * chunks spread round-robin over the workgroups. */
pkv_status pkv_probe_stream_read(const void* buf, size_t bytes, int32_t nontemporal,
                                 int32_t workgroups, uint32_t* sink, void* stream);
/* Read num_tiles tiles of tile_bytes (4096 or 8192) at the byte offsets tile_offsets
 * (device int64 [num_tiles]) into base (device, base_bytes long), eight tiles in flight per
 * workgroup, in list order. A tile that does not lie inside [0, base_bytes) or whose offset is
 * not a multiple of 16 is skipped. */
pkv_status pkv_probe_tile_gather(const void* base, size_t base_bytes,
                                 const int64_t* tile_offsets, int32_t num_tiles,
                                 int32_t tile_bytes, int32_t nontemporal, int32_t workgroups,
                                 uint32_t* sink, void* stream);

const char* pkv_status_string(pkv_status s);
int pkv_last_hip_error(void);              /* hipError_t behind the last PKV_ERR_HIP */
const char* pkv_last_error_message(void);  /* thread-local text of the last failure */
int pkv_abi_version(void);                 /* 6: V pool layout conversion */

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
