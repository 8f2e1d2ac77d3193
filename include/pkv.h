/*
 * pkv.h - C ABI of libpkv.so: the PagedAttention hot path on AMD MI355X (gfx950).
 *
 * Keys and values of every sequence live in fixed-size blocks of one physical
 * pool.  Each sequence finds its blocks through a per-sequence block table that
 * maps logical block j to a physical block id.  The blocks need not be
 * contiguous or ordered, and several sequences may reference the same physical
 * block.  Sources:
 *   "PagedAttention and vLLM, annotated", sections 4.1-4.2
 *   "vLLM & PagedAttention: Efficient Memory Management for LLM Serving",
 *   sections III, V and X
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer to memory the caller owns and keeps
 *    alive until the work on `stream` has finished.  The library allocates
 *    nothing and keeps no state between calls.  Arrays are dense (row-major,
 *    no padding) and 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    call only enqueues work and returns without synchronising.  Two calls are
 *    ordered exactly when they are ordered on their streams.
 *  - Sizes and maxima that size a launch grid (num_tokens, num_seqs,
 *    max_context_len, num_prompts, max_prompt_len, total_tokens) come from the
 *    host, so no call ever reads device memory back.
 *  - Return value: PKV_OK, or a negative pkv_status.  No call aborts, throws or
 *    prints.  On error nothing is enqueued.  The one exception is PKV_ELAUNCH,
 *    where a kernel may already be queued.  A fault inside a kernel (for example
 *    an index the caller promised was valid) shows up at the caller's next
 *    synchronisation, as HIP reports it.
 *  - Element types: pkv_dtype.  bf16 is the upper half of an IEEE float32.
 *  - Set PKV_VALIDATE=1 in the environment to make each call copy its index
 *    arrays to the host and check them before launching: table entries in
 *    range, context lengths in [1, max_context_len], slots unique and in range,
 *    copy destinations distinct and not also sources, prompt lengths in range
 *    and summing to total_tokens.  The variable is read at every call.  This
 *    mode synchronises the stream; it is for tests.  A failed check returns
 *    PKV_EINVAL and launches nothing.
 *  - PKV_DECODE_WG_PER_CU (1 to 16, default 1) sets how many workgroups per CU
 *    the per-sequence decode keeps resident; it is read at every launch and
 *    exists to measure other launch shapes.  Results do not depend on it.
 *
 * KV pool layout (both k_cache and v_cache)
 * -----------------------------------------
 *    [num_blocks][num_heads][block_size][head_dim]
 *  One (block, head) tile holds block_size tokens x head_dim values,
 *  contiguously: 4 KiB for 16 x 128 x 2 B.  A decode wavefront reads it as one
 *  fully coalesced 4 KiB burst.  Physical block b with offset o is slot
 *  b * block_size + o.  One block table per sequence is shared by all heads of
 *  the layer: a physical id names the same block index in every head's slice.
 *
 * Supported: block_size 8, 16 (the default) or 32; head_dim 64 or 128; dtype f32, f16 or bf16 for the
 * write and decode; f16 or bf16 for prefill.  Output dtype: f32, or the input
 * dtype.  Accumulation is always in f32, and the result is rounded once
 * (nearest-even) when stored.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* partition_size value that lets the library choose the context partition of
 * the decode (see pkv_paged_attn_decode). */
#define PKV_PARTITION_AUTO (-1)

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,     /* null pointer, bad size, misaligned pointer, failed PKV_VALIDATE check */
  PKV_ENOTSUP = -2,    /* block_size / head_dim / dtype combination not built, or device not gfx950 */
  PKV_ELAUNCH = -3,    /* the HIP runtime reported an error when launching */
  PKV_EDEVICE = -4,    /* the HIP runtime failed to report the current device */
  PKV_EWORKSPACE = -5  /* workspace smaller than pkv_decode_workspace_bytes() asks for */
} pkv_status;

/* Shape and element type of a KV pool (k_cache and v_cache share it). */
typedef struct {
  int64_t num_blocks; /* physical blocks in the pool */
  int32_t num_heads;  /* heads per layer (query heads = KV heads) */
  int32_t head_dim;   /* values per head */
  int32_t block_size; /* tokens per block */
  int32_t dtype;      /* pkv_dtype of the stored keys/values */
} pkv_cache_desc;

/* Version of this ABI; bumped on any incompatible change. */
int pkv_abi_version(void);

/* Static string naming a status code. */
const char* pkv_status_str(int status);

/* PKV_OK when the current HIP device is a gfx950 (MI355X); PKV_ENOTSUP or PKV_EDEVICE otherwise. */
int pkv_check_device(void);

/*
 * pkv_kv_cache_write - scatter new tokens' keys and values into their slots.
 *
 * Writes the K/V of the current tokens into the physical blocks that the block
 * tables assign to them, as one fused reshape-and-write kernel ("vLLM &
 * PagedAttention ...", section X, first kernel detail).  Prompt tokens fill
 * logical blocks left to right; a decode token goes to the next free slot of
 * its last block (same page, section V, Figure 6).
 *
 *   k, v          [num_tokens][num_heads][head_dim], desc->dtype
 *   slot_mapping  int64 [num_tokens]: destination slot of each token.  slot < 0
 *                 means "padding, skip".  A slot >= num_blocks*block_size is
 *                 skipped too, so a bad slot never writes out of bounds.
 *                 Slots must be unique within one call; with duplicates, which
 *                 token lands is unspecified.
 *   k_cache, v_cache  the pool (layout above), modified in place.
 * For every token t and head h with a valid slot:
 *   cache[slot / block_size][h][slot % block_size][:] = new[t][h][:]
 * The copy is byte-exact, with no conversion.  No other byte of the pool changes.
 * num_tokens == 0 is a no-op.
 */
int pkv_kv_cache_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                       void* k_cache, void* v_cache, const pkv_cache_desc* desc, void* stream);

/*
 * Workspace for pkv_paged_attn_decode (and its other forms), in bytes.
 * P = ceil(max_context_len / partition_size), or 1 when partition_size == 0.
 * PKV_PARTITION_AUTO is resolved exactly as the decode resolves it for the
 * same arguments.  With W = ceil(num_seqs / 4) windows, the workspace holds,
 * each region 16-byte aligned:
 *   - a work counter (16 B);
 *   - the list of units, (num_seqs + W) * P int32;
 *   - partial results in float32: P + 1 slots per (sequence, head), each
 *     head_dim values plus a running max and sum
 *     (num_seqs * num_heads * (P + 1) * (head_dim + 2) * 4 B);
 *   - the first token each sequence attends to on its own (num_seqs int32) and
 *     one record per window (W int32), for the sharing the one-call decode
 *     finds.
 * Its contents need no initialisation.  Each call rebuilds what it uses.
 * Returns 0 only for an empty or invalid shape.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * The partition size a decode call uses for these arguments, written to
 * *partition_out: partition_size itself, or what PKV_PARTITION_AUTO resolves to
 * (0 = no split) for the plain decode (shared == 0) or the shared-prefix
 * decode (shared != 0), which follow the same rule; see pkv_paged_attn_decode.
 * Host arithmetic only.  Returns PKV_OK, or PKV_EINVAL (and leaves
 * *partition_out alone) for a null partition_out, num_seqs < 0, num_heads <= 0,
 * max_context_len <= 0 or partition_size < PKV_PARTITION_AUTO.  The value is
 * not checked against the block size: the decode call does that.
 */
int pkv_decode_partition(int32_t num_seqs, int32_t num_heads, int32_t max_context_len, int32_t partition_size,
                         int32_t shared, int32_t* partition_out);

/*
 * A partition size for pkv_paged_attn_decode (and the shared-prefix decode)
 * chosen from the context lengths themselves, for callers that hold them on
 * the host (a scheduler does), written to *partition_out.  context_lens: HOST
 * int32 [num_seqs], each >= 1.  With G = ceil(num_heads / 4) head groups and
 * share = sum(context_lens) * G / 256 (one CU's part of the batch): 0 (no
 * split) when num_seqs * G >= 1024 and the longest context is at most share;
 * otherwise about share / 2 rounded up to a multiple of 32, no larger than
 * what PKV_PARTITION_AUTO gives a batch of fewer than 1024 units, between 512
 * (256 for fewer than 1024 units) and 2048 tokens, and 0 if that covers the
 * longest context.  Unlike PKV_PARTITION_AUTO it splits a large batch of
 * nearly empty contexts beside one long one.  Pass the result as
 * partition_size, to the workspace sizing call as well.  Host arithmetic only.
 * Returns PKV_OK, or PKV_EINVAL (and leaves *partition_out alone) for a null
 * pointer, num_seqs < 0, num_heads <= 0 or a length below 1: an invalid batch
 * never turns into a partition size.
 */
int pkv_decode_partition_for_lengths(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                     int32_t* partition_out);

/*
 * pkv_paged_attn_decode - attention of each sequence's current token over its
 * whole cached context, gathered block by block through its block table.
 *
 * Computes exactly ordinary softmax attention
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . k_t) v_t,  t = 0 .. context_lens[s]-1
 * ("vLLM & PagedAttention ...", section I, attention equation, with i the last
 * position).  It is evaluated block by block (section III, block-wise equation),
 * with a running normaliser across blocks ("PagedAttention and vLLM, annotated",
 * section 4.1).  context_lens[s] includes the current token, so that token's
 * K/V must already be in the pool.  Slots at or past the context length are
 * never used, whatever they hold (NaN included).  Table entries past the last
 * used block are never read.
 *
 *   q             [num_seqs][num_heads][head_dim], desc->dtype
 *   k_cache, v_cache  the pool (read only)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq] physical ids
 *   context_lens  int32 [num_seqs], each in [1, max_context_len];
 *                 max_context_len <= max_blocks_per_seq * block_size.  The
 *                 softmax over an empty context is undefined: a sequence with
 *                 context length 0 gets NaN in every output element.
 *   scale         multiplies q.k before the softmax (usually 1/sqrt(head_dim))
 *   out           [num_seqs][num_heads][head_dim] of out_dtype (PKV_F32 or desc->dtype)
 *   partition_size  tokens per context partition: a multiple of the block size,
 *                 between 16 and 4096, or 0 for no split.  Each (sequence,
 *                 partition, four consecutive heads) is one unit of work.  A
 *                 sequence spanning more than one partition is merged by a
 *                 second, reduce kernel (max-rescaled sum of the partial
 *                 results), in a fixed order.
 *                 PKV_PARTITION_AUTO picks the size from the shape alone
 *                 (num_seqs, num_heads, max_context_len).  With units =
 *                 num_seqs * ceil(num_heads / 4): no split when units >= 1024
 *                 (enough to keep every CU busy) and max_context_len <= 4096;
 *                 otherwise parts = ceil(1024 / units) (1 if units >= 1024)
 *                 and the size is ceil(max_context_len / parts) rounded up to
 *                 a multiple of 32 tokens, at least 256 and at most 2048
 *                 (which bounds the longest unit), with no split if that
 *                 covers max_context_len.  The rule does not see the context
 *                 lengths themselves: for a large batch of nearly empty
 *                 contexts beside one of up to 4096 tokens, an explicit size
 *                 (e.g. 512) balances better.  The result
 *                 depends neither on the block size nor on the device.
 *   workspace     device scratch of at least pkv_decode_workspace_bytes(...),
 *                 owned by the caller.  Calls that can run at the same time
 *                 (different streams) need separate workspaces.
 * Blocks that neighbouring sequences share are read once for all of them
 * ("vLLM & PagedAttention ...", section VII: parallel samples and common
 * prefixes map their first logical blocks onto the same physical blocks).
 * Sequences are taken in windows of four consecutive ones (0-3, 4-7, ...).
 * In a window, the sequences whose first block id equals that of the window's
 * first sequence holding a full block form a group, if there are two or more.
 * The group's J leading full blocks that all members hold with the same ids
 * (inside every member's context) are read once, with one online softmax per
 * member's query; each member then attends to its remaining tokens on its
 * own.  Nothing is assumed about the tables: the sharing is found on the
 * device at every call, and a batch without it runs exactly as before.
 * Work is spread by a small plan kernel and a persistent kernel that claims
 * units from a counter in the workspace; a reduce kernel then merges the
 * partial results of split contexts and sharing groups in a fixed order.  No
 * arithmetic depends on which workgroup ran a unit, so results are
 * deterministic, bit for bit, and do not depend on which physical ids hold the
 * blocks.  Whether blocks are shared changes only the order of the fp32 sums
 * (a group's shared blocks form partial results of their own).  A table entry
 * outside [0, num_blocks) makes that sequence's output NaN instead of reading
 * out of bounds.
 */
int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The decode in two stages, exposed so a caller can time or overlap them.
 * The arguments are identical to pkv_paged_attn_decode's.  This form does not
 * look for shared blocks: every sequence reads its blocks through its own
 * table.  _partial launches the plan and per-partition kernels.  It writes
 * `out` for sequences that fit one partition, and the workspace for the
 * others.  _reduce then merges the workspace into `out` (it launches nothing
 * when no context is split).  _partial followed by _reduce on one stream is
 * pkv_paged_attn_decode, bit for bit, for any batch in which no window's
 * sequences share leading blocks; with sharing the two agree within rounding.
 */
int pkv_paged_attn_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                                  const pkv_cache_desc* desc, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attn_decode_reduce(const void* q, const void* k_cache, const void* v_cache,
                                 const pkv_cache_desc* desc, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn_decode_noalloc - pkv_paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, preconditions, result (bit for bit) and errors are those of
 * pkv_paged_attn_decode with the same partition_size.  The workspace is a
 * fixed device array inside the library, PKV_NOALLOC_SCRATCH_BYTES per GPU,
 * which each GPU the library runs on holds until the process ends.  A call
 * whose workspace (pkv_decode_workspace_bytes for the same arguments) would
 * exceed it returns PKV_EWORKSPACE and launches nothing; use
 * pkv_paged_attn_decode with a caller-owned workspace instead.  The call itself
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 * All calls on one GPU share that GPU's array, whose contents a call rebuilds
 * before use, so calls that can overlap on one GPU (different streams, or
 * different host threads on one stream without ordering) race and must not be
 * issued; calls ordered on one stream are safe.  The array's device address is
 * looked up once per GPU, at the first call made with that GPU current
 * (PKV_EDEVICE if the lookup fails).
 */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                                  int32_t out_dtype, int32_t partition_size, void* stream);

/*
 * pkv_paged_attn_decode_shared and pkv_decode_shared_workspace_bytes are
 * pkv_paged_attn_decode and pkv_decode_workspace_bytes under the names of the
 * shared-prefix decode ("vLLM & PagedAttention ...", section VII), which the
 * one-call decode now performs itself: same arguments, same result, same
 * workspace.
 */
size_t pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size);
int pkv_paged_attn_decode_shared(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                                 int32_t out_dtype, int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * pkv_kv_read_probe - the decode's K/V reads without its arithmetic; a
 * measurement aid, not part of the attention path.
 *
 * Reads exactly the (block, head) tiles that the two-stage decode reads for
 * the same arguments (every block 0 .. ceil(context_lens[s] / block_size) - 1
 * of every sequence, keys and values, whole tiles), with the same plan,
 * persistent scheduling and nontemporal 16-byte loads ("vLLM & PagedAttention
 * ...", section III: blocks gathered through the block table), and computes no
 * attention.  Its time is the HBM rate of the decode's access pattern alone,
 * the ceiling the decode can approach; it also calibrates hardware byte
 * counters for these loads.
 *   out    uint32 [num_seqs][num_heads], all zero on entry (the caller
 *          clears it); receives the XOR of every 32-bit word of the
 *          sequence's K and V tiles for that head.
 * Other arguments, preconditions and errors as for the two-stage decode; the
 * workspace is sized by pkv_decode_workspace_bytes.  A table entry outside the
 * pool is not read and contributes nothing.
 */
int pkv_kv_read_probe(const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t num_seqs, int32_t max_context_len, int32_t partition_size, uint32_t* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_paged_attn_prefill - causal self-attention over each prompt (prompt phase).
 *
 * All positions of a prompt are known at once, so this is dense matrix-matrix
 * attention: S = scale * Q K^T masked to key <= query, a row softmax, then
 * O = P V ("vLLM & PagedAttention ...", section I: the prompt phase and the t <= i
 * limit of the attention equation).  It runs on the MFMA matrix cores, with
 * fp32 accumulation.
 *
 *   q, k, v        packed prompts [total_tokens][num_heads][head_dim] of `dtype`
 *                  (PKV_F16 or PKV_BF16).  Prompt p occupies rows
 *                  off_p .. off_p + prompt_lens[p] - 1, off_p = sum of earlier lengths.
 *   block_tables   int32 [num_prompts][max_blocks_per_seq] or NULL.  Unused here:
 *                  prefill attends over the contiguous k, v above.  After
 *                  pkv_kv_cache_write those hold the same bytes as the
 *                  prompt's blocks, so the result is the same either way.
 *                  pkv_paged_attn_prefill_cached reads through the table.
 *   prompt_lens    int32 [num_prompts], each in [0, max_prompt_len]; their sum
 *                  must equal total_tokens.  Rows beyond total_tokens are never
 *                  touched.
 *   scale          multiplies q.k (usually 1/sqrt(head_dim)); must be positive and finite
 *   out            [total_tokens][num_heads][head_dim] of out_dtype (PKV_F32 or `dtype`)
 */
int pkv_paged_attn_prefill(const void* q, const void* k, const void* v, int32_t num_heads, int32_t head_dim,
                           int32_t dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* prompt_lens, int32_t num_prompts, int64_t total_tokens,
                           int32_t max_prompt_len, float scale, void* out, int32_t out_dtype, void* stream);

/*
 * pkv_paged_attn_prefill_cached - prompt phase over a cached prefix, through the pool.
 *
 * A request whose first tokens are a shared prefix already in the cache (a
 * system prompt, few-shot examples) maps those logical blocks onto the cached
 * physical blocks.  It then runs the prompt phase only over its own new
 * tokens ("vLLM & PagedAttention ...", section VII, shared prefix).  New token i
 * of prompt p sits at position prefix_lens[p] + i.  It attends causally to
 * positions 0 .. prefix_lens[p] + i, all read through the prompt's block table
 * (section I attention equation; section III block-wise evaluation).  The new
 * tokens' K/V must already be in the pool (pkv_kv_cache_write), as in a mixed
 * step: new KV is written, then read through the tables (section V).
 *
 *   q             [total_tokens][num_heads][head_dim] of desc->dtype (PKV_F16 or PKV_BF16):
 *                 the new tokens only, packed prompt after prompt
 *   k_cache, v_cache, desc  the pool (read only)
 *   block_tables  int32 [num_prompts][max_blocks_per_seq]; row p covers positions
 *                 0 .. prefix_lens[p] + prompt_lens[p] - 1
 *   prefix_lens   int32 [num_prompts], each in [0, max_prefix_len], or NULL for no prefix
 *   prompt_lens   int32 [num_prompts], each in [0, max_prompt_len], summing to total_tokens
 *   max_prefix_len + max_prompt_len <= max_blocks_per_seq * block_size
 *   scale         positive and finite
 *   out           [total_tokens][num_heads][head_dim] of out_dtype (PKV_F32 or desc->dtype)
 * With every prefix length 0 this is causal prefill reading K/V through the
 * table: the same result as pkv_paged_attn_prefill over the same bytes.  A
 * table entry outside the pool makes the affected outputs NaN.
 */
int pkv_paged_attn_prefill_cached(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* prefix_lens,
                                  const int32_t* prompt_lens, int32_t num_prompts, int64_t total_tokens,
                                  int32_t max_prompt_len, int32_t max_prefix_len, float scale, void* out,
                                  int32_t out_dtype, void* stream);

/*
 * pkv_copy_blocks - copy whole physical blocks, for copy-on-write.
 *
 * When a sequence must write into a block it shares with others, the block is
 * copied first and the writer's table entry moves to the copy ("vLLM &
 * PagedAttention ...", section VII, Figure 8).  All such copies of a step are
 * batched into one kernel launch, instead of one small memory copy each
 * (section X, third kernel detail).
 *
 *   k_cache, v_cache  the pool (layout above), modified in place
 *   block_pairs   int64 [num_pairs][2] = (source block, destination block)
 * For every pair and every head:
 *   cache[dst][h][:][:] = cache[src][h][:][:]      (keys and values, byte-exact)
 * Pairs with an id outside [0, num_blocks) are skipped.  Destinations must be
 * distinct and must not also be sources in the same call; otherwise, which
 * bytes land is unspecified.  PKV_VALIDATE=1 checks this.  num_pairs == 0 is a
 * no-op.
 */
int pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* desc, const int64_t* block_pairs,
                    int64_t num_pairs, void* stream);

/*
 * pkv_swap_blocks - move whole blocks between two pools (swap out / swap in).
 *
 * When memory runs out, a preempted sequence's blocks are evicted all
 * together.  With swapping, they are copied to a pool in CPU memory and
 * brought back later, possibly into different physical blocks ("vLLM &
 * PagedAttention ...", section VIII; "PagedAttention and vLLM, annotated",
 * section 4.5).  This call copies the (source block, destination block)
 * pairs from one pool to another, all heads, keys and values, in one launch.  Either pool may be device memory or
 * pinned host memory (hipHostMalloc, or torch's pin_memory); the GPU reads or
 * writes host memory directly over the bus.
 *
 *   src_k, src_v      source pool, [src_num_blocks][H][B][D] as desc describes
 *   dst_k, dst_v      destination pool, [dst_num_blocks][H][B][D]
 *   desc              num_heads, head_dim, block_size and dtype of both pools
 *                     (its num_blocks is not used)
 *   block_pairs       int64 [num_pairs][2] = (source block, destination block), in
 *                     device memory or pinned host memory
 * Pairs with an id outside its pool are skipped.  Destinations must be
 * distinct.  A pool pointer that is neither device memory nor pinned host
 * memory returns PKV_EINVAL before anything is launched.  num_pairs == 0 is a
 * no-op.
 */
int pkv_swap_blocks(const void* src_k, const void* src_v, int64_t src_num_blocks, void* dst_k, void* dst_v,
                    int64_t dst_num_blocks, const pkv_cache_desc* desc, const int64_t* block_pairs,
                    int64_t num_pairs, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
