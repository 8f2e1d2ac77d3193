// Host-side interface between the C ABI (pkv_api.cpp) and the kernel launchers
// in the .hip files.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct WriteArgs {
  const void* k;
  const void* v;
  const int64_t* slot_mapping;
  int64_t num_tokens;
  void* k_cache;
  void* v_cache;
  int64_t num_blocks;
  int32_t num_heads;
  int32_t head_dim;
  int32_t dtype;
  int32_t block_shift;  // log2(tokens per block)
};

// Arguments of the decode kernels.
struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_acc;      // [S][H][num_slots][D] unnormalised partial outputs
  float* ws_ml;       // [S][H][num_slots][2]  running max (log2 units) and sum
  int32_t* work_list; // units' entries, largest first: (index << 2) | flags
  int32_t* work_ctrl; // [0] next unit to claim, [1] number of entries in work_list
  // Sharing (null when the call does not look for it): sequences are taken in
  // windows of SHARE_WINDOW consecutive ones; the members of a window that
  // hold the same leading blocks form a group whose shared blocks are read once.
  int32_t* tok_start; // [S] first token a sequence attends to on its own (0: no group)
  int32_t* win_info;  // [W] (shared full blocks J << 4) | member mask, or 0
  int32_t num_windows;
  int64_t num_blocks;
  int32_t num_heads;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t max_context_len;
  int32_t block_size;   // tokens per block: 8, 16 or 32
  int32_t part_blocks;  // blocks per partition
  int32_t num_parts;    // P: partitions of the longest allowed context
  int32_t num_slots;    // partial results per (sequence, head): P + 1 (group partitions + own)
  int32_t max_entries;  // bound on the work list: (S + W) * P
  float scale_log2;     // scale * log2(e)
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  // Cached-prefix form: K/V come from the pool through the block tables instead
  // of k/v (k_cache != nullptr selects it).
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* prefix_lens;  // may be null: no prefix
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t block_shift;  // log2(tokens per block) of the pool
  const int32_t* prompt_lens;
  void* out;
  int64_t total_tokens;
  int32_t num_prompts;
  int32_t num_heads;
  int32_t max_prompt_len;
  int32_t num_qtiles;      // query tiles of the longest prompt
  int32_t items_per_head;  // work items per head: a bound on the query tiles of one head
  int32_t heads_per_xcd;   // ceil(num_heads / 8): heads of one XCD's slice of the grid
  int32_t total_items;     // 8 * heads_per_xcd * items_per_head: the grid
  float scale_log2;
};

// Block copies from a source pool to a destination pool (the same pool for
// copy-on-write).
struct CopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int64_t* pairs;  // [num_pairs][2] (src, dst)
  int64_t num_pairs;
  int64_t src_blocks;
  int64_t dst_blocks;
  int32_t num_heads;
  int32_t tile_bytes;  // block_size * head_dim * element bytes
};

// Each returns a hipError_t from the launch.
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_kv_cache_write(const WriteArgs& a, hipStream_t stream);
// The decode: detect (when sharing is looked for), plan and persistent decode
// kernels; then the reduce, which merges partial results.
hipError_t launch_decode_partial(const DecodeArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs& a, int out_dtype, int head_dim, hipStream_t stream);
// The decode's tile reads without its arithmetic (pkv_kv_read_probe).
hipError_t launch_read_probe(const DecodeArgs& a, int dtype, int head_dim, uint32_t* out, hipStream_t stream);

// Sequences per sharing window of the decode (a group has at most this many
// members).
constexpr int SHARE_WINDOW = 4;
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t stream);

// Prefill query-tile height (rows per workgroup).
constexpr int PREFILL_BLOCK_M = 128;
// Up to this many prompts, each prefill workgroup ranks the prompts by length
// (longest first); beyond it they run in index order.
constexpr int PREFILL_DENSE_PROMPTS = 64;

// Work items per head of the prefill grid: the query tiles of one head, at
// most ceil(total_tokens / BM) + num_prompts for lengths summing to
// total_tokens, and at most num_prompts * num_qtiles.
inline int64_t prefill_items_per_head(int32_t num_prompts, int32_t num_qtiles, int64_t total_tokens) {
  const int64_t sparse = (int64_t)num_prompts * num_qtiles;
  const int64_t dense = (total_tokens + PREFILL_BLOCK_M - 1) / PREFILL_BLOCK_M + num_prompts;
  return dense < sparse ? dense : sparse;
}

}  // namespace pkv
