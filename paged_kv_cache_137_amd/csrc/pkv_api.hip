// C ABI of libpkv (declared in include/pkv.h): argument checks, dtype/shape
// dispatch to the gfx950 kernels, and mapping HIP launch errors to status codes.
// Nothing here allocates device memory, and nothing synchronises, except the
// PKV_VALIDATE=1 mode, which copies index arrays to the host to check them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr int kAbiVersion = 2;
constexpr int kBlock = 16;
constexpr int kMaxDevices = 64;
int g_arch[kMaxDevices];  // 0 = not yet checked, 1 = gfx950, -1 = other

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

// PKV_VALIDATE is read at every call, so a process (a test) can switch it.
bool validate_mode() {
  const char* e = std::getenv("PKV_VALIDATE");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PKV_EDEVICE;
  if (dev < kMaxDevices && g_arch[dev] != 0) return g_arch[dev] > 0 ? PKV_OK : PKV_ENOTSUP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PKV_EDEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch[dev] = ok ? 1 : -1;
  return ok ? PKV_OK : PKV_ENOTSUP;
}

int check_desc(const pkv_cache_desc* d) {
  if (d == nullptr) return PKV_EINVAL;
  if (d->num_blocks <= 0 || d->num_heads <= 0 || d->head_dim <= 0 || d->block_size <= 0) return PKV_EINVAL;
  if (!valid_dtype(d->dtype)) return PKV_EINVAL;
  if (d->block_size != 8 && d->block_size != 16 && d->block_size != 32) return PKV_ENOTSUP;
  if (d->head_dim != 64 && d->head_dim != 128) return PKV_ENOTSUP;
  return PKV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

int log2_block(int32_t b) { return b == 8 ? 3 : b == 32 ? 5 : 4; }

template <typename T>
bool copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st) != hipSuccess) return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

// Decode workspace, in this order (each region 16-byte aligned):
//   work_ctrl  2 int32 (+ padding to 16 bytes)
//   work_list  (S + W) * P int32, W = ceil(S / SHARE_WINDOW) windows
//   ws_acc     S * H * (P + 1) * D float
//   ws_ml      S * H * (P + 1) * 2 float
//   tok_start  S int32
//   win_info   W int32
// The one-call decode uses all of it: a sequence in a sharing group has up to
// P + 1 partial results (its group's partitions, then its own).  The two-stage
// form uses the counter, the first S * P list entries and P of the P + 1
// slots.
struct DecodePlan {
  int32_t part_blocks = 0;
  int32_t num_parts = 0;
  int32_t num_windows = 0;
  size_t list_off = 0, acc_off = 0, ml_off = 0, start_off = 0, win_off = 0;
  size_t ws_bytes = 0;
  int64_t max_entries = 0;
};

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

constexpr int32_t kHeadsPerUnit = 4;  // heads one decode unit covers (the kernel's NW)

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                       int32_t partition_size, int32_t block_size = kBlock) {
  DecodePlan p;
  if (partition_size == 0) {
    p.part_blocks = (max_context_len + block_size - 1) / block_size;
    p.num_parts = 1;
  } else {
    p.part_blocks = partition_size / block_size;
    p.num_parts = (max_context_len + partition_size - 1) / partition_size;
  }
  p.num_windows = (num_seqs + pkv::SHARE_WINDOW - 1) / pkv::SHARE_WINDOW;
  p.max_entries = ((int64_t)num_seqs + p.num_windows) * p.num_parts;
  const size_t slots = (size_t)num_seqs * num_heads * (p.num_parts + 1);
  p.list_off = 16;
  p.acc_off = p.list_off + align16((size_t)p.max_entries * sizeof(int32_t));
  p.ml_off = p.acc_off + slots * head_dim * sizeof(float);
  p.start_off = align16(p.ml_off + slots * 2 * sizeof(float));
  p.win_off = p.start_off + align16((size_t)num_seqs * sizeof(int32_t));
  p.ws_bytes = p.win_off + (size_t)p.num_windows * sizeof(int32_t);
  return p;
}

enum Stage { kPartial = 1, kReduce = 2, kBoth = 3 };

// The partition size used when the caller passes PKV_PARTITION_AUTO.  With
// enough (sequence, head group) units to keep every CU busy a few times over,
// and no context longer than kAutoMaxUnsplit tokens, contexts are not split: no
// partial results are written and no reduce runs.  Otherwise the longest
// context is cut into ceil(target / units) partitions (one when the units
// already suffice), whose size is rounded up to a multiple of 32 tokens (so the
// choice does not depend on the block size; the rounding can only lower the
// count), kept at 256 tokens or more and at kAutoMaxPartition or fewer.  The
// cap bounds the longest unit: one very long context among many short ones
// would otherwise be one unit far larger than a CU's share of the batch.  The
// shared-prefix decode follows the same rule.
constexpr int32_t kAutoHeadsPerUnit = 4;    // heads that one decode unit covers
constexpr int64_t kAutoTargetUnits = 1024;  // four units per CU on a 256-CU part
constexpr int64_t kAutoMaxUnsplit = 4096;   // longest context left whole
constexpr int64_t kAutoMaxPartition = 2048;
int32_t resolve_partition(int32_t partition_size, int32_t num_seqs, int32_t num_heads, int32_t max_context_len,
                          bool shared) {
  (void)shared;  // measured: the same choice suits both decodes
  if (partition_size != PKV_PARTITION_AUTO) return partition_size;
  const int64_t units = (int64_t)num_seqs * ((num_heads + kAutoHeadsPerUnit - 1) / kAutoHeadsPerUnit);
  if (units <= 0) return 0;
  if (units >= kAutoTargetUnits && max_context_len <= kAutoMaxUnsplit) return 0;
  const int64_t parts = units >= kAutoTargetUnits ? 1 : (kAutoTargetUnits + units - 1) / units;
  int64_t size = (max_context_len + parts - 1) / parts;
  size = (size + 31) / 32 * 32;
  if (size < 256) size = 256;
  if (size > kAutoMaxPartition) size = kAutoMaxPartition;
  if (size >= max_context_len) return 0;
  return (int32_t)size;
}

// stages: kBoth is the one-call decode (sharing found on the device by the
// plan kernel); kPartial and kReduce are the two stages of the two-stage form
// (no sharing).  The reduce runs only for split contexts.
int decode_impl(int stages, const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t num_seqs, int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len <= 0) return PKV_EINVAL;
  const int32_t bsz = desc->block_size;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * bsz) return PKV_EINVAL;
  if (out_dtype != PKV_F32 && out_dtype != desc->dtype) return PKV_ENOTSUP;
  partition_size = resolve_partition(partition_size, num_seqs, desc->num_heads, max_context_len, false);
  if (partition_size != 0 && (partition_size % bsz != 0 || partition_size < 16 || partition_size > 4096))
    return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16)) return PKV_EINVAL;
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4)) return PKV_EINVAL;
  if (desc->num_heads > 65535 || num_seqs > (1 << 24)) return PKV_EINVAL;
  const DecodePlan plan = plan_decode(num_seqs, desc->num_heads, desc->head_dim, max_context_len, partition_size, bsz);
  const int64_t groups = (desc->num_heads + kHeadsPerUnit - 1) / kHeadsPerUnit;
  // Work-list entries carry two flag bits, and the kernel counts units
  // (entries x head groups) in int32.
  if (plan.max_entries >= ((int64_t)1 << 29) || plan.max_entries * groups > ((int64_t)1 << 31) - 64)
    return PKV_EINVAL;
  if (workspace == nullptr || !aligned(workspace, 16)) return PKV_EINVAL;
  if (workspace_bytes < plan.ws_bytes) return PKV_EWORKSPACE;
  st = device_status();
  if (st != PKV_OK) return st;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);

  if (validate_mode()) {
    std::vector<int32_t> lens, tab;
    if (!copy_to_host(lens, context_lens, (size_t)num_seqs, sm)) return PKV_EDEVICE;
    if (!copy_to_host(tab, block_tables, (size_t)num_seqs * max_blocks_per_seq, sm)) return PKV_EDEVICE;
    for (int32_t s = 0; s < num_seqs; ++s) {
      if (lens[s] < 1 || lens[s] > max_context_len) return PKV_EINVAL;
      const int32_t nb = (lens[s] + bsz - 1) / bsz;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t b = tab[(size_t)s * max_blocks_per_seq + j];
        if (b < 0 || b >= desc->num_blocks) return PKV_EINVAL;
      }
    }
  }

  const bool one_call = stages == kBoth;
  pkv::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  char* ws = reinterpret_cast<char*>(workspace);
  a.work_ctrl = reinterpret_cast<int32_t*>(ws);
  a.work_list = reinterpret_cast<int32_t*>(ws + plan.list_off);
  a.ws_acc = reinterpret_cast<float*>(ws + plan.acc_off);
  a.ws_ml = reinterpret_cast<float*>(ws + plan.ml_off);
  if (one_call) {
    a.tok_start = reinterpret_cast<int32_t*>(ws + plan.start_off);
    a.win_info = reinterpret_cast<int32_t*>(ws + plan.win_off);
    a.num_windows = plan.num_windows;
  }
  a.num_blocks = desc->num_blocks;
  a.num_heads = desc->num_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.max_context_len = max_context_len;
  a.block_size = bsz;
  a.part_blocks = plan.part_blocks;
  a.num_parts = plan.num_parts;
  a.num_slots = plan.num_parts + 1;
  a.max_entries = (int32_t)(one_call ? plan.max_entries : (int64_t)num_seqs * plan.num_parts);
  a.scale_log2 = scale * 1.4426950408889634f;

  if (stages & kPartial) {
    st = launch_status(pkv::launch_decode_partial(a, desc->dtype, out_dtype, desc->head_dim, sm));
    if (st != PKV_OK) return st;
  }
  // Only split contexts leave partial results to merge: with P = 1 a sharing
  // group's unit also streams its members' own blocks and writes their outputs.
  if ((stages & kReduce) && plan.num_parts > 1) {
    st = launch_status(pkv::launch_decode_reduce(a, out_dtype, desc->head_dim, sm));
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

// Device scratch of pkv_paged_attn_decode_noalloc: the decode workspace for
// callers that cannot allocate.  Every GPU the library runs on holds its own
// copy of this array until the process ends.  In host code `scratch` names a
// host-side stand-in, not a device address: host code uses only the address
// hipGetSymbolAddress reports for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_ptr(int dev) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices];
  static bool done[kMaxDevices];
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // clear the failed query's error state
      return nullptr;           // not cached: a later call may retry
    }
    ptrs[dev] = p;
    done[dev] = true;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return kAbiVersion; }

const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_ENOTSUP: return "not supported (block size, head dim, dtype or device)";
    case PKV_ELAUNCH: return "kernel launch failed";
    case PKV_EDEVICE: return "HIP device query failed";
    case PKV_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int pkv_check_device(void) { return device_status(); }

int pkv_kv_cache_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens, void* k_cache,
                       void* v_cache, const pkv_cache_desc* desc, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return PKV_EINVAL;
  st = device_status();
  if (st != PKV_OK) return st;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int64_t> slots;
    if (!copy_to_host(slots, slot_mapping, (size_t)num_tokens, sm)) return PKV_EDEVICE;
    std::vector<int64_t> used;
    used.reserve(slots.size());
    for (int64_t x : slots) {
      if (x < 0) continue;
      if (x >= desc->num_blocks * desc->block_size) return PKV_EINVAL;
      used.push_back(x);
    }
    std::sort(used.begin(), used.end());
    if (std::adjacent_find(used.begin(), used.end()) != used.end()) return PKV_EINVAL;
  }
  pkv::WriteArgs a{};
  a.k = k;
  a.v = v;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = desc->num_blocks;
  a.num_heads = desc->num_heads;
  a.head_dim = desc->head_dim;
  a.dtype = desc->dtype;
  a.block_shift = log2_block(desc->block_size);
  return launch_status(pkv::launch_kv_cache_write(a, sm));
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                                  int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  partition_size = resolve_partition(partition_size, num_seqs, num_heads, max_context_len, false);
  if (partition_size < 0) return 0;
  return plan_decode(num_seqs, num_heads, head_dim, max_context_len, partition_size).ws_bytes;
}

int pkv_decode_partition(int32_t num_seqs, int32_t num_heads, int32_t max_context_len, int32_t partition_size,
                         int32_t shared, int32_t* partition_out) {
  if (partition_out == nullptr || num_seqs < 0 || num_heads <= 0 || max_context_len <= 0) return PKV_EINVAL;
  if (partition_size < PKV_PARTITION_AUTO) return PKV_EINVAL;
  *partition_out = resolve_partition(partition_size, num_seqs, num_heads, max_context_len, shared != 0);
  return PKV_OK;
}

int pkv_decode_partition_for_lengths(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                     int32_t* partition_out) {
  if (partition_out == nullptr || num_seqs < 0 || num_heads <= 0 || (num_seqs > 0 && context_lens == nullptr))
    return PKV_EINVAL;
  int64_t total = 0, longest = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 1) return PKV_EINVAL;
    total += context_lens[s];
    longest = context_lens[s] > longest ? context_lens[s] : longest;
  }
  if (num_seqs == 0) {
    *partition_out = 0;
    return PKV_OK;
  }
  // Each unit covers kAutoHeadsPerUnit heads of one partition; with G head
  // groups a CU's share of the batch is total * G / 256 unit-tokens.  Contexts
  // stay whole when the batch has the units and its longest context is at most
  // one CU's share; otherwise partitions of about half a share, up to
  // kAutoMaxPartition tokens and at least 512 (256 for a batch of few units):
  // below that, partial results and merges cost more than the balance gains.
  const int64_t groups = (num_heads + kAutoHeadsPerUnit - 1) / kAutoHeadsPerUnit;
  const int64_t share = total * groups / 256;
  if ((int64_t)num_seqs * groups >= kAutoTargetUnits && longest <= share) {
    *partition_out = 0;
    return PKV_OK;
  }
  int64_t size = (share / 2 + 31) / 32 * 32;
  if (num_seqs * groups < kAutoTargetUnits) {  // few units: as many as the shape rule makes, at least
    const int32_t by_shape = resolve_partition(PKV_PARTITION_AUTO, num_seqs, num_heads, (int32_t)longest, false);
    if (by_shape > 0 && by_shape < size) size = by_shape;
  }
  const int64_t floor = num_seqs * groups < kAutoTargetUnits ? 256 : 512;
  if (size < floor) size = floor;
  if (size > kAutoMaxPartition) size = kAutoMaxPartition;
  *partition_out = size >= longest ? 0 : (int32_t)size;
  return PKV_OK;
}

size_t pkv_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  partition_size = resolve_partition(partition_size, num_seqs, num_heads, max_context_len, true);
  if (partition_size < 0) return 0;
  return plan_decode(num_seqs, num_heads, head_dim, max_context_len, partition_size).ws_bytes;
}

int pkv_paged_attn_decode_shared(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                                 int32_t out_dtype, int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return decode_impl(kBoth, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, out, out_dtype, partition_size, workspace, workspace_bytes,
                     stream);
}

int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kBoth, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     max_context_len, scale, out, out_dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t max_context_len, float scale, void* out,
                                  int32_t out_dtype, int32_t partition_size, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_context_len <= 0 || partition_size < PKV_PARTITION_AUTO) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  const int32_t part = resolve_partition(partition_size, num_seqs, desc->num_heads, max_context_len, false);
  const size_t need = plan_decode(num_seqs, desc->num_heads, desc->head_dim, max_context_len, part,
                                  desc->block_size).ws_bytes;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_EWORKSPACE;
  st = device_status();
  if (st != PKV_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EDEVICE;
  void* ws = scratch_ptr(dev);
  if (ws == nullptr) return PKV_EDEVICE;
  return decode_impl(kBoth, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, max_context_len, scale, out, out_dtype, part, ws, PKV_NOALLOC_SCRATCH_BYTES, stream);
}

int pkv_kv_read_probe(const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                      int32_t num_seqs, int32_t max_context_len, int32_t partition_size, uint32_t* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len <= 0) return PKV_EINVAL;
  const int32_t bsz = desc->block_size;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * bsz) return PKV_EINVAL;
  partition_size = resolve_partition(partition_size, num_seqs, desc->num_heads, max_context_len, false);
  if (partition_size != 0 && (partition_size % bsz != 0 || partition_size < 16 || partition_size > 4096))
    return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace) return PKV_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) || !aligned(workspace, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_EINVAL;
  if (desc->num_heads > 65535 || num_seqs > (1 << 24)) return PKV_EINVAL;
  const DecodePlan plan = plan_decode(num_seqs, desc->num_heads, desc->head_dim, max_context_len, partition_size, bsz);
  const int64_t groups = (desc->num_heads + kHeadsPerUnit - 1) / kHeadsPerUnit;
  if (plan.max_entries >= ((int64_t)1 << 29) || plan.max_entries * groups > ((int64_t)1 << 31) - 64)
    return PKV_EINVAL;
  if (workspace_bytes < plan.ws_bytes) return PKV_EWORKSPACE;
  st = device_status();
  if (st != PKV_OK) return st;
  pkv::DecodeArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = reinterpret_cast<char*>(workspace);
  a.work_ctrl = reinterpret_cast<int32_t*>(ws);
  a.work_list = reinterpret_cast<int32_t*>(ws + plan.list_off);
  a.num_blocks = desc->num_blocks;
  a.num_heads = desc->num_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.max_context_len = max_context_len;
  a.block_size = bsz;
  a.part_blocks = plan.part_blocks;
  a.num_parts = plan.num_parts;
  a.num_slots = plan.num_parts + 1;
  a.max_entries = num_seqs * plan.num_parts;
  return launch_status(pkv::launch_read_probe(a, desc->dtype, desc->head_dim, out, reinterpret_cast<hipStream_t>(stream)));
}

int pkv_paged_attn_decode_partial(const void* q, const void* k_cache, const void* v_cache,
                                  const pkv_cache_desc* desc, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kPartial, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     max_context_len, scale, out, out_dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_decode_reduce(const void* q, const void* k_cache, const void* v_cache,
                                 const pkv_cache_desc* desc, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, float scale, void* out, int32_t out_dtype,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kReduce, q, k_cache, v_cache, desc, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                     max_context_len, scale, out, out_dtype, partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attn_prefill(const void* q, const void* k, const void* v, int32_t num_heads, int32_t head_dim,
                           int32_t dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* prompt_lens, int32_t num_prompts, int64_t total_tokens,
                           int32_t max_prompt_len, float scale, void* out, int32_t out_dtype, void* stream) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return valid_dtype(dtype) ? PKV_ENOTSUP : PKV_EINVAL;
  if (out_dtype != PKV_F32 && out_dtype != dtype) return PKV_ENOTSUP;
  if (head_dim != 64 && head_dim != 128) return PKV_ENOTSUP;
  if (num_heads <= 0 || num_heads > 65535 || num_prompts < 0 || num_prompts > 65535) return PKV_EINVAL;
  if (total_tokens < 0 || max_prompt_len < 0 || !(scale > 0.0f) || scale > 1e30f) return PKV_EINVAL;
  if (num_prompts == 0 || max_prompt_len == 0 || total_tokens == 0) return PKV_OK;
  if (!q || !k || !v || !out || !prompt_lens) return PKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(prompt_lens, 4))
    return PKV_EINVAL;
  if (block_tables != nullptr &&
      max_blocks_per_seq <= 0)
    return PKV_EINVAL;
  const int32_t num_qtiles = (max_prompt_len + pkv::PREFILL_BLOCK_M - 1) / pkv::PREFILL_BLOCK_M;
  const int64_t per_head = pkv::prefill_items_per_head(num_prompts, num_qtiles, total_tokens);
  const int64_t heads_per_xcd = (num_heads + 7) / 8;
  const int64_t items = 8 * heads_per_xcd * per_head;
  if (items > ((int64_t)1 << 31) - 64) return PKV_EINVAL;
  int st = device_status();
  if (st != PKV_OK) return st;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> lens;
    if (!copy_to_host(lens, prompt_lens, (size_t)num_prompts, sm)) return PKV_EDEVICE;
    int64_t sum = 0;
    for (int32_t x : lens) {
      if (x < 0 || x > max_prompt_len) return PKV_EINVAL;
      sum += x;
    }
    if (sum != total_tokens) return PKV_EINVAL;
  }
  pkv::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.prompt_lens = prompt_lens;
  a.out = out;
  a.total_tokens = total_tokens;
  a.num_prompts = num_prompts;
  a.num_heads = num_heads;
  a.max_prompt_len = max_prompt_len;
  a.num_qtiles = num_qtiles;
  a.items_per_head = (int32_t)per_head;
  a.heads_per_xcd = (int32_t)heads_per_xcd;
  a.total_items = (int32_t)items;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(pkv::launch_prefill(a, dtype, out_dtype, head_dim, sm));
}

int pkv_paged_attn_prefill_cached(const void* q, const void* k_cache, const void* v_cache, const pkv_cache_desc* desc,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* prefix_lens,
                                  const int32_t* prompt_lens, int32_t num_prompts, int64_t total_tokens,
                                  int32_t max_prompt_len, int32_t max_prefix_len, float scale, void* out,
                                  int32_t out_dtype, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (desc->dtype != PKV_F16 && desc->dtype != PKV_BF16) return PKV_ENOTSUP;
  if (out_dtype != PKV_F32 && out_dtype != desc->dtype) return PKV_ENOTSUP;
  if (desc->num_heads > 65535 || num_prompts < 0 || num_prompts > 65535) return PKV_EINVAL;
  if (total_tokens < 0 || max_prompt_len < 0 || max_prefix_len < 0 || !(scale > 0.0f) || scale > 1e30f)
    return PKV_EINVAL;
  if (num_prompts == 0 || max_prompt_len == 0 || total_tokens == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !out || !prompt_lens || !block_tables) return PKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(prompt_lens, 4) || !aligned(block_tables, 4) || !aligned(prefix_lens, 4))
    return PKV_EINVAL;
  if (max_blocks_per_seq <= 0 ||
      (int64_t)max_blocks_per_seq * desc->block_size < (int64_t)max_prompt_len + (int64_t)max_prefix_len)
    return PKV_EINVAL;
  const int32_t num_qtiles = (max_prompt_len + pkv::PREFILL_BLOCK_M - 1) / pkv::PREFILL_BLOCK_M;
  const int64_t per_head = pkv::prefill_items_per_head(num_prompts, num_qtiles, total_tokens);
  const int64_t heads_per_xcd = (desc->num_heads + 7) / 8;
  const int64_t items = 8 * heads_per_xcd * per_head;
  if (items > ((int64_t)1 << 31) - 64) return PKV_EINVAL;
  st = device_status();
  if (st != PKV_OK) return st;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int32_t> lens, pre, tab;
    if (!copy_to_host(lens, prompt_lens, (size_t)num_prompts, sm)) return PKV_EDEVICE;
    if (prefix_lens != nullptr && !copy_to_host(pre, prefix_lens, (size_t)num_prompts, sm)) return PKV_EDEVICE;
    if (!copy_to_host(tab, block_tables, (size_t)num_prompts * max_blocks_per_seq, sm)) return PKV_EDEVICE;
    int64_t sum = 0;
    for (int32_t p = 0; p < num_prompts; ++p) {
      const int32_t L = lens[p], C = prefix_lens ? pre[p] : 0;
      if (L < 0 || L > max_prompt_len || C < 0 || C > max_prefix_len) return PKV_EINVAL;
      sum += L;
      for (int32_t j = 0; j < (C + L + desc->block_size - 1) / desc->block_size; ++j) {
        const int32_t b = tab[(size_t)p * max_blocks_per_seq + j];
        if (b < 0 || b >= desc->num_blocks) return PKV_EINVAL;
      }
    }
    if (sum != total_tokens) return PKV_EINVAL;
  }
  pkv::PrefillArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.prefix_lens = prefix_lens;
  a.num_blocks = desc->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_shift = log2_block(desc->block_size);
  a.prompt_lens = prompt_lens;
  a.out = out;
  a.total_tokens = total_tokens;
  a.num_prompts = num_prompts;
  a.num_heads = desc->num_heads;
  a.max_prompt_len = max_prompt_len;
  a.num_qtiles = num_qtiles;
  a.items_per_head = (int32_t)per_head;
  a.heads_per_xcd = (int32_t)heads_per_xcd;
  a.total_items = (int32_t)items;
  a.scale_log2 = scale * 1.4426950408889634f;
  return launch_status(pkv::launch_prefill(a, desc->dtype, out_dtype, desc->head_dim, sm));
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* desc, const int64_t* block_pairs,
                    int64_t num_pairs, void* stream) {
  int st = check_desc(desc);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_EINVAL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 8)) return PKV_EINVAL;
  if (desc->num_heads > 65535) return PKV_EINVAL;
  st = device_status();
  if (st != PKV_OK) return st;
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  if (validate_mode()) {
    std::vector<int64_t> pairs;
    if (!copy_to_host(pairs, block_pairs, (size_t)num_pairs * 2, sm)) return PKV_EDEVICE;
    std::vector<int64_t> dsts, srcs;
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int64_t s0 = pairs[2 * i], d0 = pairs[2 * i + 1];
      if (s0 < 0 || s0 >= desc->num_blocks || d0 < 0 || d0 >= desc->num_blocks) return PKV_EINVAL;
      srcs.push_back(s0);
      dsts.push_back(d0);
    }
    std::sort(dsts.begin(), dsts.end());
    std::sort(srcs.begin(), srcs.end());
    if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end()) return PKV_EINVAL;
    for (int64_t d0 : dsts)
      if (std::binary_search(srcs.begin(), srcs.end(), d0)) return PKV_EINVAL;
  }
  pkv::CopyArgs a{};
  a.src_k = k_cache;
  a.src_v = v_cache;
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.pairs = block_pairs;
  a.num_pairs = num_pairs;
  a.src_blocks = desc->num_blocks;
  a.dst_blocks = desc->num_blocks;
  a.num_heads = desc->num_heads;
  a.tile_bytes = desc->block_size * desc->head_dim * (desc->dtype == PKV_F32 ? 4 : 2);
  return launch_status(pkv::launch_copy_blocks(a, sm));
}

int pkv_swap_blocks(const void* src_k, const void* src_v, int64_t src_num_blocks, void* dst_k, void* dst_v,
                    int64_t dst_num_blocks, const pkv_cache_desc* desc, const int64_t* block_pairs,
                    int64_t num_pairs, void* stream) {
  if (desc == nullptr) return PKV_EINVAL;
  pkv_cache_desc d = *desc;
  d.num_blocks = 1;
  int st = check_desc(&d);
  if (st != PKV_OK) return st;
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0) return PKV_EINVAL;
  if (num_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs) return PKV_EINVAL;
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
      !aligned(block_pairs, 8))
    return PKV_EINVAL;
  if (d.num_heads > 65535) return PKV_EINVAL;
  st = device_status();
  if (st != PKV_OK) return st;
  // Every pointer the kernel dereferences must be device memory or pinned host
  // memory; use the device-side address of pinned host memory.
  const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, block_pairs};
  void* dev_ptrs[5];
  for (int i = 0; i < 5; ++i) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ptrs[i]) != hipSuccess) {
      (void)hipGetLastError();  // clear the query's error state
      return PKV_EINVAL;
    }
    if (attr.type == hipMemoryTypeDevice) {
      dev_ptrs[i] = const_cast<void*>(ptrs[i]);
    } else if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
      const char* base_h = reinterpret_cast<const char*>(attr.hostPointer);
      dev_ptrs[i] = reinterpret_cast<char*>(attr.devicePointer) + (reinterpret_cast<const char*>(ptrs[i]) - base_h);
    } else {
      return PKV_EINVAL;
    }
  }
  hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
  pkv::CopyArgs a{};
  a.src_k = dev_ptrs[0];
  a.src_v = dev_ptrs[1];
  a.dst_k = dev_ptrs[2];
  a.dst_v = dev_ptrs[3];
  a.pairs = reinterpret_cast<const int64_t*>(dev_ptrs[4]);
  a.num_pairs = num_pairs;
  a.src_blocks = src_num_blocks;
  a.dst_blocks = dst_num_blocks;
  a.num_heads = d.num_heads;
  a.tile_bytes = d.block_size * d.head_dim * (d.dtype == PKV_F32 ? 4 : 2);
  return launch_status(pkv::launch_copy_blocks(a, sm));
}

}  // extern "C"
