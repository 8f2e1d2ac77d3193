// Block copy for copy-on-write on gfx950: every (source, destination) pair of
// the call, all heads, keys and values, in one launch.
//
// A write into a shared block first copies the block and moves the writer to
// the copy ("vLLM & PagedAttention: Efficient Memory Management for LLM
// Serving", section VII, Figure 8).  The copies of one step are batched into a
// single kernel rather than one small memory copy each (section X).
//
// The same kernel moves blocks between two pools, one of which may be pinned
// host memory: the swap-out and swap-in of a preempted sequence's blocks
// (section VIII of the same page).
//
// Decomposition: one workgroup per (pair, head).  Its 256 lanes move the 4 KiB
// (block, head) tile of keys and the one of values in 16-byte chunks, with a
// loop when a tile is larger (fp32 with head_dim 128).  Both tiles are
// contiguous, so every load and store instruction covers 4 KiB of consecutive
// bytes.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__global__ __launch_bounds__(256) void copy_blocks_kernel(const CopyArgs a, int64_t pair0) {
  const int64_t pr = pair0 + blockIdx.x;
  const int h = blockIdx.y;
  const int64_t src = a.pairs[2 * pr];
  const int64_t dst = a.pairs[2 * pr + 1];
  if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks) return;
  const int64_t tile = a.tile_bytes;
  const int64_t so = (src * a.num_heads + h) * tile;
  const int64_t dof = (dst * a.num_heads + h) * tile;
  const char* ks = reinterpret_cast<const char*>(a.src_k) + so;
  const char* vs = reinterpret_cast<const char*>(a.src_v) + so;
  char* kd = reinterpret_cast<char*>(a.dst_k) + dof;
  char* vd = reinterpret_cast<char*>(a.dst_v) + dof;
  for (int off = threadIdx.x * 16; off < a.tile_bytes; off += 256 * 16) {
    const uint4 kx = *reinterpret_cast<const uint4*>(ks + off);
    const uint4 vx = *reinterpret_cast<const uint4*>(vs + off);
    *reinterpret_cast<uint4*>(kd + off) = kx;
    *reinterpret_cast<uint4*>(vd + off) = vx;
  }
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st) {
  constexpr int64_t kMaxGridX = 1 << 30;
  for (int64_t p0 = 0; p0 < a.num_pairs; p0 += kMaxGridX) {
    const int64_t n = a.num_pairs - p0 < kMaxGridX ? a.num_pairs - p0 : kMaxGridX;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, a.num_heads), dim3(256), 0, st, a, p0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
