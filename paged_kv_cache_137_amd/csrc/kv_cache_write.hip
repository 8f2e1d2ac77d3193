// KV-cache write on gfx950: scatter each new token's key and value rows into the
// physical slots that slot_mapping names.
//
// This is the fused reshape-and-block-write step of "vLLM & PagedAttention:
// Efficient Memory Management for LLM Serving", section X.  The new K/V arrive
// as [token][head][dim].  Each (token, head) row moves as one D*elem-byte run
// to cache[slot / B][head][slot % B][:] (B tokens per block), for keys and
// values in the same kernel, in one launch.
//
// Decomposition: one lane per 16-byte chunk of a (token, head) row, keys and
// values both.  A wavefront therefore reads 1 KiB of consecutive source bytes
// per load and writes whole 16-byte chunks: HBM-bound, with no conversion (a
// byte copy).  The grid is sized on the host.  Launches are split on token
// boundaries, so that every index inside one launch fits 32 bits.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int CPR>  // 16-byte chunks per (token, head) row
__global__ __launch_bounds__(256) void kv_cache_write_kernel(const WriteArgs a, int64_t tok0, int32_t nrows) {
  const int32_t g = blockIdx.x * 256 + threadIdx.x;
  const int32_t row = g / CPR;
  if (row >= nrows) return;
  const int32_t c = g % CPR;
  const int32_t tl = row / a.num_heads;
  const int32_t h = row - tl * a.num_heads;
  const int64_t t = tok0 + tl;
  const int64_t slot = a.slot_mapping[t];
  const int sh = a.block_shift;
  if (slot < 0 || slot >= (a.num_blocks << sh)) return;  // padding token, or a slot outside the pool
  const int64_t dst = ((((slot >> sh) * a.num_heads + h) << sh) + (slot & ((1 << sh) - 1))) * CPR + c;
  const int64_t src = (t * a.num_heads + h) * CPR + c;
  const uint4 kx = reinterpret_cast<const uint4*>(a.k)[src];
  const uint4 vx = reinterpret_cast<const uint4*>(a.v)[src];
  reinterpret_cast<uint4*>(a.k_cache)[dst] = kx;
  reinterpret_cast<uint4*>(a.v_cache)[dst] = vx;
}

template <int CPR>
static hipError_t write_t(const WriteArgs& a, hipStream_t st) {
  // Rows (token, head) per launch, so that nrows * CPR stays below 2^31.
  const int64_t max_tok = ((int64_t)1 << 30) / ((int64_t)a.num_heads * CPR);
  for (int64_t t0 = 0; t0 < a.num_tokens; t0 += max_tok) {
    const int64_t nt = a.num_tokens - t0 < max_tok ? a.num_tokens - t0 : max_tok;
    const int32_t nrows = (int32_t)(nt * a.num_heads);
    const int64_t threads = (int64_t)nrows * CPR;
    const int32_t grid = (int32_t)((threads + 255) / 256);
    hipLaunchKernelGGL((kv_cache_write_kernel<CPR>), dim3(grid), dim3(256), 0, st, a, t0, nrows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_kv_cache_write(const WriteArgs& a, hipStream_t st) {
  const int es = a.dtype == 0 ? 4 : 2;
  const int cpr = a.head_dim * es / 16;
  if (cpr == 8) return write_t<8>(a, st);
  if (cpr == 16) return write_t<16>(a, st);
  return write_t<32>(a, st);
}

}  // namespace pkv
