// Paged decode attention on gfx950: one new query per sequence against its whole
// cached context, read block by block through the sequence's block table.
//
// The value computed is ordinary softmax attention for the last position of the
// sequence ("vLLM & PagedAttention: Efficient Memory Management for LLM
// Serving", section I, attention equation).  It is evaluated block by block
// (section III, block-wise equation), with the normaliser carried across blocks
// ("PagedAttention and vLLM, annotated", section 4.1: "normalize by the total
// over all blocks so far").
//
// Work decomposition (designed for CDNA4, not taken from the pages):
//  - One workgroup of 4 wavefronts per (sequence, head, context partition).
//    Wave w takes the partition's blocks w, w+4, w+8, ... so a short last
//    partition still spreads over all waves.
//  - A (block, head) tile is 16 tokens x D values stored contiguously.  A wave
//    reads it with NI 16-byte loads per lane, each load instruction covering
//    1 KiB of consecutive bytes.  Lane l holds dims (l % LPT)*VEC .. +VEC of
//    token row l / LPT.
//  - q.k: packed dot products (v_dot2 for 16-bit inputs) over the lane's VEC
//    dims, then a DPP butterfly across the LPT lanes of the token row.  Every
//    lane of the row ends with the same score.
//  - Online softmax per token row: each lane row keeps its own running max,
//    sum and VEC accumulators, so the steady state needs no cross-row traffic.
//    Rows and waves are merged once, through LDS, at the end of the partition.
//  - Software pipelining: the next block's K/V loads are issued before the
//    current block is consumed (ping-pong register sets, no branch between
//    them), so two tiles per wave are in flight.
//  - Masking of slots at or past the context length is a select (-inf score,
//    zeroed V), never a multiply, so stale NaN data in those slots cannot leak.
//  - Grid order: unit u = p + P*(s + S*h).  The hardware workgroup id is
//    remapped so that each XCD walks a contiguous range of units.  The
//    partitions of one sequence, and neighbouring sequences that share blocks,
//    then run on the same XCD and hit its L2.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int BS = 16;  // tokens per block
constexpr int NW = 4;   // wavefronts per workgroup

template <typename E, int D>
struct DecodeGeom {
  static constexpr int ES = E::bytes;
  static constexpr int VEC = 16 / ES;      // elements per 16-byte chunk
  static constexpr int LPT = D * ES / 16;  // lanes holding one token row
  static constexpr int TPI = 64 / LPT;     // token rows per wave-wide load
  static constexpr int NI = BS / TPI;      // loads per tile
  static constexpr int TILE = BS * D * ES; // bytes of one (block, head) tile
  static_assert(TPI * LPT == 64 && NI * TPI == BS, "tile must map onto a wavefront");
};

template <typename E, typename O, int D>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(const DecodeArgs a) {
  using G = DecodeGeom<E, D>;
  using C = Chunk<E>;
  constexpr int VEC = G::VEC, LPT = G::LPT, TPI = G::TPI, NI = G::NI;
  constexpr int ROWS = NW * TPI;  // online-softmax states per workgroup

  __shared__ float sm_m[ROWS];
  __shared__ float sm_l[ROWS];
  __shared__ __attribute__((aligned(16))) float sm_acc[ROWS][D];

  const int wg = blockIdx.x;
  const int u = (wg & 7) * a.per_xcd + (wg >> 3);
  if (u >= a.total_units) return;
  const int p = u % a.num_parts;
  const int su = u / a.num_parts;
  const int s = su % a.num_seqs;
  const int h = su / a.num_seqs;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPT;
  const int c = lane % LPT;

  const int64_t sh = (int64_t)s * a.num_heads + h;
  const int ctx = min(a.context_lens[s], a.max_context_len);
  const int part_tokens = a.part_blocks * BS;
  const int tok0 = p * part_tokens;
  if (ctx <= 0) {  // undefined attention: report NaN rather than garbage
    if (p == 0 && threadIdx.x < D) Out<O>::put(a.out, sh * D + threadIdx.x, __builtin_nanf(""));
    return;
  }
  if (tok0 >= ctx) return;
  const int nparts = (ctx + part_tokens - 1) / part_tokens;
  const int nblk = (min(part_tokens, ctx - tok0) + BS - 1) / BS;

  const uint4 qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) + sh * (D * G::ES) + c * 16);

  const int64_t bstride = (int64_t)a.num_heads * G::TILE;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * G::TILE + lane * 16;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * G::TILE + lane * 16;
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq + tok0 / BS;

  float m = NEG_BIG, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  auto load = [&](int phys, uint4 (&kx)[NI], uint4 (&vx)[NI]) {
    const char* kp = kbase + (int64_t)phys * bstride;
    const char* vp = vbase + (int64_t)phys * bstride;
#pragma unroll
    for (int i = 0; i < NI; ++i) kx[i] = *reinterpret_cast<const uint4*>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) vx[i] = *reinterpret_cast<const uint4*>(vp + i * 1024);
  };

  auto consume = [&](const uint4 (&kx)[NI], uint4 (&vx)[NI], int jb, bool bad) {
    const int tb = tok0 + jb * BS;  // position of the block's first token
    float sc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) sc[i] = group_sum<LPT>(C::dot(qv, kx[i])) * a.scale_log2;
    if (tb + BS > ctx) {  // partly filled last block
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool dead = tb + i * TPI + r >= ctx;
        sc[i] = dead ? -INFINITY : sc[i];
        vx[i] = dead ? make_uint4(0u, 0u, 0u, 0u) : vx[i];
      }
    }
    if (bad) {
#pragma unroll
      for (int i = 0; i < NI; ++i) sc[i] = __builtin_nanf("");
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < NI; ++i) mx = fmaxf(mx, sc[i]);
    const float alpha = fast_exp2(m - mx);
    m = mx;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pi = fast_exp2(sc[i] - m);
      l += pi;
      float vf[VEC];
      C::unpack(vx[i], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fmaf(pi, vf[e], acc[e]);
    }
  };

  for (int cb = 0; cb < nblk; cb += 64) {
    const int cn = min(64, nblk - cb);
    // The chunk's table entries, one per lane; a wave-uniform readlane picks each.
    const int tv = lane < cn ? trow[cb + lane] : 0;
    auto phys_of = [&](int j, bool& bad) {
      const int ph = __builtin_amdgcn_readlane(tv, j);
      bad = (uint64_t)(uint32_t)ph >= (uint64_t)a.num_blocks;
      return bad ? 0 : ph;
    };
    int j = w;
    if (j >= cn) continue;
    uint4 kA[NI], vA[NI], kB[NI], vB[NI];
    bool badA, badB;
    load(phys_of(j, badA), kA, vA);
    while (j + 2 * NW < cn) {
      load(phys_of(j + NW, badB), kB, vB);
      consume(kA, vA, cb + j, badA);
      load(phys_of(j + 2 * NW, badA), kA, vA);
      consume(kB, vB, cb + j + NW, badB);
      j += 2 * NW;
    }
    if (j + NW < cn) {
      load(phys_of(j + NW, badB), kB, vB);
      consume(kA, vA, cb + j, badA);
      consume(kB, vB, cb + j + NW, badB);
    } else {
      consume(kA, vA, cb + j, badA);
    }
  }

  // Merge the ROWS running states of this partition: max, rescaled sums.
  if (c == 0) {
    sm_m[w * TPI + r] = m;
    sm_l[w * TPI + r] = l;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sm_acc[w * TPI + r][c * VEC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int t = threadIdx.x;
    float M = sm_m[0];
#pragma unroll
    for (int k = 1; k < ROWS; ++k) M = fmaxf(M, sm_m[k]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      const float f = fast_exp2(sm_m[k] - M);
      Ls = fmaf(sm_l[k], f, Ls);
      A = fmaf(sm_acc[k][t], f, A);
    }
    if (nparts == 1) {
      Out<O>::put(a.out, sh * D + t, A / Ls);
    } else {
      const int64_t pi = sh * a.num_parts + p;
      a.ws_acc[pi * D + t] = A;
      if (t == 0) {
        a.ws_ml[pi * 2] = M;
        a.ws_ml[pi * 2 + 1] = Ls;
      }
    }
  }
}

// Split-context reduce: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// M = max_p m_p, with p ascending.  Sequences that fit one partition were
// finished by the partial kernel and are skipped.
template <typename O, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int ctx = min(a.context_lens[s], a.max_context_len);
  if (ctx <= 0) return;
  const int part_tokens = a.part_blocks * BS;
  const int nparts = (ctx + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;
  const int t = threadIdx.x;
  const int64_t sh = (int64_t)s * a.num_heads + h;
  const int64_t base = sh * a.num_parts;
  float M = a.ws_ml[base * 2];
  for (int p = 1; p < nparts; ++p) M = fmaxf(M, a.ws_ml[(base + p) * 2]);
  float Ls = 0.f, A = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float f = fast_exp2(a.ws_ml[(base + p) * 2] - M);
    Ls = fmaf(a.ws_ml[(base + p) * 2 + 1], f, Ls);
    A = fmaf(a.ws_acc[(base + p) * D + t], f, A);
  }
  Out<O>::put(a.out, sh * D + t, A / Ls);
}

template <typename E, typename O, int D>
static hipError_t partial_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_partial_kernel<E, O, D>), dim3(a.per_xcd * 8), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <typename O, int D>
static hipError_t reduce_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_reduce_kernel<O, D>), dim3(a.num_seqs, a.num_heads), dim3(D), 0, st, a);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t partial_out(const DecodeArgs& a, int out_dtype, hipStream_t st) {
  if (out_dtype == 0) return partial_t<E, f32_t, D>(a, st);
  return partial_t<E, E, D>(a, st);
}

// dtype codes follow pkv_dtype: 0 = f32, 1 = f16, 2 = bf16.
hipError_t launch_decode_partial(const DecodeArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128) {
    if (dtype == 0) return partial_t<f32_t, f32_t, 128>(a, st);
    if (dtype == 1) return partial_out<f16_t, 128>(a, out_dtype, st);
    return partial_out<bf16_t, 128>(a, out_dtype, st);
  }
  if (dtype == 0) return partial_t<f32_t, f32_t, 64>(a, st);
  if (dtype == 1) return partial_out<f16_t, 64>(a, out_dtype, st);
  return partial_out<bf16_t, 64>(a, out_dtype, st);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128) {
    if (out_dtype == 0) return reduce_t<f32_t, 128>(a, st);
    if (out_dtype == 1) return reduce_t<f16_t, 128>(a, st);
    return reduce_t<bf16_t, 128>(a, st);
  }
  if (out_dtype == 0) return reduce_t<f32_t, 64>(a, st);
  if (out_dtype == 1) return reduce_t<f16_t, 64>(a, st);
  return reduce_t<bf16_t, 64>(a, st);
}

}  // namespace pkv
