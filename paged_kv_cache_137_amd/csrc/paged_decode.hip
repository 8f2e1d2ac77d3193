// Paged decode attention on gfx950: one new query per sequence against its whole
// cached context, read block by block through the sequence's block table.
//
// The value computed is ordinary softmax attention for the last position of the
// sequence ("vLLM & PagedAttention: Efficient Memory Management for LLM
// Serving", section I, attention equation).  It is evaluated block by block
// (section III, block-wise equation), with the normaliser carried across blocks
// ("PagedAttention and vLLM, annotated", section 4.1: normalise by the total over
// all blocks so far).
//
// Work decomposition (designed for CDNA4, not taken from the pages):
//  - A unit of work is one (sequence, context partition) for NW consecutive
//    heads.  A plan kernel (one workgroup) lists the (sequence, partition)
//    pairs that hold tokens.  It sorts them by size, largest first, with a
//    counting sort, and resets a work counter.  The decode kernel is
//    persistent: one NW-wave workgroup per CU (one wave per SIMD, which
//    streams faster than full occupancy does) claims units from the counter
//    until none are left.  Empty partitions cost nothing, and
//    the ragged tail is spread over the whole GPU.  No output depends on which
//    workgroup ran which unit, so results are deterministic.
//  - Inside a unit, wave w takes head NW*g + w alone and streams all of the
//    partition's blocks for it.  A claim, the metadata lookups and the start of
//    the load pipeline are thus shared by NW heads, and the waves of a
//    workgroup, having equal block counts, stay in step between claims.
//  - A (block, head) tile is BS tokens x D values stored contiguously (BS = 16
//    by default; 8 and 32 are built too).  A wave
//    reads it with NI 16-byte loads per lane, each load instruction covering
//    1 KiB of consecutive bytes.  Lane l holds dims (l % LPT)*VEC .. +VEC of
//    token row l / LPT.  K/V are read with the nontemporal hint: every tile is
//    used once per unit, and keeping it out of the cache hierarchy's
//    retention raises the sustained HBM rate.  Partitions whose blocks the
//    plan kernel finds shared with a neighbouring sequence (parallel samples,
//    a common prefix) are read with cached loads instead, so that the other
//    sequences' reads of the same blocks hit in L2.
//  - q.k: packed dot products (v_dot2 for 16-bit inputs) over the lane's VEC
//    dims, then a DPP butterfly across the LPT lanes of the token row.  Every
//    lane of the row ends with the same score.
//  - Online softmax per token row: each lane row keeps its own running max,
//    sum and VEC accumulators, so the steady state needs no cross-row traffic.
//    The rows are merged once per unit with cross-lane shuffles, in a fixed
//    butterfly order; no LDS is used.
//  - Software pipelining: the next block's K/V loads are issued before the
//    current block is consumed (ping-pong register sets, no branch between
//    them), so two tiles per wave are in flight.
//  - Masking of slots at or past the context length is a select (-inf score,
//    zeroed V), never a multiply, so stale NaN data in those slots cannot leak.
#include <cstdlib>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Build-time alternatives, kept for measuring the choices they stand for
// (the defaults are the measured best): PKV_DEC_NW waves per workgroup,
// PKV_DEC_NT=0 for cached instead of nontemporal K/V loads (8% slower),
// PKV_DEC_PP=0 for one tile in flight per wave instead of two.
#ifndef PKV_DEC_NW
#define PKV_DEC_NW 4
#endif
#ifndef PKV_DEC_NT
#define PKV_DEC_NT 1
#endif
#ifndef PKV_DEC_PP
#define PKV_DEC_PP 1
#endif

constexpr int NW = PKV_DEC_NW;     // wavefronts per workgroup of the per-sequence decode
constexpr int SNW = 8;             // wavefronts per workgroup of the shared-prefix decode
constexpr int PLAN_BUCKETS = 257;  // partition sizes 0..256 blocks (larger ones share the top bucket)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load_kv16(const char* p) {
  if constexpr (NT && PKV_DEC_NT)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return *reinterpret_cast<const uint4*>(p);
}

template <typename E, int D, int BS>
struct DecodeGeom {
  static constexpr int ES = E::bytes;
  static constexpr int VEC = 16 / ES;      // elements per 16-byte chunk
  static constexpr int LPT = D * ES / 16;  // lanes holding one token row
  static constexpr int TPI = 64 / LPT;     // token rows per wave-wide load
  static constexpr int NI = BS / TPI;      // loads per tile
  static constexpr int TILE = BS * D * ES; // bytes of one (block, head) tile
  static_assert(TPI * LPT == 64 && NI * TPI == BS, "tile must map onto a wavefront");
  // Two register sets (load the next tile while consuming this one) while a
  // tile is small; one set for large tiles, where the registers would cost
  // more occupancy than the overlap gains.
  static constexpr bool PINGPONG = PKV_DEC_PP && NI <= 4;
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s) { return min(a.context_lens[s], a.max_context_len); }
// First token of a sequence's own partitions: past the blocks its sharing
// group reads for it (shared-prefix form), else 0.
__device__ __forceinline__ int seq_start(const DecodeArgs& a, int s) { return a.tok_start ? a.tok_start[s] : 0; }

// List every (sequence, partition) that holds tokens, largest partitions first,
// and reset the work counter.  A sequence with context_len <= 0 gets one entry
// (partition 0, in the smallest bucket) so that its output is written as NaN.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const DecodeArgs a) {
  __shared__ int cnt[PLAN_BUCKETS];
  const int BS = a.block_size;
  const int part_tokens = a.part_blocks * BS;
  const int P = a.num_parts;
  for (int i = threadIdx.x; i < PLAN_BUCKETS; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  // Pair i = (sequence i / P, partition i % P) gets a bucket (-1: no entry)
  // and its work-list entry.  All loads of a pair are independent of one
  // another except the table reads, which need the partition's first block:
  // two round trips to memory per batch of pairs.  A partition is tagged
  // shared (read with cached loads, so that the repeats hit in L2) when a
  // neighbouring sequence holds the same physical block at its first logical
  // position; the neighbours' table entries are read unconditionally (they are
  // in bounds) and used only where the neighbour's context reaches them.
  const int npairs = a.num_seqs * P;
  auto classify = [&](int i, int& bucket, int& entry) __attribute__((always_inline)) {
    bucket = -1;
    entry = 0;
    if (i >= npairs) return;
    const int s = i / P;
    const int p = i - s * P;
    const int ctx = clamp_ctx(a, s);
    const int ctx_l = s > 0 ? clamp_ctx(a, s - 1) : 0;
    const int ctx_r = s + 1 < a.num_seqs ? clamp_ctx(a, s + 1) : 0;
    const int t0 = seq_start(a, s) + p * part_tokens;
    if (ctx <= 0) {
      // One entry, in the smallest bucket, so that the output is written as NaN.
      if (p == 0) {
        bucket = 0;
        entry = (s * P) << 1;
      }
      return;
    }
    if (t0 >= ctx) return;
    const int nb = (min(part_tokens, ctx - t0) + BS - 1) / BS;
    const int lb = t0 / BS;
    const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks_per_seq + lb;
    const int mine = row[0];
    const int left = s > 0 ? row[-a.max_blocks_per_seq] : 0;
    const int right = s + 1 < a.num_seqs ? row[a.max_blocks_per_seq] : 0;
    const int shared = (ctx_l > lb * BS && left == mine) || (ctx_r > lb * BS && right == mine);
    bucket = min(nb, PLAN_BUCKETS - 1);
    entry = ((s * P + p) << 1) | shared;
  };
  // Up to R pairs per thread are classified at once (their loads overlap) and
  // kept in registers for the placement pass; larger batches classify again.
  constexpr int R = 4;
  const int per_pass = R * (int)blockDim.x;
  int bucket[R], entry[R];
  for (int base = 0; base < npairs; base += per_pass) {
#pragma unroll
    for (int k = 0; k < R; ++k) classify(base + threadIdx.x + k * (int)blockDim.x, bucket[k], entry[k]);
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (bucket[k] >= 0) atomicAdd(&cnt[bucket[k]], 1);
  }
  __syncthreads();
  // Exclusive scan of the bucket counts in descending bucket order: thread i
  // (i < PLAN_BUCKETS) owns bucket PLAN_BUCKETS-1-i.  Wave-level inclusive scans
  // with shuffles, then the earlier waves' totals are added.
  {
    __shared__ int wave_tot[(PLAN_BUCKETS + 63) / 64];
    const int i = threadIdx.x;
    const int lane = i & 63, wv = i >> 6;
    const int b = PLAN_BUCKETS - 1 - i;
    const int mine = i < PLAN_BUCKETS ? cnt[b] : 0;
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (i < PLAN_BUCKETS && lane == 63) wave_tot[wv] = incl;
    if (i == PLAN_BUCKETS - 1 && lane != 63) wave_tot[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int k = 0; k < wv && k < (PLAN_BUCKETS + 63) / 64; ++k) before += wave_tot[k];
    if (i < PLAN_BUCKETS) cnt[b] = before + incl - mine;
    if (i == PLAN_BUCKETS - 1) {
      a.work_ctrl[0] = 0;
      a.work_ctrl[1] = before + incl;
      a.work_ctrl[2] = 0;
    }
  }
  __syncthreads();
  auto place = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < R; ++k)
      if (bucket[k] >= 0) a.work_list[atomicAdd(&cnt[bucket[k]], 1)] = entry[k];
  };
  if (npairs <= per_pass) {
    place();  // the single batch is still in registers
  } else {
    for (int base = 0; base < npairs; base += per_pass) {
#pragma unroll
      for (int k = 0; k < R; ++k) classify(base + threadIdx.x + k * (int)blockDim.x, bucket[k], entry[k]);
      place();
    }
  }
}

// One (sequence, partition) unit of the per-sequence decode, for head h:
// entry e of the work list.  Called by one wave; lanes as described above.
template <typename E, typename O, int D, int BS>
__device__ __forceinline__ void private_unit(const DecodeArgs& a, int e, int h) {
  using G = DecodeGeom<E, D, BS>;
  using C = Chunk<E>;
  constexpr int VEC = G::VEC, LPT = G::LPT, TPI = G::TPI, NI = G::NI;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int H = a.num_heads;
  const int part_tokens = a.part_blocks * BS;
  const int64_t bstride = (int64_t)H * G::TILE;
  const int tagged = a.work_list[e];
  const bool reuse = tagged & 1;  // blocks shared with a neighbouring sequence
  const int entry = tagged >> 1;
  const int s = entry / a.num_parts;
  const int p = entry - s * a.num_parts;
  const int64_t sh = (int64_t)s * H + h;
  const int ctx = clamp_ctx(a, s);
  const int st0 = seq_start(a, s);
  const int tok0 = st0 + p * part_tokens;
  if (ctx <= 0) {  // undefined attention: report NaN rather than garbage
    for (int t = lane; t < D; t += 64) Out<O>::put(a.out, sh * D + t, __builtin_nanf(""));
    return;
  }
  if (tok0 >= ctx) return;
  const int nparts = (ctx - st0 + part_tokens - 1) / part_tokens;
  const bool direct = nparts == 1 && st0 == 0;  // the whole context is this unit's
  const int nblk = (min(part_tokens, ctx - tok0) + BS - 1) / BS;

  const uint4 qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) + sh * (D * G::ES) + c * 16);
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * G::TILE + lane * 16;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * G::TILE + lane * 16;
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq + tok0 / BS;

  float m = NEG_BIG, l = 0.f;
  float acc[VEC];
#pragma unroll
  for (int e2 = 0; e2 < VEC; ++e2) acc[e2] = 0.f;


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
    for (int e2 = 0; e2 < VEC; ++e2) acc[e2] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pi = fast_exp2(sc[i] - m);
      l += pi;
      float vf[VEC];
      C::unpack(vx[i], vf);
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) acc[e2] = fmaf(pi, vf[e2], acc[e2]);
    }
  };

  // The whole stream is instantiated once per load kind, so that the choice
  // is made once per unit and the loop bodies stay straight-line.
  auto run = [&](auto nt_c) {
    constexpr bool NTL = decltype(nt_c)::value;
    auto load = [&](int phys, uint4 (&kx)[NI], uint4 (&vx)[NI]) {
      const char* kp = kbase + (int64_t)phys * bstride;
      const char* vp = vbase + (int64_t)phys * bstride;
#pragma unroll
      for (int i = 0; i < NI; ++i) kx[i] = load_kv16<NTL>(kp + i * 1024);
#pragma unroll
      for (int i = 0; i < NI; ++i) vx[i] = load_kv16<NTL>(vp + i * 1024);
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
      int j = 0;
      if constexpr (G::PINGPONG) {
        uint4 kA[NI], vA[NI], kB[NI], vB[NI];
        bool badA, badB;
        load(phys_of(j, badA), kA, vA);
        while (j + 2 < cn) {
          load(phys_of(j + 1, badB), kB, vB);
          consume(kA, vA, cb + j, badA);
          load(phys_of(j + 2, badA), kA, vA);
          consume(kB, vB, cb + j + 1, badB);
          j += 2;
        }
        if (j + 1 < cn) {
          load(phys_of(j + 1, badB), kB, vB);
          consume(kA, vA, cb + j, badA);
          consume(kB, vB, cb + j + 1, badB);
        } else {
          consume(kA, vA, cb + j, badA);
        }
      } else {
        for (; j < cn; ++j) {
          uint4 kA[NI], vA[NI];
          bool badA;
          load(phys_of(j, badA), kA, vA);
          consume(kA, vA, cb + j, badA);
        }
      }
    }
  };
  if (reuse) run(std::false_type{});
  else run(std::true_type{});

  // Merge the wave's TPI token rows (lanes c, c + LPT, ... hold the same
  // dims): common maximum, rescaled sums, in a fixed butterfly order.
  float M = m;
#pragma unroll
  for (int sft = LPT; sft < 64; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft, 64));
  const float f = fast_exp2(m - M);
  float Ls = l * f;
#pragma unroll
  for (int e2 = 0; e2 < VEC; ++e2) acc[e2] *= f;
#pragma unroll
  for (int sft = LPT; sft < 64; sft <<= 1) {
    Ls += __shfl_xor(Ls, sft, 64);
#pragma unroll
    for (int e2 = 0; e2 < VEC; ++e2) acc[e2] += __shfl_xor(acc[e2], sft, 64);
  }
  if (r == 0) {
    if (direct) {
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) Out<O>::put(a.out, sh * D + c * VEC + e2, acc[e2] / Ls);
    } else {
      const int64_t pi = sh * a.num_parts + p;
      float* dst = a.ws_acc + pi * D + c * VEC;
#pragma unroll
      for (int e2 = 0; e2 < VEC; e2 += 4)
        *reinterpret_cast<float4*>(dst + e2) = make_float4(acc[e2], acc[e2 + 1], acc[e2 + 2], acc[e2 + 3]);
      if (c == 0) *reinterpret_cast<float2*>(a.ws_ml + pi * 2) = make_float2(M, Ls);
    }
  }
}

template <typename E, typename O, int D, int BS>
__global__ __launch_bounds__(NW * 64) void decode_partial_kernel(const DecodeArgs a) {
  __shared__ int sm_unit[2];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.num_heads;
  const int HG = (H + NW - 1) / NW;  // head groups
  const int total = a.work_ctrl[1] * HG;
  for (int it = 0;; ++it) {
    // Claim the next unit; the slot alternates so one barrier suffices.
    if (threadIdx.x == 0) sm_unit[it & 1] = atomicAdd(&a.work_ctrl[0], 1);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(sm_unit[it & 1]);
    if (u >= total) break;
    const int e = u / HG;
    const int h = (u - e * HG) * NW + w;
    if (h < H) private_unit<E, O, D, BS>(a, e, h);  // else a partial last head group
  }
}

// Split-context reduce: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// M = max_p m_p, with p ascending.  Sequences that fit one partition were
// finished by the partial kernel and are skipped.
template <typename O, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int ctx = clamp_ctx(a, s);
  if (ctx <= 0) return;
  const int part_tokens = a.part_blocks * a.block_size;
  const int nparts = (ctx + part_tokens - 1) / part_tokens;
  if (nparts <= 1) return;
  const int t = threadIdx.x;
  const int64_t sh = (int64_t)s * a.num_heads + h;
  const int64_t base = sh * a.num_parts;
  // Up to RP partitions: every (m, l) and partial value is loaded at once, so
  // the merge waits for memory once.  The arithmetic and its order are the
  // same either way.
  constexpr int RP = 8;
  if (nparts <= RP) {
    float mp[RP], lp[RP], ap[RP];
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      if (p < nparts) {
        const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (base + p) * 2);
        mp[p] = ml.x;
        lp[p] = ml.y;
        ap[p] = a.ws_acc[(base + p) * D + t];
      }
    }
    float M = mp[0];
#pragma unroll
    for (int p = 1; p < RP; ++p)
      if (p < nparts) M = fmaxf(M, mp[p]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      if (p < nparts) {
        const float f = fast_exp2(mp[p] - M);
        Ls = fmaf(lp[p], f, Ls);
        A = fmaf(ap[p], f, A);
      }
    }
    Out<O>::put(a.out, sh * D + t, A / Ls);
    return;
  }
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

// ---------------------------------------------------------------------------
// Shared-prefix decode.  Parallel samples of one request, or requests with a
// common prefix, hold the same physical blocks at the start of their tables
// ("vLLM & PagedAttention ...", section VII: shared blocks with reference
// counts).  Reading such a block once for all the sequences that hold it, with
// one query per sequence, gives the same attention with fewer bytes.
//
// Sequences are taken in windows of SHARE_WINDOW consecutive ones.  The
// leader of a window is its first sequence that holds a full block; the
// members are the window's sequences whose first block id is the leader's.
// J is the number of leading full blocks that every member holds with the
// leader's ids, all inside every member's context.  A window with two or more
// members and J >= 1 is a group.  decode_shared_kernel reads a group's J
// blocks once, in partitions (group units), writing one partial result per
// member, and runs each member's tokens J*BS .. ctx-1 as ordinary
// per-sequence units (tok_start); the reduce merges both kinds of partial
// results.

// One wave per window.
__global__ __launch_bounds__(1024) void share_detect_kernel(const DecodeArgs a) {
  constexpr int GW = SHARE_WINDOW;
  const int lane = threadIdx.x & 63;
  const int win = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (win >= a.num_windows) return;
  const int BS = a.block_size;
  const int s0 = win * GW;
  int nfull[GW];
  const int32_t* rows[GW];
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    const int s = s0 + i;
    nfull[i] = s < a.num_seqs ? max(clamp_ctx(a, s), 0) / BS : 0;
    rows[i] = a.block_tables + (int64_t)min(s, a.num_seqs - 1) * a.max_blocks_per_seq;
  }
  int lead = -1;
#pragma unroll
  for (int i = GW - 1; i >= 0; --i)
    if (nfull[i] >= 1) lead = i;
  int mask = 0, J = 0;
  if (lead >= 0) {
    const int32_t* lrow = a.block_tables + (int64_t)(s0 + lead) * a.max_blocks_per_seq;
    const int first = lrow[0];
    int lim = nfull[lead];
    mask = 1 << lead;
#pragma unroll
    for (int i = 0; i < GW; ++i)
      if (i != lead && nfull[i] >= 1 && rows[i][0] == first) {
        mask |= 1 << i;
        lim = min(lim, nfull[i]);
      }
    if (__builtin_popcount(mask) >= 2) {
      // The first block where some member's id differs from the leader's.
      J = lim;
      for (int j0 = 0; j0 < lim; j0 += 64) {
        const int j = j0 + lane;
        bool diff = false;
        if (j < lim) {
          const int lv = lrow[j];
#pragma unroll
          for (int i = 0; i < GW; ++i)
            if ((mask >> i) & 1) diff |= rows[i][j] != lv;
        }
        const unsigned long long b = __ballot(diff);
        if (b != 0ull) {
          J = j0 + __builtin_ctzll(b);
          break;
        }
      }
    }
  }
  const bool grp = __builtin_popcount(mask) >= 2 && J >= 1;
  if (lane == 0) a.win_info[win] = grp ? (J << 4) | mask : 0;
  if (lane < GW && s0 + lane < a.num_seqs) a.tok_start[s0 + lane] = grp && ((mask >> lane) & 1) ? J * BS : 0;
}

// One group unit: entry e = (window, partition of the shared blocks), head h.
// The wave streams head h of the group's shared blocks once and keeps one
// online softmax per member (its own query), with the same lane layout as
// decode_partial_kernel.  Every shared block is full and inside every
// member's context, so no slot is masked.
template <typename E, typename O, int D, int BS>
__device__ __forceinline__ void group_unit(const DecodeArgs& a, int e, int h) {
  using G = DecodeGeom<E, D, BS>;
  using C = Chunk<E>;
  constexpr int VEC = G::VEC, LPT = G::LPT, NI = G::NI;
  constexpr int GW = SHARE_WINDOW;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int H = a.num_heads;
  const int part_tokens = a.part_blocks * BS;
  const int64_t bstride = (int64_t)H * G::TILE;
  const int win = e / a.num_parts;
  const int p = e - win * a.num_parts;
  const int info = __builtin_amdgcn_readfirstlane(a.win_info[win]);
  if (info == 0) return;
  const int J = info >> 4, mask = info & 15;
  const int tok0 = p * part_tokens;
  const int tend = min(tok0 + part_tokens, J * BS);
  if (tok0 >= tend) return;
  const int nblk = (tend - tok0) / BS;
  const int s0 = win * GW;

  uint4 qv[GW];
  float m[GW], l[GW], acc[GW][VEC];
#pragma unroll
  for (int i = 0; i < GW; ++i) {
    qv[i] = make_uint4(0u, 0u, 0u, 0u);
    if ((mask >> i) & 1)
      qv[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) +
                                              ((int64_t)(s0 + i) * H + h) * (D * G::ES) + c * 16);
    m[i] = NEG_BIG;
    l[i] = 0.f;
#pragma unroll
    for (int e2 = 0; e2 < VEC; ++e2) acc[i][e2] = 0.f;
  }
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * G::TILE + lane * 16;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * G::TILE + lane * 16;
  const int lead = __builtin_ctz(mask);
  const int32_t* trow = a.block_tables + (int64_t)(s0 + lead) * a.max_blocks_per_seq + tok0 / BS;

  // Where 16 lanes hold a token row and a tile takes at most four loads, every
  // member slot is computed, present or not (an absent member has q = 0 and
  // its results are never stored): one branch-free body lets the compiler
  // interleave the members' dependency chains (measured 3% faster at 128
  // dims, 16-bit, 16-token blocks).  Elsewhere absent members are skipped,
  // which keeps the register count, and so the occupancy, where it was.
  constexpr bool ALL_MEMBERS = NI <= 4 && LPT == 16;
  auto consume = [&](const uint4 (&kx)[NI], const uint4 (&vx)[NI], bool bad) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      if constexpr (!ALL_MEMBERS) {
        if (!((mask >> g) & 1)) continue;
      }
      float sc[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) sc[i] = group_sum<LPT>(C::dot(qv[g], kx[i])) * a.scale_log2;
      if (bad) {
#pragma unroll
        for (int i = 0; i < NI; ++i) sc[i] = __builtin_nanf("");
      }
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < NI; ++i) mx = fmaxf(mx, sc[i]);
      const float alpha = fast_exp2(m[g] - mx);
      m[g] = mx;
      l[g] *= alpha;
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) acc[g][e2] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pi = fast_exp2(sc[i] - mx);
        l[g] += pi;
        float vf[VEC];
        C::unpack(vx[i], vf);
#pragma unroll
        for (int e2 = 0; e2 < VEC; ++e2) acc[g][e2] = fmaf(pi, vf[e2], acc[g][e2]);
      }
    }
  };
  auto load = [&](int phys, uint4 (&kx)[NI], uint4 (&vx)[NI]) {
    const char* kp = kbase + (int64_t)phys * bstride;
    const char* vp = vbase + (int64_t)phys * bstride;
#pragma unroll
    for (int i = 0; i < NI; ++i) kx[i] = load_kv16<true>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) vx[i] = load_kv16<true>(vp + i * 1024);
  };
  for (int cb = 0; cb < nblk; cb += 64) {
    const int cn = min(64, nblk - cb);
    const int tv = lane < cn ? trow[cb + lane] : 0;
    auto phys_of = [&](int j, bool& bad) {
      const int ph = __builtin_amdgcn_readlane(tv, j);
      bad = (uint64_t)(uint32_t)ph >= (uint64_t)a.num_blocks;
      return bad ? 0 : ph;
    };
    int j = 0;
    // One tile in flight: the members' accumulators take the registers a
    // second set would need, and the kernel keeps the occupancy of the
    // per-sequence units it shares.
    for (; j < cn; ++j) {
      uint4 kA[NI], vA[NI];
      bool badA;
      load(phys_of(j, badA), kA, vA);
      consume(kA, vA, badA);
    }
  }

  // Per member: merge the wave's token rows, then store the partial result.
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    if (!((mask >> g) & 1)) continue;
    float M = m[g];
#pragma unroll
    for (int sft = LPT; sft < 64; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft, 64));
    const float f = fast_exp2(m[g] - M);
    float Ls = l[g] * f;
    float av[VEC];
#pragma unroll
    for (int e2 = 0; e2 < VEC; ++e2) av[e2] = acc[g][e2] * f;
#pragma unroll
    for (int sft = LPT; sft < 64; sft <<= 1) {
      Ls += __shfl_xor(Ls, sft, 64);
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) av[e2] += __shfl_xor(av[e2], sft, 64);
    }
    if (r == 0) {
      const int64_t pi = ((int64_t)(s0 + g) * H + h) * a.num_parts + p;
      float* dst = a.ws_acc_sh + pi * D + c * VEC;
#pragma unroll
      for (int e2 = 0; e2 < VEC; e2 += 4)
        *reinterpret_cast<float4*>(dst + e2) = make_float4(av[e2], av[e2 + 1], av[e2 + 2], av[e2 + 3]);
      if (c == 0) *reinterpret_cast<float2*>(a.ws_ml_sh + pi * 2) = make_float2(M, Ls);
    }
  }
}

// Persistent kernel of the shared-prefix form: the group units (window,
// partition of the shared blocks, SNW heads) first, then the per-sequence
// units of the plan's list, claimed from one counter, so that the two kinds
// fill each other's gaps.
template <typename E, typename O, int D, int BS>
__global__ __launch_bounds__(SNW * 64) void decode_shared_kernel(const DecodeArgs a) {
  __shared__ int sm_unit[2];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.num_heads;
  const int HG = (H + SNW - 1) / SNW;
  const int ng = a.num_windows * a.num_parts * HG;
  const int total = ng + a.work_ctrl[1] * HG;
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) sm_unit[it & 1] = atomicAdd(&a.work_ctrl[0], 1);
    __syncthreads();
    int u = __builtin_amdgcn_readfirstlane(sm_unit[it & 1]);
    if (u >= total) break;
    const bool grp = u < ng;
    if (!grp) u -= ng;
    const int e = u / HG;
    const int h = (u - e * HG) * SNW + w;
    if (h >= H) continue;  // a partial last head group
    if (grp) group_unit<E, O, D, BS>(a, e, h);
    else private_unit<E, O, D, BS>(a, e, h);
  }
}

// Merge of the shared-prefix form: the group's partial results over the
// shared blocks (partitions ascending), then the sequence's own (ascending).
// A sequence outside any group with one partition was finished by the
// partial kernel.
template <typename O, int D>
__global__ __launch_bounds__(D) void decode_reduce_shared_kernel(const DecodeArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int ctx = clamp_ctx(a, s);
  if (ctx <= 0) return;
  const int part_tokens = a.part_blocks * a.block_size;
  const int st0 = a.tok_start[s];
  const int nsh = (st0 + part_tokens - 1) / part_tokens;
  const int npriv = (ctx - st0 + part_tokens - 1) / part_tokens;
  if (st0 == 0 && npriv <= 1) return;
  const int t = threadIdx.x;
  const int64_t sh = (int64_t)s * a.num_heads + h;
  const int64_t base = sh * a.num_parts;
  float M = NEG_BIG;
  for (int p = 0; p < nsh; ++p) M = fmaxf(M, a.ws_ml_sh[(base + p) * 2]);
  for (int p = 0; p < npriv; ++p) M = fmaxf(M, a.ws_ml[(base + p) * 2]);
  float Ls = 0.f, A = 0.f;
  for (int p = 0; p < nsh; ++p) {
    const float f = fast_exp2(a.ws_ml_sh[(base + p) * 2] - M);
    Ls = fmaf(a.ws_ml_sh[(base + p) * 2 + 1], f, Ls);
    A = fmaf(a.ws_acc_sh[(base + p) * D + t], f, A);
  }
  for (int p = 0; p < npriv; ++p) {
    const float f = fast_exp2(a.ws_ml[(base + p) * 2] - M);
    Ls = fmaf(a.ws_ml[(base + p) * 2 + 1], f, Ls);
    A = fmaf(a.ws_acc[(base + p) * D + t], f, A);
  }
  Out<O>::put(a.out, sh * D + t, A / Ls);
}

// Workgroups of a persistent kernel: per_cu on every CU of the device (at
// most the kernel's occupancy), never more than there are units.  The CU
// count and the occupancy are cached per kernel and device.
template <auto KERNEL>
static int persistent_grid(int block, int64_t units, int per_cu) {
  constexpr int kMaxDev = 64;
  static int cus_occ[kMaxDev][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int cus = dev < kMaxDev ? cus_occ[dev][0] : 0, occ = dev < kMaxDev ? cus_occ[dev][1] : 0;
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, KERNEL, block, 0) != hipSuccess || occ <= 0) occ = 1;
    if (dev < kMaxDev) {
      cus_occ[dev][0] = cus;
      cus_occ[dev][1] = occ;
    }
  }
  const int64_t n = (int64_t)cus * (occ < per_cu ? occ : per_cu);
  return (int)(units < n ? units : n);
}

// Workgroups per CU of the per-sequence decode: 1, or the value of the
// environment variable PKV_DECODE_WG_PER_CU (1 to 16; read at every launch,
// for measuring other launch shapes).
static int decode_wg_per_cu() {
  const char* e = std::getenv("PKV_DECODE_WG_PER_CU");
  if (e == nullptr) return 1;
  const int v = std::atoi(e);
  return v >= 1 && v <= 16 ? v : 1;
}

template <typename E, typename O, int D, int BS>
static hipError_t partial_bs(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, st, a);
  // One workgroup per CU: one wave per SIMD, two tiles in flight per wave.
  // On MI355X this streams the gathered tiles faster than running the
  // kernel at its full occupancy (measured 4% faster on the Llama-2-7B-shape
  // step and 11% on the OPT-13B-shape one): more outstanding requests lower
  // the HBM rate of this random 4 KiB-tile stream instead of raising it.
  const int grid = persistent_grid<decode_partial_kernel<E, O, D, BS>>(NW * 64, ((int64_t)a.total_units + NW - 1) / NW,
                                                                       decode_wg_per_cu());
  hipLaunchKernelGGL((decode_partial_kernel<E, O, D, BS>), dim3(grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

template <typename E, typename O, int D>
static hipError_t partial_t(const DecodeArgs& a, hipStream_t st) {
  if (a.block_size == 8) return partial_bs<E, O, D, 8>(a, st);
  if (a.block_size == 32) return partial_bs<E, O, D, 32>(a, st);
  return partial_bs<E, O, D, 16>(a, st);
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

template <typename E, typename O, int D, int BS>
static hipError_t shared_bs(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(share_detect_kernel, dim3((a.num_windows + 15) / 16), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, st, a);
  const int64_t units = ((int64_t)a.num_windows * a.num_parts + a.total_units) * ((a.num_heads + SNW - 1) / SNW);
  // One 8-wave workgroup per CU (two waves per SIMD): a unit covers 8 heads,
  // and the group units' arithmetic (four queries per tile) gets a second wave
  // per SIMD.  Measured faster than 4-wave workgroups at one, two or four per
  // CU.
  const int grid = persistent_grid<decode_shared_kernel<E, O, D, BS>>(SNW * 64, units, 1);
  hipLaunchKernelGGL((decode_shared_kernel<E, O, D, BS>), dim3(grid), dim3(SNW * 64), 0, st, a);
  return hipGetLastError();
}

template <typename E, typename O, int D>
static hipError_t shared_t(const DecodeArgs& a, hipStream_t st) {
  if (a.block_size == 8) return shared_bs<E, O, D, 8>(a, st);
  if (a.block_size == 32) return shared_bs<E, O, D, 32>(a, st);
  return shared_bs<E, O, D, 16>(a, st);
}

template <typename E, int D>
static hipError_t shared_out(const DecodeArgs& a, int out_dtype, hipStream_t st) {
  if (out_dtype == 0) return shared_t<E, f32_t, D>(a, st);
  return shared_t<E, E, D>(a, st);
}

hipError_t launch_decode_shared_partial(const DecodeArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128) {
    if (dtype == 0) return shared_t<f32_t, f32_t, 128>(a, st);
    if (dtype == 1) return shared_out<f16_t, 128>(a, out_dtype, st);
    return shared_out<bf16_t, 128>(a, out_dtype, st);
  }
  if (dtype == 0) return shared_t<f32_t, f32_t, 64>(a, st);
  if (dtype == 1) return shared_out<f16_t, 64>(a, out_dtype, st);
  return shared_out<bf16_t, 64>(a, out_dtype, st);
}

template <typename O, int D>
static hipError_t reduce_shared_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_reduce_shared_kernel<O, D>), dim3(a.num_seqs, a.num_heads), dim3(D), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_shared_reduce(const DecodeArgs& a, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128) {
    if (out_dtype == 0) return reduce_shared_t<f32_t, 128>(a, st);
    if (out_dtype == 1) return reduce_shared_t<f16_t, 128>(a, st);
    return reduce_shared_t<bf16_t, 128>(a, st);
  }
  if (out_dtype == 0) return reduce_shared_t<f32_t, 64>(a, st);
  if (out_dtype == 1) return reduce_shared_t<f16_t, 64>(a, st);
  return reduce_shared_t<bf16_t, 64>(a, st);
}

}  // namespace pkv
