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
//  - A unit of work covers NW consecutive heads of one (sequence, context
//    partition), or of one partition of the leading blocks that a group of
//    neighbouring sequences share (parallel samples, a common prefix: the same
//    physical ids at the start of their tables, "vLLM & PagedAttention ...",
//    section VII).  A group unit reads those blocks once and keeps one online
//    softmax per member's query.
//  - A plan kernel (one workgroup) finds the groups, lists the units that
//    hold tokens and sorts them by size, largest first, with a counting sort.  The
//    decode kernel is persistent: one NW-wave workgroup per CU (one wave per
//    SIMD, which streams faster than full occupancy does) claims units from a
//    counter until none are left.  Empty partitions cost nothing, and the ragged
//    tail is spread over the whole GPU.
//  - A sequence whose context is one unit writes its output directly; so do
//    a group's members when contexts are not split (the group unit then also
//    streams each member's own blocks).  The others write one partial result
//    (running max, sum, unnormalised output) per unit, and a reduce kernel
//    merges them in a fixed order, so no output depends on which workgroup ran
//    which unit.
//  - Inside a unit, wave w takes head NW*g + w alone and streams all of the
//    partition's blocks for it.  A claim, the metadata lookups and the start of
//    the load pipeline are thus shared by NW heads.
//  - A (block, head) tile is BS tokens x D values stored contiguously (BS = 16
//    by default; 8 and 32 are built too).  A wave reads it with NI 16-byte loads
//    per lane, each load instruction covering 1 KiB of consecutive bytes.  Lane
//    l holds dims (l % LPT)*VEC .. +VEC of token row l / LPT.  K/V are read with
//    the nontemporal hint: every tile is used once per unit, and keeping it out
//    of the cache hierarchy's retention raises the sustained HBM rate.
//    Partitions whose first block a neighbouring sequence also holds outside a
//    group are read with cached loads instead, so that the neighbour's read of
//    the same block hits in L2.
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

constexpr int NW = 4;              // wavefronts (heads) per workgroup of the decode
constexpr int PLAN_BUCKETS = 257;  // partition sizes 0..256 blocks (larger ones share the top bucket)

// Work-list entries: (index << ENTRY_SHIFT) | flags.  The index is
// sequence * P + partition for a sequence's own units, window * P + partition
// for a group unit.
constexpr int ENTRY_REUSE = 1;  // read with cached loads (a neighbour reads the same first block)
constexpr int ENTRY_GROUP = 2;  // a group unit
constexpr int ENTRY_SHIFT = 2;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ uint4 load_kv16(const char* p) {
  if constexpr (NT)
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
  static constexpr bool PINGPONG = NI <= 4;
};

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s) { return min(a.context_lens[s], a.max_context_len); }
// First token of a sequence's own partitions: past the blocks its sharing
// group reads for it, else 0.
__device__ __forceinline__ int seq_start(const DecodeArgs& a, int s) { return a.tok_start ? a.tok_start[s] : 0; }
// Partitions of a sequence's shared leading blocks (read by its group's units).
__device__ __forceinline__ int shared_parts(const DecodeArgs& a, int s, int part_tokens) {
  return (seq_start(a, s) + part_tokens - 1) / part_tokens;
}

// Sharing, found by the plan workgroup.  Sequences are taken in windows of
// SHARE_WINDOW consecutive ones.  The leader of a window is its first sequence
// holding a full block; the members are the window's sequences whose first
// block id is the leader's; J is the number of leading full blocks that every
// member holds with the leader's ids, all inside every member's context.  With
// two or more members and J >= 1 the window is a group: win_info =
// (J << 4) | member mask, and each member's own tokens start at J * block_size.
// Otherwise win_info = 0 and they start at 0.
// Windows are handled in passes of DET_CAP.  In a pass, one thread per window
// finds the leader, the members and the fewest full blocks among them (lim);
// windows with fewer than two members are settled.  The others' J is the first
// block, below lim, where some member's id differs from the leader's: threads
// take (window, block) pairs, 64 blocks per round, and keep the minimum in LDS.
constexpr int DET_CAP = 1024;
struct DetectLds {
  int win[DET_CAP], lead[DET_CAP], mask[DET_CAP], lim[DET_CAP], J[DET_CAP];
  int ncand, maxlim;
};
// Batches of up to PLAN_SEQ_CAP sequences (one detection pass) keep each
// sequence's clamped context length, first block id and first own token, and
// each window's win_info, in the plan workgroup's LDS: one round trip to memory
// fills them, and detection and classification then read LDS.  Larger batches
// read memory each time.
constexpr int PLAN_SEQ_CAP = DET_CAP * SHARE_WINDOW;
struct PlanSeqLds {
  int ctx[PLAN_SEQ_CAP], first[PLAN_SEQ_CAP], start[PLAN_SEQ_CAP], winfo[DET_CAP];
};

__device__ void detect_all(const DecodeArgs& a, DetectLds& d, PlanSeqLds& L, bool cached) {
  constexpr int GW = SHARE_WINDOW;
  const int BS = a.block_size;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  for (int w0 = 0; w0 < a.num_windows; w0 += DET_CAP) {
    if (tid == 0) {
      d.ncand = 0;
      d.maxlim = 0;
    }
    __syncthreads();
    for (int k = tid; k < DET_CAP && w0 + k < a.num_windows; k += nthr) {
      const int win = w0 + k;
      const int s0 = win * GW;
      int nfull[GW], first[GW];
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int s = s0 + i;
        const int ctx = s < a.num_seqs ? (cached ? L.ctx[s] : clamp_ctx(a, s)) : 0;
        nfull[i] = max(ctx, 0) / BS;
        first[i] = s < a.num_seqs ? (cached ? L.first[s] : a.block_tables[(int64_t)s * a.max_blocks_per_seq]) : 0;
      }
      int lead = -1;
#pragma unroll
      for (int i = GW - 1; i >= 0; --i)
        if (nfull[i] >= 1) lead = i;
      int mask = 0, lim = 0;
      if (lead >= 0) {
        int fl = first[0], nl = nfull[0];
#pragma unroll
        for (int i = 1; i < GW; ++i)
          if (i == lead) {
            fl = first[i];
            nl = nfull[i];
          }
        lim = nl;
#pragma unroll
        for (int i = 0; i < GW; ++i)
          if (nfull[i] >= 1 && first[i] == fl) {
            mask |= 1 << i;
            lim = min(lim, nfull[i]);
          }
      }
      if (__builtin_popcount(mask) >= 2) {
        const int c = atomicAdd(&d.ncand, 1);
        d.win[c] = win;
        d.lead[c] = s0 + lead;
        d.mask[c] = mask;
        d.lim[c] = lim;
        d.J[c] = lim;
        atomicMax(&d.maxlim, lim);
      } else {
        a.win_info[win] = 0;
        if (cached) L.winfo[win] = 0;
#pragma unroll
        for (int i = 0; i < GW; ++i)
          if (s0 + i < a.num_seqs) {
            a.tok_start[s0 + i] = 0;
            if (cached) L.start[s0 + i] = 0;
          }
      }
    }
    __syncthreads();
    const int nc = d.ncand;
    const int maxlim = d.maxlim;
    // Each thread takes up to four (window, block) pairs at once and issues all
    // their table reads before comparing, so the reads overlap.
    constexpr int QB = 4;
    for (int jr = 0; jr < maxlim; jr += 64) {
      const int total = nc * 64;
      for (int q0 = tid; q0 < total; q0 += QB * nthr) {
        int lv[QB], wv[QB][GW];
        bool act[QB];
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int q = q0 + u * nthr;
          const int c = min(q >> 6, nc - 1);
          const int j = jr + (q & 63);
          // d.J only shrinks; a stale read costs a redundant check
          act[u] = q < total && j < d.lim[c] && j < d.J[c];
          const int32_t* lrow = a.block_tables + (int64_t)d.lead[c] * a.max_blocks_per_seq;
          const int32_t* wrow = a.block_tables + (int64_t)d.win[c] * GW * a.max_blocks_per_seq;
          const int mask = d.mask[c];
          lv[u] = act[u] ? lrow[j] : 0;
#pragma unroll
          for (int i = 0; i < GW; ++i)
            wv[u][i] = act[u] && ((mask >> i) & 1) ? wrow[(int64_t)i * a.max_blocks_per_seq + j] : 0;
        }
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          if (!act[u]) continue;
          const int q = q0 + u * nthr;
          const int c = q >> 6;
          const int mask = d.mask[c];
          bool diff = false;
#pragma unroll
          for (int i = 0; i < GW; ++i)
            if ((mask >> i) & 1) diff |= wv[u][i] != lv[u];
          if (diff) atomicMin(&d.J[c], jr + (q & 63));
        }
      }
      __syncthreads();
    }
    for (int c = tid; c < nc; c += nthr) {
      const int win = d.win[c], mask = d.mask[c], J = d.J[c];
      const bool grp = J >= 1;
      a.win_info[win] = grp ? (J << 4) | mask : 0;
      if (cached) L.winfo[win] = grp ? (J << 4) | mask : 0;
#pragma unroll
      for (int i = 0; i < GW; ++i) {
        const int s = win * GW + i;
        if (s < a.num_seqs) {
          a.tok_start[s] = grp && ((mask >> i) & 1) ? J * BS : 0;
          if (cached) L.start[s] = grp && ((mask >> i) & 1) ? J * BS : 0;
        }
      }
    }
    __syncthreads();
  }
}

// The plan: list every unit that holds tokens (a sequence's own partitions
// and, when sharing was looked for, the groups' partitions), largest first,
// and reset the work counter.  A sequence with context_len <= 0 gets one entry
// (partition 0, in the smallest bucket) so that its output is written as NaN.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const DecodeArgs a) {
  __shared__ int cnt[PLAN_BUCKETS];
  __shared__ DetectLds det;
  __shared__ PlanSeqLds seq;
  const int BS = a.block_size;
  const int part_tokens = a.part_blocks * BS;
  const int P = a.num_parts;
  for (int i = threadIdx.x; i < PLAN_BUCKETS; i += blockDim.x) cnt[i] = 0;
  const bool cached = a.num_seqs <= PLAN_SEQ_CAP;
  if (cached) {
    for (int s = threadIdx.x; s < a.num_seqs; s += blockDim.x) {
      seq.ctx[s] = clamp_ctx(a, s);
      seq.first[s] = a.win_info != nullptr ? a.block_tables[(int64_t)s * a.max_blocks_per_seq] : 0;
      seq.start[s] = 0;
    }
    __syncthreads();
  }
  if (a.win_info != nullptr) detect_all(a, det, seq, cached);  // ends with a barrier
  __syncthreads();
  auto ctx_of = [&](int s) { return cached ? seq.ctx[s] : clamp_ctx(a, s); };
  auto start_of = [&](int s) { return cached ? seq.start[s] : seq_start(a, s); };
  // Pair i < npairs is (sequence i / P, partition i % P); pair npairs + j is
  // (window j / P, partition j % P) of the shared blocks.  Each gets a bucket
  // (-1: no entry) and its work-list entry.  A sequence's partition is tagged
  // for cached loads when a neighbouring sequence holds the same physical block
  // at its first logical position; the neighbours' table entries are read
  // unconditionally (they are in bounds) and used only where the neighbour's
  // context reaches them.
  const int npairs = a.num_seqs * P;
  const int ngroup = a.win_info != nullptr ? a.num_windows * P : 0;
  const int ntotal = npairs + ngroup;
  auto classify = [&](int i, int& bucket, int& entry) __attribute__((always_inline)) {
    bucket = -1;
    entry = 0;
    if (i >= ntotal) return;
    if (i >= npairs) {
      const int j = i - npairs;
      const int win = j / P;
      const int p = j - win * P;
      const int info = cached ? seq.winfo[win] : a.win_info[win];
      if (info == 0) return;
      const int J = info >> 4;
      const int tok0 = p * part_tokens;
      const int tend = min(tok0 + part_tokens, J * BS);
      if (tok0 >= tend) return;
      int nb = (tend - tok0) / BS;
      if (P == 1) {  // unsplit: the group unit also streams each member's own blocks
#pragma unroll
        for (int g = 0; g < SHARE_WINDOW; ++g)
          if ((info >> g) & 1) nb += (ctx_of(win * SHARE_WINDOW + g) + BS - 1) / BS - J;
      }
      bucket = min(nb, PLAN_BUCKETS - 1);
      entry = (j << ENTRY_SHIFT) | ENTRY_GROUP;
      return;
    }
    const int s = i / P;
    const int p = i - s * P;
    const int ctx = ctx_of(s);
    const int ctx_l = s > 0 ? ctx_of(s - 1) : 0;
    const int ctx_r = s + 1 < a.num_seqs ? ctx_of(s + 1) : 0;
    const int t0 = start_of(s) + p * part_tokens;
    if (ctx <= 0) {
      // One entry, in the smallest bucket, so that the output is written as NaN.
      if (p == 0) {
        bucket = 0;
        entry = (s * P) << ENTRY_SHIFT;
      }
      return;
    }
    if (t0 >= ctx) return;
    if (P == 1 && t0 > 0) return;  // a group member's own blocks: its group unit streams them
    const int nb = (min(part_tokens, ctx - t0) + BS - 1) / BS;
    const int lb = t0 / BS;
    const int32_t* row = a.block_tables + (int64_t)s * a.max_blocks_per_seq + lb;
    const int mine = row[0];
    const int left = s > 0 ? row[-a.max_blocks_per_seq] : 0;
    const int right = s + 1 < a.num_seqs ? row[a.max_blocks_per_seq] : 0;
    const int shared = (ctx_l > lb * BS && left == mine) || (ctx_r > lb * BS && right == mine);
    bucket = min(nb, PLAN_BUCKETS - 1);
    entry = ((s * P + p) << ENTRY_SHIFT) | (shared ? ENTRY_REUSE : 0);
  };
  // Up to R pairs per thread are classified at once (their loads overlap) and
  // kept in registers for the placement pass; larger batches classify again.
  constexpr int R = 4;
  const int per_pass = R * (int)blockDim.x;
  int bucket[R], entry[R];
  for (int base = 0; base < ntotal; base += per_pass) {
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
  if (ntotal <= per_pass) {
    place();  // the single batch is still in registers
  } else {
    for (int base = 0; base < ntotal; base += per_pass) {
#pragma unroll
      for (int k = 0; k < R; ++k) classify(base + threadIdx.x + k * (int)blockDim.x, bucket[k], entry[k]);
      place();
    }
  }
}

// Stream the (block, head) tiles of table entries trow[0 .. nblk-1] through
// consume(k tile, v tile, entry index, bad id): lane l's 16-byte pieces of
// tile rows, two tiles in flight per wave (ping-pong register sets) while a
// tile takes at most four loads.  An id outside the pool is never read; its
// tile is consumed with `bad` set.
template <typename G, bool NT, typename F>
__device__ __forceinline__ void stream_tiles(const DecodeArgs& a, const int32_t* trow, int nblk, const char* kbase,
                                             const char* vbase, int64_t bstride, F&& consume) {
  constexpr int NI = G::NI;
  const int lane = threadIdx.x & 63;
  auto load = [&](int phys, uint4 (&kx)[NI], uint4 (&vx)[NI]) {
    const char* kp = kbase + (int64_t)phys * bstride;
    const char* vp = vbase + (int64_t)phys * bstride;
#pragma unroll
    for (int i = 0; i < NI; ++i) kx[i] = load_kv16<NT>(kp + i * 1024);
#pragma unroll
    for (int i = 0; i < NI; ++i) vx[i] = load_kv16<NT>(vp + i * 1024);
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
}

// One lane row's online-softmax step over a tile of BS token rows: scores
// q.k (log2 units), masked by selection at or past ctx (tb = the tile's first
// position), NaN for a bad id; then the running max, sum and accumulators.
template <typename E, int D, int BS>
__device__ __forceinline__ void softmax_tile(const DecodeArgs& a, const uint4& qv, const uint4 (&kx)[DecodeGeom<E, D, BS>::NI],
                                             uint4 (&vx)[DecodeGeom<E, D, BS>::NI], int tb, int ctx, bool bad,
                                             float& m, float& l, float (&acc)[DecodeGeom<E, D, BS>::VEC]) {
  using G = DecodeGeom<E, D, BS>;
  using C = Chunk<E>;
  constexpr int VEC = G::VEC, LPT = G::LPT, TPI = G::TPI, NI = G::NI;
  const int r = (threadIdx.x & 63) / LPT;
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
}

// Merge the wave's TPI token rows (lanes c, c + LPT, ... hold the same dims):
// common maximum, rescaled sums, in a fixed butterfly order.  Every lane ends
// with the row-merged M, Ls and acc of its dims.
template <int LPT, int VEC>
__device__ __forceinline__ void merge_rows(float m, float l, const float (&acc)[VEC], float& M, float& Ls,
                                           float (&av)[VEC]) {
  M = m;
#pragma unroll
  for (int sft = LPT; sft < 64; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft, 64));
  const float f = fast_exp2(m - M);
  Ls = l * f;
#pragma unroll
  for (int e2 = 0; e2 < VEC; ++e2) av[e2] = acc[e2] * f;
#pragma unroll
  for (int sft = LPT; sft < 64; sft <<= 1) {
    Ls += __shfl_xor(Ls, sft, 64);
#pragma unroll
    for (int e2 = 0; e2 < VEC; ++e2) av[e2] += __shfl_xor(av[e2], sft, 64);
  }
}

// One (sequence, partition) unit of the decode for head h: work-list entry
// `tagged`.  Called by one wave; lanes as described above.  The partial result
// goes to slot shared_parts + p of the sequence's slots.
template <typename E, typename O, int D, int BS>
__device__ __forceinline__ void private_unit(const DecodeArgs& a, int tagged, int h) {
  using G = DecodeGeom<E, D, BS>;
  constexpr int VEC = G::VEC, LPT = G::LPT, NI = G::NI;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;
  const int c = lane % LPT;
  const int H = a.num_heads;
  const int part_tokens = a.part_blocks * BS;
  const int64_t bstride = (int64_t)H * G::TILE;
  const bool reuse = tagged & ENTRY_REUSE;  // blocks shared with a neighbouring sequence
  const int entry = tagged >> ENTRY_SHIFT;
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
    softmax_tile<E, D, BS>(a, qv, kx, vx, tok0 + jb * BS, ctx, bad, m, l, acc);
  };
  // The stream is instantiated once per load kind, so that the choice is made
  // once per unit and the loop bodies stay straight-line.
  if (reuse) stream_tiles<G, false>(a, trow, nblk, kbase, vbase, bstride, consume);
  else stream_tiles<G, true>(a, trow, nblk, kbase, vbase, bstride, consume);

  float M, Ls, av[VEC];
  merge_rows<LPT, VEC>(m, l, acc, M, Ls, av);
  if (r == 0) {
    if (direct) {
#pragma unroll
      for (int e2 = 0; e2 < VEC; ++e2) Out<O>::put(a.out, sh * D + c * VEC + e2, av[e2] / Ls);
    } else {
      const int64_t pi = sh * a.num_slots + shared_parts(a, s, part_tokens) + p;
      float* dst = a.ws_acc + pi * D + c * VEC;
#pragma unroll
      for (int e2 = 0; e2 < VEC; e2 += 4)
        *reinterpret_cast<float4*>(dst + e2) = make_float4(av[e2], av[e2 + 1], av[e2 + 2], av[e2 + 3]);
      if (c == 0) *reinterpret_cast<float2*>(a.ws_ml + pi * 2) = make_float2(M, Ls);
    }
  }
}

// One group unit: entry (window, partition p of the shared blocks), head h.
// The wave streams head h of the group's shared blocks once and keeps one
// online softmax per member (its own query), with the same lane layout as a
// sequence's own unit.  Every shared block is full and inside every member's
// context, so no slot is masked.  When contexts are not split (P = 1) the unit
// then streams each member's own remaining blocks with that member's query
// and writes the members' outputs; otherwise each member's partial result goes
// to its slot p and its own partitions are units of their own.
template <typename E, typename O, int D, int BS>
__device__ __forceinline__ void group_unit(const DecodeArgs& a, int tagged, int h) {
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
  const int e = tagged >> ENTRY_SHIFT;
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
  const bool tails = a.num_parts == 1;

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
  // interleave the members' dependency chains.  Elsewhere absent members are
  // skipped, which keeps the register count, and so the occupancy, where it
  // was.
  constexpr bool ALL_MEMBERS = NI <= 4 && LPT == 16;
  auto consume = [&](const uint4 (&kx)[NI], const uint4 (&vx)[NI], int, bool bad) {
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
  stream_tiles<G, true>(a, trow, nblk, kbase, vbase, bstride, consume);

  // Per member: its own remaining blocks (unsplit contexts), then the merge
  // of the wave's token rows and the store.
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    if (!((mask >> g) & 1)) continue;
    const int s = s0 + g;
    const int64_t sh = (int64_t)s * H + h;
    if (tails) {
      const int ctx = clamp_ctx(a, s);
      const int own = (ctx + BS - 1) / BS - J;  // blocks past the shared ones
      const int32_t* orow = a.block_tables + (int64_t)s * a.max_blocks_per_seq + J;
      auto consume1 = [&](const uint4 (&kx)[NI], uint4 (&vx)[NI], int jb, bool bad) {
        softmax_tile<E, D, BS>(a, qv[g], kx, vx, (J + jb) * BS, ctx, bad, m[g], l[g], acc[g]);
      };
      if (own > 0) stream_tiles<G, true>(a, orow, own, kbase, vbase, bstride, consume1);
    }
    float M, Ls, av[VEC];
    merge_rows<LPT, VEC>(m[g], l[g], acc[g], M, Ls, av);
    if (r == 0) {
      if (tails) {
#pragma unroll
        for (int e2 = 0; e2 < VEC; ++e2) Out<O>::put(a.out, sh * D + c * VEC + e2, av[e2] / Ls);
      } else {
        const int64_t pi = sh * a.num_slots + p;
        float* dst = a.ws_acc + pi * D + c * VEC;
#pragma unroll
        for (int e2 = 0; e2 < VEC; e2 += 4)
          *reinterpret_cast<float4*>(dst + e2) = make_float4(av[e2], av[e2 + 1], av[e2 + 2], av[e2 + 3]);
        if (c == 0) *reinterpret_cast<float2*>(a.ws_ml + pi * 2) = make_float2(M, Ls);
      }
    }
  }
}

// The merge of one (sequence, head): out = sum_k 2^(m_k - M) acc_k /
// sum_k 2^(m_k - M) l_k over its slots k ascending (its group's partitions,
// then its own), M = max_k m_k; thread t takes dim t.  A sequence whose one
// unit wrote the output directly is skipped.
template <typename O, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const DecodeArgs a) {
  const int s = blockIdx.x;
  const int h = blockIdx.y;
  const int ctx = clamp_ctx(a, s);
  const int part_tokens = a.part_blocks * a.block_size;
  const int st0 = seq_start(a, s);
  if (ctx <= 0 || (st0 == 0 && ctx <= part_tokens)) return;
  const int nsl = shared_parts(a, s, part_tokens) + (ctx > st0 ? (ctx - st0 + part_tokens - 1) / part_tokens : 0);
  const int t = threadIdx.x;
  const int64_t sh = (int64_t)s * a.num_heads + h;
  const int64_t base = sh * a.num_slots;
  // Up to RP slots: every (m, l) and partial value is loaded at once, so the
  // merge waits for memory once.  The arithmetic and its order are the same
  // either way.
  constexpr int RP = 8;
  if (nsl <= RP) {
    float mp[RP], lp[RP], ap[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      if (k < nsl) {
        const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (base + k) * 2);
        mp[k] = ml.x;
        lp[k] = ml.y;
        ap[k] = a.ws_acc[(base + k) * D + t];
      }
    }
    float M = NEG_BIG;
#pragma unroll
    for (int k = 0; k < RP; ++k)
      if (k < nsl) M = fmaxf(M, mp[k]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      if (k < nsl) {
        const float f = fast_exp2(mp[k] - M);
        Ls = fmaf(lp[k], f, Ls);
        A = fmaf(ap[k], f, A);
      }
    }
    Out<O>::put(a.out, sh * D + t, A / Ls);
    return;
  }
  float M = NEG_BIG;
  for (int k = 0; k < nsl; ++k) M = fmaxf(M, a.ws_ml[(base + k) * 2]);
  float Ls = 0.f, A = 0.f;
  for (int k = 0; k < nsl; ++k) {
    const float f = fast_exp2(a.ws_ml[(base + k) * 2] - M);
    Ls = fmaf(a.ws_ml[(base + k) * 2 + 1], f, Ls);
    A = fmaf(a.ws_acc[(base + k) * D + t], f, A);
  }
  Out<O>::put(a.out, sh * D + t, A / Ls);
}

// Persistent decode kernel: claims units (work-list entry, head group) from
// the counter until none are left.
template <typename E, typename O, int D, int BS>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const DecodeArgs a) {
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
    if (h >= H) continue;  // a partial last head group
    const int tagged = __builtin_amdgcn_readfirstlane(a.work_list[e]);
    if (tagged & ENTRY_GROUP) group_unit<E, O, D, BS>(a, tagged, h);
    else private_unit<E, O, D, BS>(a, tagged, h);
  }
}

// Read probe: the decode's tile reads without its arithmetic.  The same plan,
// units, scheduling and loads as the two-stage decode; each wave folds every
// 32-bit word of the K and V tiles it reads (whole tiles, the slots past the
// context included) with XOR, and out[s][h] receives the fold over the
// sequence's blocks 0 .. ceil(ctx / BS) - 1 (XOR of the units' folds).  It
// measures how fast this access pattern streams from HBM.
template <typename E, int D, int BS>
__global__ __launch_bounds__(NW * 64) void read_probe_kernel(const DecodeArgs a, uint32_t* out) {
  using G = DecodeGeom<E, D, BS>;
  constexpr int NI = G::NI;
  __shared__ int sm_unit[2];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int H = a.num_heads;
  const int HG = (H + NW - 1) / NW;
  const int64_t bstride = (int64_t)H * G::TILE;
  const int part_tokens = a.part_blocks * BS;
  const int total = a.work_ctrl[1] * HG;
  for (int it = 0;; ++it) {
    if (threadIdx.x == 0) sm_unit[it & 1] = atomicAdd(&a.work_ctrl[0], 1);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(sm_unit[it & 1]);
    if (u >= total) break;
    const int e = u / HG;
    const int h = (u - e * HG) * NW + w;
    if (h >= H) continue;
    const int entry = __builtin_amdgcn_readfirstlane(a.work_list[e]) >> ENTRY_SHIFT;
    const int s = entry / a.num_parts;
    const int p = entry - s * a.num_parts;
    const int ctx = clamp_ctx(a, s);
    const int tok0 = p * part_tokens;
    if (ctx <= 0 || tok0 >= ctx) continue;
    const int nblk = (min(part_tokens, ctx - tok0) + BS - 1) / BS;
    const char* kbase = reinterpret_cast<const char*>(a.k_cache) + (int64_t)h * G::TILE + lane * 16;
    const char* vbase = reinterpret_cast<const char*>(a.v_cache) + (int64_t)h * G::TILE + lane * 16;
    const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq + tok0 / BS;
    uint32_t x = 0;
    auto consume = [&](const uint4 (&kx)[NI], const uint4 (&vx)[NI], int, bool) {
#pragma unroll
      for (int i = 0; i < NI; ++i) x ^= kx[i].x ^ kx[i].y ^ kx[i].z ^ kx[i].w ^ vx[i].x ^ vx[i].y ^ vx[i].z ^ vx[i].w;
    };
    stream_tiles<G, true>(a, trow, nblk, kbase, vbase, bstride, consume);
#pragma unroll
    for (int sft = 1; sft < 64; sft <<= 1) x ^= (uint32_t)__shfl_xor((int)x, sft, 64);
    if (lane == 0) atomicXor(out + (int64_t)s * H + h, x);
  }
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

// Workgroups per CU of the decode: 1, or the value of the environment
// variable PKV_DECODE_WG_PER_CU (1 to 16; read at every launch, for measuring
// other launch shapes).
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
  const int64_t units = (int64_t)a.max_entries * ((a.num_heads + NW - 1) / NW);
  const int grid = persistent_grid<decode_kernel<E, O, D, BS>>(NW * 64, units, decode_wg_per_cu());
  hipLaunchKernelGGL((decode_kernel<E, O, D, BS>), dim3(grid), dim3(NW * 64), 0, st, a);
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

template <typename E, int D, int BS>
static hipError_t probe_bs(const DecodeArgs& a, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, st, a);
  const int64_t units = (int64_t)a.max_entries * ((a.num_heads + NW - 1) / NW);
  const int grid = persistent_grid<read_probe_kernel<E, D, BS>>(NW * 64, units, 1);
  hipLaunchKernelGGL((read_probe_kernel<E, D, BS>), dim3(grid), dim3(NW * 64), 0, st, a, out);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t probe_d(const DecodeArgs& a, uint32_t* out, hipStream_t st) {
  if (a.block_size == 8) return probe_bs<E, D, 8>(a, out, st);
  if (a.block_size == 32) return probe_bs<E, D, 32>(a, out, st);
  return probe_bs<E, D, 16>(a, out, st);
}

hipError_t launch_read_probe(const DecodeArgs& a, int dtype, int head_dim, uint32_t* out, hipStream_t st) {
  // Only the element size matters to the loads: fp16 and bf16 share the 16-bit geometry.
  if (head_dim == 128) return dtype == 0 ? probe_d<f32_t, 128>(a, out, st) : probe_d<f16_t, 128>(a, out, st);
  return dtype == 0 ? probe_d<f32_t, 64>(a, out, st) : probe_d<f16_t, 64>(a, out, st);
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
