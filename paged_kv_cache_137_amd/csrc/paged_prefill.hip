// Causal prefill (prompt-phase) attention on gfx950 matrix cores.
//
// All positions of a prompt are known at once, so attention is a dense
// matrix-matrix product, S = scale * Q K^T masked to key <= query, then a row
// softmax and O = P V ("vLLM & PagedAttention: Efficient Memory Management for
// LLM Serving", section I: the prompt phase, and the t <= i limit of the
// attention equation).
//
// Design for CDNA4 (the pages give no kernel for this step):
//  - Workgroup = 4 wavefronts = 128 query rows of one (prompt, head).  Each wave
//    owns 32 queries.  Key/value tiles of 32 rows are staged in LDS and shared
//    (32 KiB of LDS per workgroup at 128 dims), and three workgroups share a CU:
//    the third wave per SIMD hides more latency than the larger tiles of two
//    workgroups saved in barriers.  LDS is double-buffered: the next tile's
//    K/V go from HBM straight into
//    LDS (buffer loads that write LDS, no registers on the way) while the
//    current tile is multiplied.  Each wave waits for its own loads, then one
//    barrier per tile publishes the tile.
//  - Each half-wave keeps a lane-local partial row sum against a shared
//    reference maximum.  The halves exchange only when that reference moves
//    (rarely), and once at the end.
//  - Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 on
//    16-bit inputs and fp32 accumulation.  Each lane's 16 accumulator values
//    then belong to a single query (its column).  The online softmax (running
//    max, rescale, row sum) is lane-local plus one exchange between the two
//    half-waves.
//  - The output is accumulated transposed as well: O^T += V^T P^T, so the
//    per-query rescale stays lane-local.  P^T is fed from the score registers
//    directly.  Its key order inside an MFMA k-step follows the accumulator
//    layout.  V stays row-major in LDS; the V^T operand comes from gfx950's
//    transposing LDS reads (ds_read_b64_tr_b16) in that same key order.
//  - Probabilities are exp2(s * scale * log2 e - m): one FMA and one v_exp each.
//    They are rounded once to the input type for the MFMA.  The row sum adds
//    the rounded values (v_dot2 against ones), so the normalisation matches
//    what was accumulated.  The reference maximum m moves only when a row's
//    maximum rises by more than 8 (log2 units).  Probabilities then stay below
//    2^8, and the 64-value accumulator rescale is rare.  Workgroups whose rows
//    have fewer than 256 keys (where rounding weighs most) track the maximum
//    exactly instead, so each row's largest probability is exactly 1.
//  - Rows with few keys feel the rounding of P most: with two or three keys a
//    bf16 probability's relative error of up to 2^-9 moves the output by up to
//    about 2^-9 |v_1 - v_0| / 4.  So in a prompt's first key tile (the only
//    tile of its first 32 rows) bf16 probabilities get a second, low part,
//    bf16(P - bf16(P)), multiplied with the same V^T fragments and added to
//    the row sum; that tile costs eight more MFMAs per wave.
//  - Causality: key tiles past the workgroup's last query are never loaded.
//    Key tiles past a wave's last query are skipped by that wave, and a wave
//    whose queries all lie past the prompt end (in a prompt's last, partial
//    query tile) multiplies nothing: it only loads and waits.  Tiles that
//    straddle the diagonal or the prompt end are masked by selecting -inf.
//  - Query tiles are dispatched longest first, to even out the causal
//    triangle's load: prompts in order of context length (up to 64 prompts,
//    ranked by each workgroup), and each prompt's tiles in descending order.
//    Only tiles that exist get a workgroup.
//  - Cached-prefix variant: keys and values are gathered from the paged pool
//    through the prompt's block table, with the same LDS tiles: each 1 KiB run
//    of rows lies in one block, and each wave load gets a buffer descriptor
//    over exactly that block's rows.  Positions before the prompt's new tokens
//    are a shared prefix that is already cached ("vLLM & PagedAttention ...",
//    section VII: the prompt phase runs only over the request's own input).
//    The causal limit is then shifted by the prefix length.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Buffer resource word 3 for gfx9-family parts: raw (untyped) 32-bit dword access.
constexpr int BUF_RSRC_WORD3 = 0x00020000;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 64 lanes x 16 bytes from a buffer straight into LDS: lane l's bytes land at
// lds + 16*l (lds is wave-uniform).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voffset, 0, 0, 0);
}
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i addresses 4 16-bit
// values (row i of a 16 x 4 matrix M); lane j receives M[j/4 + 4k][j%4], k = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(lds_ptr_t)p));
}
// Wait for this wave's outstanding vector-memory operations (loads into LDS included).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename E>
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c);
template <>
__device__ __forceinline__ f32x16_t mfma32<bf16_t>(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16_t mfma32<f16_t>(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two floats rounded (nearest even) into one packed 16-bit pair.
template <typename E> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  f16x2_t v;
  v.x = (_Float16)lo;
  v.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// acc + both halves of a packed pair, as one v_dot2 against (1, 1).
template <typename E> __device__ __forceinline__ float rowsum2(uint32_t w, float acc);
template <>
__device__ __forceinline__ float rowsum2<bf16_t>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}
template <>
__device__ __forceinline__ float rowsum2<f16_t>(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc, false);
}

// Store four outputs x * inv.  The product is rounded to float32 first (no
// contraction), and a 16-bit output is that float rounded to nearest even.
template <typename O> struct Store4;
template <> struct Store4<f32_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d, float inv) {
#pragma clang fp contract(off)
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = make_float4(a * inv, b * inv, c * inv, d * inv);
  }
};
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d, float inv) {
#pragma clang fp contract(off)
    float ra = a * inv, rb = b * inv, rc = c * inv, rd = d * inv;
    asm volatile("" : "+v"(ra), "+v"(rb), "+v"(rc), "+v"(rd));
    // v_cvt_pk_bf16_f32: round to nearest even
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = make_uint2(pack2<bf16_t>(ra, rb), pack2<bf16_t>(rc, rd));
  }
};
template <> struct Store4<f16_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d, float inv) {
#pragma clang fp contract(off)
    const float ra = a * inv, rb = b * inv, rc = c * inv, rd = d * inv;
    const uint32_t x = (uint32_t)f32_to_f16_bits(ra) | ((uint32_t)f32_to_f16_bits(rb) << 16);
    const uint32_t y = (uint32_t)f32_to_f16_bits(rc) | ((uint32_t)f32_to_f16_bits(rd) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = make_uint2(x, y);
  }
};

// PB = 0:        keys/values are the prompt's own packed rows (a fresh prompt).
// PB = 8, 16, 32: keys/values are read from the pool (blocks of PB tokens)
//                 through the prompt's block table.  The first prefix_lens[p]
//                 positions are a cached prefix; the prompt's new tokens follow
//                 (their K/V already written).
template <typename E, typename O, int D, int PB>
__global__ __launch_bounds__(256, 3) void prefill_kernel(const PrefillArgs a) {
  constexpr bool PAGED = PB != 0;
  constexpr int SH = PB == 8 ? 3 : PB == 16 ? 4 : PB == 32 ? 5 : 0;  // log2 of the block size
  static_assert(!PAGED || (1 << SH) == PB, "block size 8, 16 or 32");
  constexpr int BM = PREFILL_BLOCK_M;  // query rows per workgroup (4 waves x 32)
  constexpr int BN = 32;               // keys per LDS tile
  constexpr int U = BN / 32;           // 32-key sub-tiles per tile
  constexpr int KS = D / 16;           // k-steps of Q K^T
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int ROWB = D * 2;          // bytes of one K or V row
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;     // rows per 1 KiB wave load into LDS
  constexpr int IPW = BN / RPI / 4;    // such loads per wave, per tensor and tile
  constexpr int TILE = BN * ROWB;      // bytes of one K or V tile
  constexpr float RESCALE_SLACK = 8.0f;  // log2 units a row maximum may rise before rescaling
  static_assert(IPW * RPI * 4 == BN, "a tile must map onto 4 waves of 1 KiB loads");
  static_assert(!PAGED || RPI <= PB, "a 1 KiB run of rows must lie in one block");
  // Two LDS buffers per tensor: tile n is read from one while tile n+1 is
  // loaded into the other.  Tiles are row-major [key][dim], dense, filled by
  // buffer loads that write LDS directly.  The 16-byte chunks of each row are
  // XOR-swizzled by the row index, so that the fragment reads below touch
  // every bank evenly.  Separate objects, so the compiler can tell a pending
  // load into one buffer from the reads of the other.
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[TILE], k_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[TILE], v_lds1[TILE];
  auto kbuf = [&](int b) -> unsigned char* { return b ? k_lds1 : k_lds0; };
  auto vbuf = [&](int b) -> unsigned char* { return b ? v_lds1 : v_lds0; };
  // Swizzled chunk of a row: K's fragment reads take one 16-byte chunk from
  // each of 16 consecutive rows; V's transposing reads take 8 bytes from each
  // of 8 consecutive rows, in runs of 4 chunks.  Each is an involution.
  auto kswz = [](int row, int ch) { return D == 128 ? ch ^ (row & 15) : ch ^ ((row >> 1) & 7); };
  auto vswz = [](int row, int ch) { return D == 128 ? ch ^ (4 * (row & 3)) : ch ^ (4 * ((row >> 1) & 1)); };

  // Work items.  Consecutive workgroups go to the 8 XCDs in turn, so the grid
  // is 8 slices, one per XCD, of heads_per_xcd * items_per_head items each.
  // Slice x holds heads x, x + 8, x + 16, ...  Within a slice the items run
  // prompt after prompt, and for each prompt every head's query tiles, longest
  // first.  The prompts' order:
  //  - up to PREFILL_DENSE_PROMPTS prompts: by context length (prefix + new
  //    tokens), longest first, ties by index; each workgroup ranks the prompts
  //    itself, one per lane.  The longest causal rows of every head start
  //    first and the short ones fill the end.
  //  - more prompts: index order, found by a prefix scan over the prompts in
  //    chunks of 64.
  // Only query tiles that exist get an item (a few items past the last tile
  // return at once).  The heads of one prompt run side by side on one XCD,
  // whose L2 holds the K/V that their query tiles reread.
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int k = wg >> 3;  // position in the slice
  const int HX = a.heads_per_xcd;
  if (k >= HX * a.items_per_head) return;
  const int lane = threadIdx.x & 63;
  const int np = a.num_prompts;
  int pr = -1, nq_p = 0, start_p = 0, L = 0;
  long long off = 0;  // row offset of the prompt: the sum of the earlier prompts' lengths
  if (np <= PREFILL_DENSE_PROMPTS) {
    const int lj = lane < np ? max(a.prompt_lens[lane], 0) : 0;
    int key = lj;
    if constexpr (PAGED) {
      if (a.prefix_lens != nullptr && lane < np) key += max(a.prefix_lens[lane], 0);
    }
    const int nq = (int)(((int64_t)lj + BM - 1) / BM);  // this lane's prompt's query tiles
    // start: tiles of the prompts ahead of this lane's in the order.
    int start = 0;
    for (int i = 0; i < np; ++i) {
      const int ki = __builtin_amdgcn_readlane(key, i);
      const int ni = __builtin_amdgcn_readlane(nq, i);
      start += (ki > key || (ki == key && i < lane)) ? ni : 0;
    }
    const unsigned long long hit = __ballot(lane < np && k >= HX * start && k < HX * (start + nq));
    if (hit == 0ull) return;  // past the last tile of the slice
    pr = (int)__builtin_ctzll(hit);
    L = __builtin_amdgcn_readlane(lj, pr);
    nq_p = __builtin_amdgcn_readlane(nq, pr);
    start_p = __builtin_amdgcn_readlane(start, pr);
    off = lane < pr ? lj : 0;
  } else {
    int base = 0;  // tiles of the earlier chunks
    for (int c0 = 0; c0 < np; c0 += 64) {
      const int i = c0 + lane;
      const int lj = i < np ? max(a.prompt_lens[i], 0) : 0;
      const int nq = (int)(((int64_t)lj + BM - 1) / BM);
      int incl = nq;  // inclusive prefix sum of the chunk's tile counts
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      const int excl = base + incl - nq;
      if (k < HX * (base + tot)) {
        const unsigned long long hit = __ballot(i < np && k >= HX * excl && k < HX * (excl + nq));
        const int pl = (int)__builtin_ctzll(hit);  // nonempty: k lies in this chunk
        pr = c0 + pl;
        L = __builtin_amdgcn_readlane(lj, pl);
        nq_p = __builtin_amdgcn_readlane(nq, pl);
        start_p = __builtin_amdgcn_readlane(excl, pl);
        off += lane < pl ? lj : 0;
        break;
      }
      base += tot;
      off += lj;
    }
    if (pr < 0) return;  // past the last tile of the slice
  }
  const int rem = k - HX * start_p;
  const int hl = rem / nq_p;
  const int h = xcd + 8 * hl;
  if (h >= a.num_heads) return;
  const int qt = nq_p - 1 - (rem - hl * nq_p);
  const int m0 = qt * BM;
  L = __builtin_amdgcn_readfirstlane(L);  // one value for the workgroup (keeps descriptors scalar)
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) off += __shfl_xor(off, sft, 64);
  // Every lane holds the same sum; make that visible to the compiler, so that
  // the buffer descriptors built from it live in scalar registers.
  off = (long long)(((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(off >> 32)) << 32) |
                    (uint32_t)__builtin_amdgcn_readfirstlane((int)off));
  if (off + L > a.total_tokens) L = (int)max(0ll, (long long)a.total_tokens - off);
  // C: cached prefix tokens ahead of the new ones; keys are indexed by absolute
  // position 0 .. C+L-1, and new token i sits at position C + i.
  int C = 0;
  const int32_t* trow = nullptr;
  if constexpr (PAGED) {
    const int cap = a.max_blocks_per_seq << SH;
    C = a.prefix_lens != nullptr ? min(max(a.prefix_lens[pr], 0), cap) : 0;
    // One value for the whole workgroup: say so, so that the buffer
    // descriptors built from it stay scalar.
    C = __builtin_amdgcn_readfirstlane(C);
    L = __builtin_amdgcn_readfirstlane(min(L, cap - C));
    trow = a.block_tables + (int64_t)pr * a.max_blocks_per_seq;
  }
  if (L <= m0) return;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31;
  const int hf = lane >> 5;
  const int qrow0 = m0 + w * 32;  // first query of this wave
  const int qi = qrow0 + ql;      // this lane's query
  const int64_t rs = (int64_t)a.num_heads * D;  // elements between consecutive tokens
  const uint32_t rsb = (uint32_t)(rs * 2);       // the same, in bytes
  const char* qb = reinterpret_cast<const char*>(a.q) + (off * rs + (int64_t)h * D) * 2;
  const char* kb = reinterpret_cast<const char*>(a.k) + (off * rs + (int64_t)h * D) * 2;
  const char* vb = reinterpret_cast<const char*>(a.v) + (off * rs + (int64_t)h * D) * 2;
  const float c = a.scale_log2;  // > 0

  // Q as the B operand of S^T = K Q^T: k-step kk holds dims kk*16 + hf*8 .. +8.
  uint4 qf[KS];
  if (qi < L) {
    const char* qp = qb + (int64_t)qi * rsb + hf * 16;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = *reinterpret_cast<const uint4*>(qp + kk * 32);
  } else {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Paged form: the block ids of the next tile to be loaded, one tile ahead
  // (lane j of each wave holds the id of the tile's block j), and the first
  // key that lies in a block outside the pool.  Such a block is never read;
  // every query that would see it gets NaN.
  constexpr int NBT = PAGED ? BN / PB : 1;
  int idv = 0;
  int bad_key = 0x7fffffff;
  auto load_ids = [&](int n0) {
    if constexpr (PAGED) {
      const int e = (n0 >> SH) + lane;
      const int last = (C + L - 1) >> SH;  // the table entry of the last key
      idv = lane < NBT && e <= last ? trow[e] : 0;
    }
  };
  load_ids(0);

  // The tile at key n0 straight from HBM into LDS buffer b.  Each wave load
  // fills one 1 KiB run of RPI rows: lane l's 16 bytes land at byte 16*l of
  // the run, so it loads the logical chunk that the swizzle puts there.  The
  // buffer descriptor covers exactly the rows that exist: rows past the end
  // (and every row of a block outside the pool) read as zeros.
  auto gdma = [&](int n0, int b) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const unsigned long long badm = __ballot(lane < NBT && (uint64_t)(uint32_t)idv >= (uint64_t)a.num_blocks);
      if (badm != 0ull) bad_key = min(bad_key, n0 + ((int)__builtin_ctzll(badm) << SH));
      const char* kpool = reinterpret_cast<const char*>(a.k_cache);
      const char* vpool = reinterpret_cast<const char*>(a.v_cache);
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int blk = w * IPW + j;
        const int row0 = blk * RPI;  // first row of the run, within the tile
        const int key0 = n0 + row0;
        const int ph = __builtin_amdgcn_readlane(idv, row0 >> SH);
        const bool ok = (uint64_t)(uint32_t)ph < (uint64_t)a.num_blocks;
        // Uniform, but computed through a 64-bit vector compare: say so, or the
        // compiler wraps each load in a loop over distinct descriptors.
        const int valid = __builtin_amdgcn_readfirstlane(ok ? min(max(C + L - key0, 0), RPI) : 0);
        const int64_t first = ((((int64_t)(ok ? ph : 0) * a.num_heads + h) << SH) + (key0 & (PB - 1))) * ROWB;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kpool + first), (short)0, valid * ROWB, BUF_RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vpool + first), (short)0, valid * ROWB, BUF_RSRC_WORD3);
        const int r = lane / CPR, pc = lane % CPR;
        buffer_load_lds16(rk, kbuf(b) + blk * 1024, r * ROWB + kswz(row0 + r, pc) * 16);
        buffer_load_lds16(rv, vbuf(b) + blk * 1024, r * ROWB + vswz(row0 + r, pc) * 16);
      }
      load_ids(n0 + BN);
    } else {
      // Offsets stay below 64 * rsb <= 64 * 65535 * 128 * 2 < 2^31 under the
      // ABI's limits.
      const int rows = min(L - n0, BN);  // >= 1: n0 < L here
      const int nrec = (rows - 1) * (int)rsb + D * 2;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kb + (int64_t)n0 * rsb), (short)0, nrec, BUF_RSRC_WORD3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vb + (int64_t)n0 * rsb), (short)0, nrec, BUF_RSRC_WORD3);
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int blk = w * IPW + j;
        const int row = blk * RPI + lane / CPR;
        const int pc = lane % CPR;
        buffer_load_lds16(rk, kbuf(b) + blk * 1024, row * rsb + kswz(row, pc) * 16);
        buffer_load_lds16(rv, vbuf(b) + blk * 1024, row * rsb + vswz(row, pc) * 16);
      }
    }
  };
  // The loads into LDS complete asynchronously: each wave waits for its own,
  // then the barrier publishes the tile to the whole workgroup.
  auto publish = [&]() __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
  };

  // Lane part of the V^T read addresses (transposing reads below).  Lane
  // (ql, hf) points at row 4*hf + i16/4 of each 16-key step and dims
  // 32*db + (ql & 16) + 4*(i16 % 4) .. +4; the row's swizzle depends only on
  // the row modulo 4 (D = 128) or 8 (D = 64), which adding the step's key
  // offset (a multiple of 8) keeps.
  int vlane[DB];
  {
    const int i16 = ql & 15;
    const int vrow = 4 * hf + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int dim = db * 32 + (ql & 16) + 4 * (i16 & 3);
      vlane[db] = vrow * ROWB + vswz(vrow, dim >> 3) * 16 + (dim & 7) * 2;
    }
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float mrow = NEG_BIG, lrow = 0.f;
  const int lim = C + min(qi, L - 1);  // last key position this query may see

  const int kend = C + min(L, m0 + BM);     // keys any query of the workgroup sees
  const int wkend = C + min(L, qrow0 + 32); // keys any query of this wave sees
  // Workgroups whose rows have fewer than 256 keys (a prompt's first query
  // tile behind a prefix of under 128 tokens) track each row's maximum exactly,
  // so that the row's largest probability is exactly 1 and free of rounding;
  // longer rows let the maximum rise by the slack first.
  const float slack = (C + m0 < 128) ? 0.f : RESCALE_SLACK;
  const bool act = qrow0 < L;                // the wave holds at least one query

  // One tile of BN keys from LDS buffer `buf`, starting at key n0, as U
  // sub-tiles of 32 keys whose score chains are independent (with U > 1 their
  // MFMAs interleave).  Lane (ql, hf) score element j of sub-tile u is key
  // n0 + 32u + 8*(j/4) + 4*hf + j%4 against query qi.  MASKED tiles select
  // -inf for every key past the query (or past the prompt end).  Every tile
  // body is one instantiation per MASKED value, so the accumulators stay in
  // place across iterations.
  //
  // The two half-waves hold different keys of the same queries.  Each keeps a
  // lane-local partial row sum against a shared reference maximum mrow.  They
  // exchange values only when mrow must move: when some row's maximum rises by
  // more than the slack.
  auto tile = [&](auto masked_c, int buf, int n0) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    f32x16_t st[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j) st[u][j] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = u * 32 + ql;
        const unsigned char* kr = kbuf(buf) + row * ROWB + kswz(row, 2 * kk + hf) * 16;
        st[u] = mfma32<E>(*reinterpret_cast<const uint4*>(kr), qf[kk], st[u]);
      }

    if constexpr (MASKED) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int room = lim - (n0 + 32 * u + 4 * hf);  // element j is visible iff its offset <= room
#pragma unroll
        for (int j = 0; j < 16; ++j) st[u][j] = (8 * (j >> 2) + (j & 3) > room) ? -INFINITY : st[u][j];
      }
    }
    float lmax = st[0][0];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 16; ++j) lmax = fmaxf(lmax, st[u][j]);
    const float mt = lmax * c;  // this half's maximum over the tile, log2 units
    if (__any(mt > mrow + slack)) {
      const float mnew = fmaxf(mrow, fmaxf(mt, __shfl_xor(mt, 32, 64)));
      const float alpha = fast_exp2(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      mrow = mnew;
    }

    uint32_t pk[U][8];
    // The first key tile of a prompt holds the rows with the fewest keys, whose
    // outputs feel the rounding of P most; there P also gets a second, low
    // part (P - bf16(P), rounded) and a second P V product below.
    const bool split = std::is_same_v<E, bf16_t> && MASKED && n0 == 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float p0 = fast_exp2(fmaf(st[u][2 * jj], c, -mrow)), p1 = fast_exp2(fmaf(st[u][2 * jj + 1], c, -mrow));
        pk[u][jj] = pack2<E>(p0, p1);
        lrow = rowsum2<E>(pk[u][jj], lrow);
        st[u][2 * jj] = p0;
        st[u][2 * jj + 1] = p1;
      }

    // O^T += V^T P^T in k-steps of 16 keys.  In step (u, kk2), element i of lane
    // (ql, hf) stands for key n0 + 32u + 16*kk2 + 8*(i/4) + 4*hf + i%4 on both
    // operands.  V^T comes from transposing reads: in each group of 16 lanes,
    // lane i points at 4 values of row kb0 + i/4, dims d0 + 4*(i%4); lane j
    // then receives dim d0 + j of rows kb0 .. kb0+3.  The lane part of each
    // address is vlane[db]; the step's key offset is a constant.
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const uint4 pb = make_uint4(pk[u][4 * kk2], pk[u][4 * kk2 + 1], pk[u][4 * kk2 + 2], pk[u][4 * kk2 + 3]);
        const int kofs = (u * 32 + 16 * kk2) * ROWB;  // first key of the step, within the LDS tile
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint2 lo = lds_read_tr16(vbuf(buf) + vlane[db] + kofs);
          const uint2 hi = lds_read_tr16(vbuf(buf) + vlane[db] + kofs + 8 * ROWB);
          o[db] = mfma32<E>(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[db]);
        }
      }
    if (split) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float h0 = __uint_as_float(pk[u][jj] << 16), h1 = __uint_as_float(pk[u][jj] & 0xffff0000u);
          // Parts below 2^-12 of the high part are dropped: the largest
          // probability's own rounding residue (from the FMA against the
          // row maximum) then adds nothing, and a one-key row stays exactly v_0.
          const float d0 = st[u][2 * jj] - h0, d1 = st[u][2 * jj + 1] - h1;
          pk[u][jj] = pack2<E>(fabsf(d0) >= h0 * 0x1p-12f ? d0 : 0.f, fabsf(d1) >= h1 * 0x1p-12f ? d1 : 0.f);
          lrow = rowsum2<E>(pk[u][jj], lrow);
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const uint4 pb = make_uint4(pk[u][4 * kk2], pk[u][4 * kk2 + 1], pk[u][4 * kk2 + 2], pk[u][4 * kk2 + 3]);
          const int kofs = (u * 32 + 16 * kk2) * ROWB;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint2 lo = lds_read_tr16(vbuf(buf) + vlane[db] + kofs);
            const uint2 hi = lds_read_tr16(vbuf(buf) + vlane[db] + kofs + 8 * ROWB);
            o[db] = mfma32<E>(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[db]);
          }
        }
    }
  };

  // Tiles below nfull hold keys that every query of the workgroup sees, all
  // before the prompt end (C + m0 < C + L): no masking.  The remaining tiles
  // (at most BM / BN + 1) straddle a diagonal or the prompt end; a wave skips a
  // tile that lies wholly in its queries' future.  Tile t+1 is loaded while
  // tile t is multiplied; one barrier per tile.
  const int ntiles = (kend + BN - 1) / BN;
  const int nfull = min((C + m0) / BN, ntiles);
  gdma(0, 0);
  publish();
  // Steps are unrolled in pairs, so that every LDS address names its buffer
  // at compile time (the compiler then sees that a load into one buffer and
  // the reads of the other do not overlap).
  auto step = [&](auto masked_c, auto buf_c, int tt) __attribute__((always_inline)) {
    constexpr int b = decltype(buf_c)::value;
    if (tt + 1 < ntiles) gdma((tt + 1) * BN, b ^ 1);
    if (act && (!decltype(masked_c)::value || tt * BN < wkend)) tile(masked_c, b, tt * BN);
    publish();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  int tt = 0;
  for (; tt + 1 < nfull; tt += 2) {
    step(std::false_type(), B0(), tt);
    step(std::false_type(), B1(), tt + 1);
  }
  for (; tt < ntiles; tt += 2) {
    step(std::true_type(), B0(), tt);
    if (tt + 1 < ntiles) step(std::true_type(), B1(), tt + 1);
  }
  lrow += __shfl_xor(lrow, 32, 64);  // the two halves' partial row sums

  if (qi < L) {
    const float inv = (PAGED && lim >= bad_key) ? __builtin_nanf("") : 1.0f / lrow;
    const int64_t ob = (off + qi) * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * hf;
        Store4<O>::put(a.out, ob + d0, o[db][4 * grp], o[db][4 * grp + 1], o[db][4 * grp + 2],
                       o[db][4 * grp + 3], inv);
      }
  }
}

template <typename E, typename O, int D, int PB>
static hipError_t prefill_t(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<E, O, D, PB>), dim3(a.total_items), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E, int PB>
static hipError_t prefill_d(const PrefillArgs& a, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128)
    return out_dtype == 0 ? prefill_t<E, f32_t, 128, PB>(a, st) : prefill_t<E, E, 128, PB>(a, st);
  return out_dtype == 0 ? prefill_t<E, f32_t, 64, PB>(a, st) : prefill_t<E, E, 64, PB>(a, st);
}

template <typename E>
static hipError_t prefill_e(const PrefillArgs& a, int out_dtype, int head_dim, hipStream_t st) {
  if (a.k_cache == nullptr) return prefill_d<E, 0>(a, out_dtype, head_dim, st);
  if (a.block_shift == 3) return prefill_d<E, 8>(a, out_dtype, head_dim, st);
  if (a.block_shift == 5) return prefill_d<E, 32>(a, out_dtype, head_dim, st);
  return prefill_d<E, 16>(a, out_dtype, head_dim, st);
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t st) {
  if (dtype == 1) return prefill_e<f16_t>(a, out_dtype, head_dim, st);
  return prefill_e<bf16_t>(a, out_dtype, head_dim, st);
}

}  // namespace pkv
