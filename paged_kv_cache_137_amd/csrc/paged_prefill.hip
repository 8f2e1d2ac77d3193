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
//    owns 32 queries.  Key/value tiles of 64 rows are staged in LDS and shared.
//  - Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 on
//    16-bit inputs and fp32 accumulation.  Each lane's 16 accumulator values
//    then belong to a single query (its column).  The online softmax (running
//    max, rescale, row sum) is lane-local plus one exchange between the two
//    half-waves.
//  - The output is accumulated transposed as well: O^T += V^T P^T, so the
//    per-query rescale stays lane-local.  P^T is fed from the score registers
//    directly.  Its key order inside an MFMA k-step follows the accumulator
//    layout.  V^T is read from LDS in that same key order.  V is written into
//    LDS transposed ([dim][key]) when it is staged.
//  - Probabilities are rounded once to the input type for the MFMA.  The row
//    sum adds the rounded values, so the normalisation matches what was
//    accumulated.
//  - Causality: key tiles past the workgroup's last query are never loaded.
//    Key tiles past a wave's last query are skipped by that wave.  Tiles that
//    straddle the diagonal or the prompt end are masked by selecting -inf.
//  - Query tiles are dispatched longest-first (descending tile index), to even
//    out the causal triangle's load.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

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
template <typename E> __device__ __forceinline__ float sum2(uint32_t w);
template <> __device__ __forceinline__ float sum2<bf16_t>(uint32_t w) { return bf16_lo(w) + bf16_hi(w); }
template <> __device__ __forceinline__ float sum2<f16_t>(uint32_t w) { return f16_lo(w) + f16_hi(w); }

template <typename O> struct Store4;
template <> struct Store4<f32_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = make_float4(a, b, c, d);
  }
};
template <> struct Store4<bf16_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d) {
    const uint32_t x = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    const uint32_t y = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = make_uint2(x, y);
  }
};
template <> struct Store4<f16_t> {
  __device__ __forceinline__ static void put(void* base, int64_t i, float a, float b, float c, float d) {
    const uint32_t x = (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
    const uint32_t y = (uint32_t)f32_to_f16_bits(c) | ((uint32_t)f32_to_f16_bits(d) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + i) = make_uint2(x, y);
  }
};

template <typename E, typename O, int D>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillArgs a) {
  constexpr int BM = PREFILL_BLOCK_M;  // query rows per workgroup (4 waves x 32)
  constexpr int BN = 64;               // keys per LDS tile
  constexpr int KS = D / 16;           // k-steps of Q K^T
  constexpr int DB = D / 32;           // 32-row blocks of O^T
  constexpr int KROW = D * 2 + 16;     // LDS bytes per K row, padded against bank conflicts
  constexpr int VROW = BN * 2 + 8;     // LDS bytes per V^T row, padded likewise
  __shared__ __attribute__((aligned(16))) unsigned char k_lds[BN * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[D * VROW];

  const int qt = a.num_qtiles - 1 - (int)blockIdx.x;
  const int h = blockIdx.y;
  const int pr = blockIdx.z;
  const int m0 = qt * BM;
  int L = a.prompt_lens[pr];
  if (L <= m0) return;

  // Row offset of this prompt: the sum of the earlier prompts' lengths.
  const int lane = threadIdx.x & 63;
  long long off = 0;
  for (int i = lane; i < pr; i += 64) off += max(a.prompt_lens[i], 0);
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) off += __shfl_xor(off, sft, 64);
  if (off + L > a.total_tokens) L = (int)max(0ll, (long long)a.total_tokens - off);
  if (L <= m0) return;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 31;
  const int hf = lane >> 5;
  const int qrow0 = m0 + w * 32;  // first query of this wave
  const int qi = qrow0 + ql;      // this lane's query
  const int64_t rs = (int64_t)a.num_heads * D;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + off * rs + (int64_t)h * D;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k) + off * rs + (int64_t)h * D;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v) + off * rs + (int64_t)h * D;

  // Q as the B operand of S^T = K Q^T: k-step kk holds dims kk*16 + hf*8 .. +8.
  uint4 qf[KS];
  if (qi < L) {
    const uint16_t* qp = qb + (int64_t)qi * rs + hf * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = *reinterpret_cast<const uint4*>(qp + kk * 16);
  } else {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = make_uint4(0u, 0u, 0u, 0u);
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float mrow = NEG_BIG, lrow = 0.f;

  const int kend = min(L, m0 + BM);     // keys any query of the workgroup sees
  const int wkend = min(L, qrow0 + 32); // keys any query of this wave sees

  for (int n0 = 0; n0 < kend; n0 += BN) {
    __syncthreads();  // the previous tile's LDS reads are finished
    // K tile, row-major [key][dim]; rows past the prompt are zero.
    for (int idx = threadIdx.x; idx < BN * (D / 8); idx += 256) {
      const int row = idx / (D / 8), ch = idx % (D / 8);
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (n0 + row < L) val = *reinterpret_cast<const uint4*>(kb + (int64_t)(n0 + row) * rs + ch * 8);
      *reinterpret_cast<uint4*>(k_lds + row * KROW + ch * 16) = val;
    }
    // V tile, transposed to [dim][key]: each thread moves 4 keys x 8 dims.
    for (int idx = threadIdx.x; idx < (BN / 4) * (D / 8); idx += 256) {
      const int g = idx % (BN / 4), ch = idx / (BN / 4);
      uint4 rr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = n0 + 4 * g + i;
        rr[i] = key < L ? *reinterpret_cast<const uint4*>(vb + (int64_t)key * rs + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
      }
      const uint32_t w0[4] = {rr[0].x, rr[0].y, rr[0].z, rr[0].w};
      const uint32_t w1[4] = {rr[1].x, rr[1].y, rr[1].z, rr[1].w};
      const uint32_t w2[4] = {rr[2].x, rr[2].y, rr[2].z, rr[2].w};
      const uint32_t w3[4] = {rr[3].x, rr[3].y, rr[3].z, rr[3].w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {  // dword qd holds dims ch*8 + 2qd and 2qd+1
        const uint2 even = make_uint2((w0[qd] & 0xffffu) | (w1[qd] << 16), (w2[qd] & 0xffffu) | (w3[qd] << 16));
        const uint2 odd = make_uint2((w0[qd] >> 16) | (w1[qd] & 0xffff0000u), (w2[qd] >> 16) | (w3[qd] & 0xffff0000u));
        *reinterpret_cast<uint2*>(v_lds + (ch * 8 + 2 * qd) * VROW + g * 8) = even;
        *reinterpret_cast<uint2*>(v_lds + (ch * 8 + 2 * qd + 1) * VROW + g * 8) = odd;
      }
    }
    __syncthreads();
    if (n0 >= wkend) continue;  // every key of this tile is in this wave's future

    // S^T for two 32-key sub-tiles.  Lane (ql, hf) element j is key
    // n0 + sub*32 + 8*(j/4) + 4*hf + j%4 against query qi.
    f32x16_t st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int j = 0; j < 16; ++j) st[sub][j] = 0.f;
      const unsigned char* kr = k_lds + (sub * 32 + ql) * KROW + hf * 16;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) st[sub] = mfma32<E>(*reinterpret_cast<const uint4*>(kr + kk * 32), qf[kk], st[sub]);
    }

    const bool need_mask = (n0 + BN - 1 > qrow0) || (n0 + BN > L);
    float mx = mrow;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = st[sub][j] * a.scale_log2;
        if (need_mask) {
          const int key = n0 + sub * 32 + 8 * (j >> 2) + 4 * hf + (j & 3);
          x = (key > qi || key >= L) ? -INFINITY : x;
        }
        st[sub][j] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = fast_exp2(mrow - mx);
    mrow = mx;

    uint32_t pk[2][8];
    float ps = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        pk[sub][jj] = pack2<E>(fast_exp2(st[sub][2 * jj] - mx), fast_exp2(st[sub][2 * jj + 1] - mx));
        ps += sum2<E>(pk[sub][jj]);
      }
    ps += __shfl_xor(ps, 32, 64);
    lrow = lrow * alpha + ps;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[db][j] *= alpha;

    // O^T += V^T P^T over k-steps of 16 keys.  In step kk2, element i of lane
    // (ql, hf) stands for key n0 + 16*kk2 + 8*(i/4) + 4*hf + i%4, on both operands.
#pragma unroll
    for (int kk2 = 0; kk2 < BN / 16; ++kk2) {
      const int sub = kk2 >> 1, hh = (kk2 & 1) * 4;
      const uint4 pb = make_uint4(pk[sub][hh], pk[sub][hh + 1], pk[sub][hh + 2], pk[sub][hh + 3]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* vr = v_lds + (db * 32 + ql) * VROW;
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + (16 * kk2 + 4 * hf) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + (16 * kk2 + 8 + 4 * hf) * 2);
        o[db] = mfma32<E>(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[db]);
      }
    }
  }

  if (qi < L) {
    const int64_t ob = (off + qi) * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * hf;
        Store4<O>::put(a.out, ob + d0, o[db][4 * grp] / lrow, o[db][4 * grp + 1] / lrow,
                       o[db][4 * grp + 2] / lrow, o[db][4 * grp + 3] / lrow);
      }
  }
}

template <typename E, typename O, int D>
static hipError_t prefill_t(const PrefillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((prefill_kernel<E, O, D>), dim3(a.num_qtiles, a.num_heads, a.num_prompts), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename E>
static hipError_t prefill_d(const PrefillArgs& a, int out_dtype, int head_dim, hipStream_t st) {
  if (head_dim == 128) return out_dtype == 0 ? prefill_t<E, f32_t, 128>(a, st) : prefill_t<E, E, 128>(a, st);
  return out_dtype == 0 ? prefill_t<E, f32_t, 64>(a, st) : prefill_t<E, E, 64>(a, st);
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int out_dtype, int head_dim, hipStream_t st) {
  if (dtype == 1) return prefill_d<f16_t>(a, out_dtype, head_dim, st);
  return prefill_d<bf16_t>(a, out_dtype, head_dim, st);
}

}  // namespace pkv
