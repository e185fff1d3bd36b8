// Shared device helpers of the DSpark round kernels (gfx950 / CDNA4, wave64).
//
// Contents: vector types, an accurate fp32 exp, wave/block reductions, the
// Markov bias block (bf16 MFMA or fp32 FMA), and the workspace layout shared
// by the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Column tile of the draft/residual partials: one workgroup of 4 waves, each
// wave owns 64 consecutive columns.
constexpr int TILE = 256;
constexpr int WCOLS = 64;
// Rows of the gathered W1 block held in LDS per pass (4 MFMA row blocks of 32).
constexpr int RCH = 128;
// Column tile of the target-row partials (16 floats per lane of a wave) and
// the column segment one verify-stream workgroup covers: two such tiles per
// wave (8 per workgroup), one per wave for the greedy arg-max.
constexpr int VTILE = 1024;
__host__ __device__ constexpr int stream_seg(bool greedy) { return (greedy ? 4 : 8) * VTILE; }
constexpr int VSEG = 4 * VTILE;  // the smaller segment (grid-size checks)
// Sentinel "no rejection" position in the per-request rejection slot.
constexpr int NO_REJECT = 1 << 30;

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// exp(x) for the softmax weights: 2^(x log2 e) on v_exp_f32.  The relative
// error is about (|x| + 1) * 6e-8 with a random sign per element; weighted by
// the probabilities it moves a CDF value by far less than 1e-7 (x <= ~0 here:
// arguments are shifted by the running maximum).  Arguments below -100
// return 0 (also -inf); NaN propagates.
__device__ __forceinline__ float exp_acc(float x) {
  const float L2E = 1.44269502162933349609375f;  // fp32 nearest to log2(e)
  const float r = __builtin_amdgcn_exp2f(x * L2E);
  return (x < -100.f) ? 0.f : r;
}

// Weight element to fp32 (bf16 bits are the high half of an fp32).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Element c of 8 bytes of weights (4 bf16 or 2 fp32).
template <typename WT>
__device__ __forceinline__ float elem_of(uint2 v, int c);
template <>
__device__ __forceinline__ float elem_of<uint16_t>(uint2 v, int c) {
  const uint32_t w = (c < 2) ? v.x : v.y;
  return __uint_as_float((c & 1) ? (w & 0xFFFF0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float elem_of<float>(uint2 v, int c) {
  return __uint_as_float(c == 0 ? v.x : v.y);
}

// exp(x) as a bare 2^(x log2 e) (no clamp; -inf gives 0, NaN propagates).
// sc = log2(e) / T folds the temperature into the same multiply.
__device__ __forceinline__ float exp2_scaled(float x, float sc) { return __builtin_amdgcn_exp2f(x * sc); }
constexpr float LOG2E_F = 1.44269502162933349609375f;

__device__ __forceinline__ bool is_bad(float x) { return !(x == x) || __builtin_isinf(x); }

// ---------------------------------------------------------------------------
// cross-lane helpers (wave64)

// Lane exchange without the LDS unit (a __shfl is a ds_bpermute, with an LDS
// round trip per call): DPP moves within 16-lane rows and the gfx950
// permlane swaps between rows.  A butterfly combine takes, in every lane, op
// of the lane's value and its partner's: quad xor 1, quad xor 2, the mirror
// lane within 8 and within 16, then the other row of the row pair (xor 16)
// and the other half of the wave (xor 32).  Both operands of every op are
// the same two values in both partner lanes, so a commutative op leaves the
// same bits in all 64 lanes.
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHR = 0x110;    // + n: lane i of a row reads lane i - n
constexpr int DPP_ROW_ROR = 0x120;    // + n: lane i of a row reads lane (i - n) mod 16
constexpr int DPP_WAVE_SHR1 = 0x138;  // lane i reads lane i - 1
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;  // lane 15 of each row into the next row
constexpr int DPP_ROW_BCAST31 = 0x143;  // lane 31 into rows 2 and 3

// v of the DPP source lane; lanes without a source (or outside ROW_MASK) get old.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(0u, __float_as_uint(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {  // 0.0 where there is no source
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(0u, (uint32_t)b);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>(0u, (uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// The values of a lane and of its partner lane ^ 16 (swap16) or ^ 32 (swap32),
// in an order that depends only on the pair (row-pair low row first).
struct LanePair {
  uint32_t a, b;
};
__device__ __forceinline__ LanePair swap16(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return LanePair{r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return LanePair{r[0], r[1]};
}
__device__ __forceinline__ float max_xor32(float v) {
  const LanePair p = swap32(__float_as_uint(v));
  return fmaxf(__uint_as_float(p.a), __uint_as_float(p.b));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const LanePair p = swap32(__float_as_uint(v));
  return __uint_as_float(p.a) + __uint_as_float(p.b);
}

// Commutative butterfly reduction of a float over the wave (all lanes get it).
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_f32<DPP_QUAD_XOR1>(v));
  v = op(v, dpp_f32<DPP_QUAD_XOR2>(v));
  v = op(v, dpp_f32<DPP_ROW_HALF_MIRROR>(v));
  v = op(v, dpp_f32<DPP_ROW_MIRROR>(v));
  const LanePair p = swap16(__float_as_uint(v));
  v = op(__uint_as_float(p.a), __uint_as_float(p.b));
  const LanePair q = swap32(__float_as_uint(v));
  return op(__uint_as_float(q.a), __uint_as_float(q.b));
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
  v = op(v, (int)dpp_u32<DPP_QUAD_XOR1>(0u, (uint32_t)v));
  v = op(v, (int)dpp_u32<DPP_QUAD_XOR2>(0u, (uint32_t)v));
  v = op(v, (int)dpp_u32<DPP_ROW_HALF_MIRROR>(0u, (uint32_t)v));
  v = op(v, (int)dpp_u32<DPP_ROW_MIRROR>(0u, (uint32_t)v));
  const LanePair p = swap16((uint32_t)v);
  v = op((int)p.a, (int)p.b);
  const LanePair q = swap32((uint32_t)v);
  return op((int)q.a, (int)q.b);
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
// (value, index) maximum with the lowest index on ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float v2 = dpp_f32<CTRL>(v);
  const int i2 = (int)dpp_u32<CTRL>(0u, (uint32_t)i);
  argmax_merge(v, i, v2, i2);
}
__device__ __forceinline__ void argmax_pair(float& v, int& i, LanePair pv, LanePair pi) {
  v = __uint_as_float(pv.a);
  i = (int)pi.a;
  argmax_merge(v, i, __uint_as_float(pv.b), (int)pi.b);
}
// Lane 0 (and every lane whose values are not NaN) gets the wave's argmax.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<DPP_QUAD_XOR1>(v, i);
  argmax_step<DPP_QUAD_XOR2>(v, i);
  argmax_step<DPP_ROW_HALF_MIRROR>(v, i);
  argmax_step<DPP_ROW_MIRROR>(v, i);
  argmax_pair(v, i, swap16(__float_as_uint(v)), swap16((uint32_t)i));
  argmax_pair(v, i, swap32(__float_as_uint(v)), swap32((uint32_t)i));
}
// Value of lane ^ D for D in {1, 2, 4, 8, 16, 32}.
template <int D>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  static_assert(D == 1 || D == 2 || D == 4 || D == 8 || D == 16 || D == 32, "lane distance");
  const int lane = threadIdx.x & 63;
  if constexpr (D == 1) {
    return dpp_u32<DPP_QUAD_XOR1>(0u, v);
  } else if constexpr (D == 2) {
    return dpp_u32<DPP_QUAD_XOR2>(0u, v);
  } else if constexpr (D == 4) {
    const uint32_t down = dpp_u32<DPP_ROW_ROR + 4>(0u, v), up = dpp_u32<DPP_ROW_ROR + 12>(0u, v);
    return (lane & 4) ? down : up;
  } else if constexpr (D == 8) {
    return dpp_u32<DPP_ROW_ROR + 8>(0u, v);
  } else if constexpr (D == 16) {
    const LanePair p = swap16(v);
    return ((lane >> 4) & 1) ? p.a : p.b;
  } else {
    const LanePair p = swap32(v);
    return (lane >> 5) ? p.a : p.b;
  }
}
template <int D>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t v) {
  return ((uint64_t)lane_xor_u32<D>((uint32_t)(v >> 32)) << 32) | lane_xor_u32<D>((uint32_t)v);
}
// argmax with the partner lane ^ 32 only
__device__ __forceinline__ void argmax_xor32(float& v, int& i) {
  argmax_pair(v, i, swap32(__float_as_uint(v)), swap32((uint32_t)i));
}

// Block-wide exclusive scan of one value per thread (blockDim.x == 256):
// thread t gets the sum of the values of threads 0..t-1, computed by a fixed
// tree (deterministic).  `tmp` is __shared__ T[256].
template <typename T>
__device__ __forceinline__ T block_exscan_256(T v, T* tmp) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  const T shifted = (t > 0) ? tmp[t - 1] : T(0);
  __syncthreads();
  tmp[t] = shifted;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const T add = (t >= o) ? tmp[t - o] : T(0);
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const T ex = tmp[t];
  __syncthreads();
  return ex;
}

__device__ __forceinline__ void raise_err(int32_t* err, int bits) { atomicOr(err, bits); }

__device__ __forceinline__ int checked_token(int tok, int V, int32_t* err) {
  if (tok < 0 || tok >= V) {
    raise_err(err, DSPARK_DERR_TOKEN);
    return 0;
  }
  return tok;
}
__device__ __forceinline__ float checked_uniform(float u, int32_t* err) {
  if (!(u >= 0.f && u < 1.f)) {
    raise_err(err, DSPARK_DERR_UNIFORM);
    return 0.f;
  }
  return u;
}

// Streaming loads (non-temporal: logit rows and W2 are read once per pass).
__device__ __forceinline__ f32x4 ld_stream4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ uint32_t ld_stream_u32(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Raw buffer loads: a uniform (SGPR) resource, one 32-bit per-lane byte offset
// and a uniform byte offset per load, so long unrolled load sequences cost one
// VGPR of address instead of a 64-bit address pair each.  Offsets at or past
// num_records read 0.  AUX_NT marks the load non-temporal.
constexpr int AUX_NT = 2;
// W2 is re-read every draft step: plain (temporal) loads let it stay in the
// memory-side cache while the streamed logit rows go non-temporal.
constexpr int AUX_W2 = 0;
// sc1: device-coherent access.  Stores write through to memory and loads do
// not hit a copy another XCD's L2 may hold; used for every word that one
// workgroup writes and another reads within the same launch.
constexpr int AUX_DEV = 16;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
template <int AUX = AUX_NT>
__device__ __forceinline__ uint32_t buf_u32(rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff, (int)soff, AUX);
}
template <int AUX = AUX_NT>
__device__ __forceinline__ u32x4 buf_u32x4(rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, AUX);
}

// ---------------------------------------------------------------------------
// Markov bias block.
//
// Computes, for up to 4 row blocks of 32 requests (rows of the LDS block A,
// which holds the gathered W1 rows) and the 64 columns [cbase, cbase + 64) a
// wave owns, bias[row][col] = sum_k A[row][k] * W2[k][col] with fp32
// accumulation, in the MFMA 32x32x16 output layout:
//
//   acc[rb][p][t], lane l = 32 h + j:
//     row = 32 rb + j,   col = cbase + 16 (t / 4) + 8 h + 2 (t % 4) + p
//
// The W2 operand is loaded as dwords (columns col, col+1 of one k row), which
// gives two MFMA operands per load (p = 0: even columns, p = 1: odd columns):
// each load instruction reads 2 x 128 contiguous bytes.  Columns >= V (V is a
// multiple of 8) contribute zeros.
//
// load() issues the loads of the whole k range at once (one memory round trip;
// 8 KS dwords per lane) and mma() consumes them, so a caller can put other
// loads in flight between the two.  KS (a power of two >= r/16) is a template
// parameter so the fragment stays in registers; loads are branch-free (invalid
// addresses are clamped to valid memory and the value masked).
constexpr int MAX_KS = DSPARK_MAX_RANK / 16;

template <typename WT>
struct BiasBlock;

template <>
struct BiasBlock<uint16_t> {
  static constexpr int APAD = 8;  // bf16 elements of LDS row padding
  template <int KS>
  struct Frag {
    uint32_t w[KS][8];
  };
  // Columns past V load column 0 (a finite weight): every consumer masks
  // those columns through the logits it adds (-inf there), so no select is
  // applied here and the loads stay in flight until the first MFMA needs them.
  // One k step of the fragment (rows kk*16 + 8h + e, e < 8); ks >= r/16
  // repeats the last step (never multiplied).
  __device__ static __forceinline__ void load_ks(uint32_t (&w)[8], const uint16_t* __restrict__ W2,
                                                 int V, int r, int cbase, int ks) {
    const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
    const int col = cbase + 2 * j;
    const rsrc_t rs = make_rsrc(W2, (size_t)r * V * 2);
    const uint32_t voff = (uint32_t)(8 * h * V + (col < V ? col : 0)) * 2u;
    const int kk = min(ks, r / 16 - 1);
#pragma unroll
    for (int e = 0; e < 8; e++) w[e] = buf_u32<AUX_W2>(rs, voff, (uint32_t)((kk * 16 + e) * V) * 2u);
  }
  template <int KS>
  __device__ static __forceinline__ void load(Frag<KS>& F, const uint16_t* __restrict__ W2, int V,
                                              int r, int cbase) {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) load_ks(F.w[ks], W2, V, r, cbase, ks);
  }
  template <int KS>
  __device__ static __forceinline__ void operands(const Frag<KS>& F, int ks, bf16x8& a0, bf16x8& a1) {
    u32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      lo[e] = (F.w[ks][2 * e] & 0xFFFFu) | (F.w[ks][2 * e + 1] << 16);
      hi[e] = (F.w[ks][2 * e] >> 16) | (F.w[ks][2 * e + 1] & 0xFFFF0000u);
    }
    a0 = __builtin_bit_cast(bf16x8, lo);
    a1 = __builtin_bit_cast(bf16x8, hi);
  }
  // B operand row block rb: rows (rb*32 + j) of A_lds.  All four row blocks are
  // computed (rows past the request count are zero in A_lds), so the loop has
  // no data-dependent branch and the LDS reads of a k step are issued together.
  template <int KS>
  __device__ static __forceinline__ void mma(const Frag<KS>& F, int r, const uint16_t* A_lds,
                                             int a_stride, int /*nrb*/, f32x16 (&acc)[4][2]) {
    const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
    const int nks = r / 16;
    const uint16_t* ap = A_lds + j * a_stride + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      if (ks < nks) {
        u32x4 bb[4];
#pragma unroll
        for (int rb = 0; rb < 4; rb++)
          bb[rb] = *reinterpret_cast<const u32x4*>(ap + rb * 32 * a_stride + ks * 16);
        bf16x8 a0, a1;
        operands(F, ks, a0, a1);
#pragma unroll
        for (int rb = 0; rb < 4; rb++) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, bb[rb]);
          acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[rb][0], 0, 0, 0);
          acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[rb][1], 0, 0, 0);
        }
      }
    }
  }
  // In-place conversion of a loaded fragment to MFMA operand form (w[ks][0..3]
  // = a0, w[ks][4..7] = a1), done once per tile by the partials kernel.
  template <int KS>
  __device__ static __forceinline__ void to_operands(Frag<KS>& F) {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      bf16x8 a0, a1;
      operands(F, ks, a0, a1);
      const u32x4 lo = __builtin_bit_cast(u32x4, a0), hi = __builtin_bit_cast(u32x4, a1);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        F.w[ks][e] = lo[e];
        F.w[ks][4 + e] = hi[e];
      }
    }
  }
  // mma_rb on a fragment already in operand form.  The B operands of all k
  // steps are read from LDS before the MFMA chain starts.
  template <int KS>
  __device__ static __forceinline__ void mma_rb_op(const Frag<KS>& F, int r, const uint16_t* A_rows,
                                                   int a_stride, f32x16 (&acc)[2]) {
    const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
    const int nks = r / 16;
    const uint16_t* ap = A_rows + j * a_stride + 8 * h;
    auto op = [&](int ks, int half) {
      return __builtin_bit_cast(bf16x8, u32x4{F.w[ks][4 * half], F.w[ks][4 * half + 1],
                                              F.w[ks][4 * half + 2], F.w[ks][4 * half + 3]});
    };
    if (nks == KS) {
      u32x4 bb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ks++) bb[ks] = *reinterpret_cast<const u32x4*>(ap + ks * 16);
      // materialise every B operand before the chain (otherwise the
      // scheduler re-reads LDS into one register set and stalls on each)
#pragma unroll
      for (int ks = 0; ks < KS; ks++) asm volatile("" : "+v"(bb[ks]));
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, bb[ks]);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(ks, 0), b, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(ks, 1), b, acc[1], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        if (ks < nks) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ap + ks * 16));
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(ks, 0), b, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(ks, 1), b, acc[1], 0, 0, 0);
        }
      }
    }
  }
  // One row block: rows j of A_rows (32 requests) against the wave's 64
  // columns; acc[p] as in mma.  The full-rank case has no branch in the k loop.
  template <int KS>
  __device__ static __forceinline__ void mma_rb(const Frag<KS>& F, int r, const uint16_t* A_rows,
                                                int a_stride, f32x16 (&acc)[2]) {
    const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
    const int nks = r / 16;
    const uint16_t* ap = A_rows + j * a_stride + 8 * h;
    if (nks == KS) {
      u32x4 bb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ks++) bb[ks] = *reinterpret_cast<const u32x4*>(ap + ks * 16);
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        bf16x8 a0, a1;
        operands(F, ks, a0, a1);
        const bf16x8 b = __builtin_bit_cast(bf16x8, bb[ks]);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        if (ks < nks) {
          bf16x8 a0, a1;
          operands(F, ks, a0, a1);
          const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ap + ks * 16));
          acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0], 0, 0, 0);
          acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1], 0, 0, 0);
        }
      }
    }
  }
  // W1 row fragments of one request (lanes with j == 0 hold W1[tok][ks*16 + 8h .. +8],
  // the others zero) for mma_row.
  template <int KS>
  struct Row {
    u32x4 b[KS];
  };
  template <int KS>
  __device__ static __forceinline__ void load_row(Row<KS>& B, const uint16_t* __restrict__ W1, int r,
                                                  int tok) {
    const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
    const int nks = r / 16;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int kk = min(ks, nks - 1);
      const u32x4 x = *reinterpret_cast<const u32x4*>(W1 + (size_t)tok * r + kk * 16 + 8 * h);
      B.b[ks] = (j == 0 && ks < nks) ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Output row 0 of row block 0 (the request whose W1 row is in B).
  template <int KS>
  __device__ static __forceinline__ void mma_row(const Frag<KS>& F, int r, const Row<KS>& B,
                                                 f32x16 (&acc)[2]) {
    const int nks = r / 16;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      if (ks < nks) {
        bf16x8 a0, a1;
        operands(F, ks, a0, a1);
        const bf16x8 bb = __builtin_bit_cast(bf16x8, B.b[ks]);
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bb, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bb, acc[1], 0, 0, 0);
      }
    }
  }
};

// fp32 factors: same lane/element mapping, scalar FMA in ascending k.  W2 is
// read inside mma (the fp32 path is the small-workload path).
template <>
struct BiasBlock<float> {
  static constexpr int APAD = 4;
  template <int KS>
  struct Frag {
    const float* W2;
    int V, cbase;
  };
  template <int KS>
  __device__ static __forceinline__ void load(Frag<KS>& F, const float* __restrict__ W2, int V, int,
                                              int cbase) {
    F.W2 = W2;
    F.V = V;
    F.cbase = cbase;
  }
  // Row k of W2 at the lane's columns c0 + 2 q + p -> w[g][p][q], c0 = cbase
  // + 16 g + 8 h: two 16-byte loads per group.  c0 and V are multiples of 8,
  // so a group's eight columns lie all below V or all past it (then 0).
  template <int KS>
  __device__ static __forceinline__ void w2_at(const Frag<KS>& F, int k, float (&w)[4][2][4]) {
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int g = 0; g < 4; g++) {
      const int c0 = F.cbase + 16 * g + 8 * h;
      float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
      if (c0 < F.V) {
        const float4* src = reinterpret_cast<const float4*>(F.W2 + (size_t)k * F.V + c0);
        lo = src[0];
        hi = src[1];
      }
      w[g][0][0] = lo.x; w[g][1][0] = lo.y; w[g][0][1] = lo.z; w[g][1][1] = lo.w;
      w[g][0][2] = hi.x; w[g][1][2] = hi.y; w[g][0][3] = hi.z; w[g][1][3] = hi.w;
    }
  }
  template <int KS>
  __device__ static inline void mma(const Frag<KS>& F, int r, const float* A_lds, int a_stride,
                                    int nrb, f32x16 (&acc)[4][2]) {
    const int j = (threadIdx.x & 63) & 31;
#pragma unroll 4
    for (int k = 0; k < r; k++) {
      float w[4][2][4];
      w2_at(F, k, w);
#pragma unroll
      for (int rb = 0; rb < 4; rb++) {
        if (rb < nrb) {  // fp32 path: skip empty row blocks
          const float a = A_lds[(rb * 32 + j) * a_stride + k];
#pragma unroll
          for (int g = 0; g < 4; g++)
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
              for (int p = 0; p < 2; p++) acc[rb][p][4 * g + q] = fmaf(a, w[g][p][q], acc[rb][p][4 * g + q]);
        }
      }
    }
  }
  template <int KS>
  __device__ static __forceinline__ void to_operands(Frag<KS>&) {}
  template <int KS>
  __device__ static inline void mma_rb_op(const Frag<KS>& F, int r, const float* A_rows, int a_stride,
                                          f32x16 (&acc)[2]) {
    mma_rb<KS>(F, r, A_rows, a_stride, acc);
  }
  template <int KS>
  __device__ static inline void mma_rb(const Frag<KS>& F, int r, const float* A_rows, int a_stride,
                                       f32x16 (&acc)[2]) {
    const int j = (threadIdx.x & 63) & 31;
#pragma unroll 4
    for (int k = 0; k < r; k++) {
      float w[4][2][4];
      w2_at(F, k, w);
      const float a = A_rows[j * a_stride + k];
#pragma unroll
      for (int g = 0; g < 4; g++)
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int p = 0; p < 2; p++) acc[p][4 * g + q] = fmaf(a, w[g][p][q], acc[p][4 * g + q]);
    }
  }
  template <int KS>
  struct Row {
    const float* w1;
  };
  template <int KS>
  __device__ static __forceinline__ void load_row(Row<KS>& B, const float* __restrict__ W1, int r,
                                                  int tok) {
    B.w1 = W1 + (size_t)tok * r;
  }
  template <int KS>
  __device__ static inline void mma_row(const Frag<KS>& F, int r, const Row<KS>& B,
                                        f32x16 (&acc)[2]) {
#pragma unroll 4
    for (int k = 0; k < r; k++) {
      float w[4][2][4];
      w2_at(F, k, w);
      const float a = B.w1[k];
#pragma unroll
      for (int g = 0; g < 4; g++)
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int p = 0; p < 2; p++) acc[p][4 * g + q] = fmaf(a, w[g][p][q], acc[p][4 * g + q]);
    }
  }
};

// Number of 16-wide k steps rounded up to a power of two (template dispatch).
__host__ __device__ inline int ks_bucket(int r) {
  const int n = r / 16;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 16;
}
#define DSPARK_DISPATCH_KS(r, BODY)                  \
  switch (ks_bucket(r)) {                            \
    case 1: { constexpr int KS = 1; BODY; } break;   \
    case 2: { constexpr int KS = 2; BODY; } break;   \
    case 4: { constexpr int KS = 4; BODY; } break;   \
    case 8: { constexpr int KS = 8; BODY; } break;   \
    default: { constexpr int KS = 16; BODY; } break; \
  }

// Gather rows A[i] = W1[tok(i)] (i < nrows; the rest zero) into LDS: every
// thread first issues all of its 16-byte loads (branch-free: a zero row loads
// row 0 and is masked), then stores them.  tok(i) is supplied by a functor; a
// negative token gives a zero row.  rows_cap * (r / EPV) must not exceed
// 256 * PER, PER = the per-thread piece count (blockDim.x == 256).
template <typename WT, int PER>
struct W1Gather {
  u32x4 v[PER];
  int dst[PER];
  // Issue the loads (registers only).
  template <typename TokF>
  __device__ __forceinline__ void load(const WT* __restrict__ W1, int V, int r, int nrows, int rows_cap,
                                       int a_stride, TokF tok_of) {
    constexpr int EPV = 16 / sizeof(WT);  // elements per 16-byte piece
    const int pieces = r / EPV;
    const int total = rows_cap * pieces;
    const rsrc_t rs = make_rsrc(W1, (size_t)V * r * sizeof(WT));
#pragma unroll
    for (int i = 0; i < PER; i++) {
      const int idx = threadIdx.x + 256 * i;
      const int row = idx / pieces, pc = idx - row * pieces;
      int t = -1;
      if (idx < total && row < nrows) t = tok_of(row);
      const u32x4 x = buf_u32x4<0>(rs, (uint32_t)(max(t, 0) * r + pc * EPV) * (uint32_t)sizeof(WT), 0u);
      v[i] = (t >= 0) ? x : u32x4{0u, 0u, 0u, 0u};
      dst[i] = (idx < total) ? row * a_stride + pc * EPV : -1;
    }
  }
  __device__ __forceinline__ void store(WT* A_lds) const {
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (dst[i] >= 0) *reinterpret_cast<u32x4*>(A_lds + dst[i]) = v[i];
  }
};

template <typename WT, int PER, typename TokF>
__device__ __forceinline__ void gather_w1_rows(const WT* __restrict__ W1, int V, int r, int nrows,
                                               int rows_cap, WT* A_lds, int a_stride, TokF tok_of) {
  W1Gather<WT, PER> g;
  g.load(W1, V, r, nrows, rows_cap, a_stride, tok_of);
  g.store(A_lds);
}

// Logit values of one row at the columns a lane holds in the bias-block
// layout: out[p][t] for col = cbase + 16 (t/4) + 8 h + 2 (t%4) + p.  The rows
// are addressed through a buffer resource `rs` anchored at a row-set start and
// the lane's row byte offset `roff`.  Invalid rows/columns read as -inf.
__device__ __forceinline__ void load_row_cols(rsrc_t rs, uint32_t roff, bool rowv, int V, int cbase,
                                              float (&out)[2][16]) {
  const int h = (threadIdx.x & 63) >> 5;
  const int c0 = cbase + 8 * h;
  const uint32_t voff = rowv ? roff + (uint32_t)c0 * 4u : 0u;
#pragma unroll
  for (int g = 0; g < 4; g++) {
    const bool ok = rowv && c0 + 16 * g < V;
    const f32x4 lo = __builtin_bit_cast(f32x4, buf_u32x4(rs, voff, (uint32_t)g * 64u));
    const f32x4 hi = __builtin_bit_cast(f32x4, buf_u32x4(rs, voff, (uint32_t)g * 64u + 16u));
    const float ninf = -INFINITY;
    out[0][4 * g + 0] = ok ? lo[0] : ninf;
    out[1][4 * g + 0] = ok ? lo[1] : ninf;
    out[0][4 * g + 1] = ok ? lo[2] : ninf;
    out[1][4 * g + 1] = ok ? lo[3] : ninf;
    out[0][4 * g + 2] = ok ? hi[0] : ninf;
    out[1][4 * g + 2] = ok ? hi[1] : ninf;
    out[0][4 * g + 3] = ok ? hi[2] : ninf;
    out[1][4 * g + 3] = ok ? hi[3] : ninf;
  }
}

// Row-contiguous staging of logit rows through LDS.  Reading a 32-row block
// so that each load instruction covers 1 KiB of a single row (instead of one
// 32-byte piece of 32 rows, as the MFMA output layout would) doubles the
// achieved HBM bandwidth on rows that are megabytes apart.
//
// Block rb of a 128-row chunk: wave w loads rows 4i + w (i = 0..7) of the
// block, lane l columns [tile0 + 4l, tile0 + 4l + 4).  Staged row stride:
constexpr int BSTRIDE = TILE + 4;  // floats

__device__ __forceinline__ void stage_load(u32x4 (&v)[8], rsrc_t rs, uint32_t row_bytes, int rb,
                                           int nrows, int V, int tile0) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = tile0 + 4 * lane;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int rl = rb * 32 + 4 * i + wave;
    const bool ok = rl < nrows && col < V;
    v[i] = buf_u32x4(rs, ok ? (uint32_t)rl * row_bytes + (uint32_t)col * 4u : 0u, 0u);
  }
}
__device__ __forceinline__ void stage_store(const u32x4 (&v)[8], float* X) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; i++) *reinterpret_cast<u32x4*>(X + (4 * i + wave) * BSTRIDE + 4 * lane) = v[i];
}
// Direct-to-LDS variant: the 32 rows of block rb go straight from memory to
// X + i * BSTRIDE (row i of the block) with 16-byte loads, one 1 KiB row
// piece per instruction and no register staging.  Wave w issues rows w, w+4,
// ... (always 8 loads per wave, so vmcnt-based waits can count them; rows past
// nrows re-read row 0 and are masked by the reader).  The whole offset is in
// the per-lane voffset, which the buffer range check covers: columns past V
// read the following row or, past the resource, zero; the reader masks them.
__device__ __forceinline__ void stage_dma(rsrc_t rs, uint32_t row_bytes, int rb, int nrows, int tile0,
                                          float* X) {
  // the LDS address (M0) must be provably wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t coff = (uint32_t)(tile0 + 4 * lane) * 4u;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int rl = rb * 32 + 4 * i + wave;
    const uint32_t voff = (rl < nrows ? (uint32_t)rl * row_bytes : 0u) + coff;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(X + (4 * i + wave) * BSTRIDE), 16, (int)voff, 0, 0,
        AUX_NT);
  }
}
// Workgroup barrier for LDS traffic: completes this wave's LDS operations and
// meets the other waves.  Unlike __syncthreads it does not wait for the
// wave's outstanding global loads, so direct-to-LDS loads issued for later
// units stay in flight; data they write is waited for explicitly (wait_vmcnt)
// before the barrier that publishes it.  The memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14] (count up to 63), expcnt [6:4] and lgkmcnt
// [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Same without any masking (every column of the tile is below V; rows past
// the request count are never reported).
__device__ __forceinline__ void stage_read_full(const float* X, int wcol0, float (&out)[2][16]) {
  const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; g++) {
    const int c = wcol0 + 16 * g + 8 * h;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(X + j * BSTRIDE + c);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(X + j * BSTRIDE + c + 4);
    out[0][4 * g + 0] = lo[0];
    out[1][4 * g + 0] = lo[1];
    out[0][4 * g + 1] = lo[2];
    out[1][4 * g + 1] = lo[3];
    out[0][4 * g + 2] = hi[0];
    out[1][4 * g + 2] = hi[1];
    out[0][4 * g + 3] = hi[2];
    out[1][4 * g + 3] = hi[3];
  }
}
// The lane's bias-block columns of staged row j (= lane & 31); invalid -> -inf.
__device__ __forceinline__ void stage_read(const float* X, bool rowv, int V, int cbase, int wcol0,
                                           float (&out)[2][16]) {
  const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; g++) {
    const int c = wcol0 + 16 * g + 8 * h;
    const bool ok = rowv && cbase + 16 * g + 8 * h < V;
    const f32x4 lo = *reinterpret_cast<const f32x4*>(X + j * BSTRIDE + c);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(X + j * BSTRIDE + c + 4);
    const float ninf = -INFINITY;
    out[0][4 * g + 0] = ok ? lo[0] : ninf;
    out[1][4 * g + 0] = ok ? lo[1] : ninf;
    out[0][4 * g + 1] = ok ? lo[2] : ninf;
    out[1][4 * g + 1] = ok ? lo[3] : ninf;
    out[0][4 * g + 2] = ok ? hi[0] : ninf;
    out[1][4 * g + 2] = ok ? hi[1] : ninf;
    out[0][4 * g + 3] = ok ? hi[2] : ninf;
    out[1][4 * g + 3] = ok ? hi[3] : ninf;
  }
}

// Column (relative to cbase) of element (p, t) for a lane with half h.
__device__ __forceinline__ int elem_col(int p, int t, int h) {
  return 16 * (t >> 2) + 8 * h + 2 * (t & 3) + p;
}

// Tree sum of the 32 values a lane holds (fixed order: deterministic).
__device__ __forceinline__ float tree_sum32(const float (&e)[2][16]) {
  float s[16];
#pragma unroll
  for (int t = 0; t < 16; t++) s[t] = e[0][t] + e[1][t];
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
    for (int t = 0; t < w; t++) s[t] = s[t] + s[t + w];
  return s[0];
}

// ---------------------------------------------------------------------------
// Workspace layout (identical on host and device).  All offsets 256-aligned.
// RNN head parameters and its state table (see k_rnn_state).
struct RnnHead {
  const void* Wx;      // [3][r][r] input weights of the update, reset and candidate gates
  const void* Ws;      // [3][r][r] recurrent weights, same gate order
  const float* bias;   // [3][r]
  void* states;        // [R][gamma][r] out: s_1..s_gamma in the weights' storage type
  double* gates;       // workspace [3][R][r]: u, candidate input part, g * s
};

// Parts of dspark_verify: the target-row stream (independent of the draft)
// and the rest.
enum { VERIFY_ALL = 0, VERIFY_STREAM = 1, VERIFY_FINISH = 2 };

// Sync region of the fused draft (at a fixed offset): epoch and done
// counter, then one tagged token word per request (up to 1024 requests).
constexpr size_t SYNC_EPOCH = 0;
constexpr size_t SYNC_DONE = 4;
constexpr size_t SYNC_TOKW = 256;
constexpr size_t SYNC_BYTES = SYNC_TOKW + 8 * 1024;
// Bytes of one sealed tile record of the fused draft: two 16-byte words of
// three payload dwords and a seal.
constexpr size_t FREC_BYTES = 32;
// Real-time limit of one fused-draft wait (s_memrealtime runs at 100 MHz).
constexpr uint64_t FUSED_SPIN_TICKS = 50000000ull;

struct WsLayout {
  size_t err;      // int32 error word
  size_t sync;     // fused-draft sync words (SYNC_* offsets)
  size_t trec;     // float4 [R][nt][2]     draft tile records (see select.h)
  size_t rowstat;  // double2[R][gamma+1]   target row (max, sum) or (max, argmax)
  size_t rej;      // int32  [R]            first rejected position (NO_REJECT if none)
  size_t vpart;    // float2 [R][gamma+1][nvt] target 1024-column tile partials
  size_t tp;       // float  [R][gamma]     p_k(x_k) of evaluated positions
  size_t rrec;     // float4 [R][nt][2]     residual tile records
  size_t tvpart;   // float  [R*gamma][nt]  acceptance-label tile sums
  size_t rnn;      // double [3][R][256]   RNN head gate outputs (update, candidate input part, reset * state)
  size_t frec;     // [R][nt] x FREC_BYTES   sealed tile records of the fused draft
  size_t total;
};

__host__ __device__ inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(int R, int gamma, int V) {
  WsLayout L;
  const size_t nt = (size_t)ceil_div(V, TILE), nvt = (size_t)ceil_div(V, VTILE);
  size_t o = 0;
  L.err = o;      o = ws_align(o + 256);
  L.sync = o;     o = ws_align(o + SYNC_BYTES);
  L.trec = o;     o = ws_align(o + (size_t)R * nt * 32);
  L.rowstat = o;  o = ws_align(o + (size_t)R * (gamma + 1) * 16);
  L.rej = o;      o = ws_align(o + (size_t)R * 4);
  L.vpart = o;    o = ws_align(o + (size_t)R * (gamma + 1) * nvt * 8);
  L.tp = o;       o = ws_align(o + (size_t)R * gamma * 4);
  L.rrec = o;     o = ws_align(o + (size_t)R * nt * 32);
  L.tvpart = o;   o = ws_align(o + (size_t)R * gamma * nt * 4);
  L.rnn = o;      o = ws_align(o + (size_t)3 * R * DSPARK_MAX_RANK * 8);
  L.frec = o;     o = ws_align(o + (size_t)R * nt * FREC_BYTES);
  L.total = o;
  return L;
}

// Compute units of the current device (host side; one workgroup per CU for the
// persistent tile loops).
int device_cu_count();

// Launch-timing hook (host side, thread-local): see dspark_profile_arm.
void prof_before(int kid, hipStream_t stream);
void prof_after(int kid, hipStream_t stream);
// Launches to issue for one call site of kernel kid (more than 1 only while
// the timing hook is armed with a repeat count for it).
int prof_repeat(int kid);

template <typename T>
__host__ __device__ inline T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

// The parts of a workspace the draft uses: the error word, the one-launch
// draft's sync words (SYNC_* offsets) and sealed tile records, and the
// per-step path's tile records (each R * ceil(V / 256) * 32 bytes; a call
// uses one of the two record regions, so they may coincide).
struct DraftWs {
  int32_t* err;
  uint8_t* sync;
  uint32_t* frec;
  float4* trec;
};
__host__ inline DraftWs draft_ws(void* ws, int R, int gamma, int V) {
  const WsLayout L = ws_layout(R, gamma, V);
  return DraftWs{ws_ptr<int32_t>(ws, L.err), ws_ptr<uint8_t>(ws, L.sync), ws_ptr<uint32_t>(ws, L.frec),
                 ws_ptr<float4>(ws, L.trec)};
}

}  // namespace dspark
