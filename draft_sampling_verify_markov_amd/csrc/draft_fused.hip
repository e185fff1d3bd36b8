// Markov-head sequential drafting, all gamma steps in one persistent launch.
//
// Source: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), section "Arquitetura": Semi-Autoregressive Generation
// and the Markov head (the bias of position k is W1[x_{k-1}] . W2, added to the
// base logits, then x_k is sampled; positions are sequential, requests and
// vocabulary columns are data-parallel).  Same arithmetic as the per-step
// kernels in draft.hip; this file changes where the data lives:
//
//   * one workgroup per compute unit (all resident at once), each owning the
//     256-column tiles b and b + G of the vocabulary;
//   * the W2 fragments of those tiles are loaded into registers once and stay
//     there for all gamma steps (W2 is read from HBM once per call instead of
//     once per step);
//   * per step: bias MFMA + base add + softmax tile records for every request
//     (as k_draft_partials); the workgroups b, b + G, ... < R each draw
//     request b's token (as k_draft_select) and publish it; every workgroup
//     gathers the new tokens' W1 rows and goes on;
//   * the units of a step are software-pipelined in every wave: the MFMA
//     chain of the next unit is issued interleaved with the epilogue (max,
//     exponentials, sums) of the current one and with the direct-to-LDS loads
//     of the unit after next, so the matrix and vector units work at once;
//   * the next step's first base rows are loaded while the token words are
//     awaited.
//
// Cross-workgroup exchange.  The eight XCDs of the chip have separate L2
// caches, so every word another workgroup reads is written and read with the
// device-coherent cache policy (sc1: written through to memory, read past a
// possibly stale L2 copy): the tile records and the token words.  Each
// 16-byte record word carries a seal (the tag epoch + step mixed with its
// payload) and a token word is (tag << 32) | token, so a reader polls the
// words themselves until they carry the tag it needs: no flag, no fence (an
// L2 writeback and invalidate) and no wait for store completion.  The
// per-workspace epoch is advanced by gamma by the last workgroup to finish,
// so the tags of one call never match another's and nothing needs clearing
// between calls (the workspace is cleared once, at init).  Every wait is
// bounded by a real-time limit; on expiry the kernel sets DSPARK_DERR_SYNC
// and all workgroups still run to completion.
#include <cstdlib>

#include "select.h"

namespace dspark {

// Largest request count of the fused launch (tokens of a step held in LDS).
constexpr int FUSED_MAX_R = 1024;
// Largest tile count (vocabulary <= 512 * 256 columns): a drawing thread
// polls the records of at most two tiles.
constexpr int FUSED_MAX_NT = 512;
constexpr int FUSED_TPL = FUSED_MAX_NT / 256;

struct FusedArgs {
  const float* base;
  const uint16_t* W1;
  const uint16_t* W2;
  const int32_t* anchor;
  const float* u_draft;
  int R, gamma, V, r;
  float T, invT;
  int32_t* tokens;
  float* probs;
  float* stats;
  uint32_t* frec;  // [R][nt] sealed tile records, FREC_BYTES each
  int32_t* err;
  uint32_t* epoch;
  uint32_t* done;
  uint64_t* tokw;   // [R] (tag << 32) | token
  uint64_t spin_ticks;
};

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Seal of a 16-byte record word: the tag (epoch + step) mixed with the
// word's three payload dwords.  A reader accepts a word when its fourth dword
// equals seal(want, payload): a word of another step fails on the tag, and a
// word read torn between two writes fails on the payload (a false accept needs
// a 32-bit collision).
__device__ __forceinline__ uint32_t seal(uint32_t tag, uint32_t a, uint32_t b, uint32_t c) {
  const uint32_t h = a * 0x9E3779B1u + __builtin_rotateleft32(b, 11) * 0x85EBCA77u +
                     __builtin_rotateleft32(c, 23) * 0xC2B2AE3Du;
  return tag ^ h ^ (h >> 15);
}

// Bias block of one 32-request row block against the wave's 64 columns on a
// resident operand-form W2 fragment (r == 16 KS): the B operands are read
// from LDS eight k steps at a time, which keeps the register footprint below
// what a co-running kernel's wave needs.
template <int KS>
__device__ __forceinline__ void mma_resident(const typename BiasBlock<uint16_t>::template Frag<KS>& F,
                                             const uint16_t* A_rows, int a_stride, f32x16 (&acc)[2]) {
  constexpr int BATCH = KS < 8 ? KS : 8;
  const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
  const uint16_t* ap = A_rows + j * a_stride + 8 * h;
#pragma unroll
  for (int k0 = 0; k0 < KS; k0 += BATCH) {
    u32x4 bb[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; i++) bb[i] = *reinterpret_cast<const u32x4*>(ap + (k0 + i) * 16);
#pragma unroll
    for (int i = 0; i < BATCH; i++) asm volatile("" : "+v"(bb[i]));
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      const int ks = k0 + i;
      const bf16x8 b = __builtin_bit_cast(bf16x8, bb[i]);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][0], F.w[ks][1], F.w[ks][2], F.w[ks][3]});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][4], F.w[ks][5], F.w[ks][6], F.w[ks][7]});
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1], 0, 0, 0);
    }
  }
}

// Direct-to-LDS loads of one unit's 32 base rows (as stage_dma), issued one
// 1 KiB row piece per wave at a time; `on` (wave-uniform) is false when the
// unit lies past the step, whose rows are issued after the draws.
struct DmaPlan {
  rsrc_t rs;
  uint32_t row_bytes, coff;
  int rb, nrows;
  float* X;
  bool on;
};
__device__ __forceinline__ void dma_row(const DmaPlan& d, int i) {
  if (!d.on) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = d.rb * 32 + 4 * i + wave;
  const uint32_t voff = (rl < d.nrows ? (uint32_t)rl * d.row_bytes : 0u) + d.coff;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      d.rs, (__attribute__((address_space(3))) void*)(d.X + (4 * i + wave) * BSTRIDE), 16, (int)voff, 0, 0, AUX_NT);
}

// Where a unit's per-wave reduction goes: row rl of this wave's slice of the
// workgroup's LDS reduction arrays.
struct UnitOut {
  float (*m)[RCH];
  float (*s)[RCH];
  int (*i)[RCH];
  int wave, rl;
  int32_t* err;
};

// One pipelined unit step of a wave: the 8 direct-to-LDS row loads of a later
// unit first, then 8 parts fenced by sched_barrier: part p issues the MFMAs
// of k steps [p KS / 8, (p + 1) KS / 8) of the NEXT unit's bias block (rows
// A_next against the resident fragment F, into accN) and one eighth of the
// epilogue of the current unit (accC + base values bv: the maximum, the
// exponentials and their fixed-order tree sum, the cross-half reduction and
// the LDS write; greedy: the arg-max).  The fences keep the VALU
// work of the epilogue in the shadow of the MFMAs instead of after them; the
// arithmetic and its order are those of the unpipelined loop, so the results
// are bit-identical.  The B operands of part p + 1 are read from LDS during
// part p.
template <int KS, bool GREEDY, bool NEXT>
__device__ __forceinline__ void unit_block(const typename BiasBlock<uint16_t>::template Frag<KS>& F,
                                           const uint16_t* A_next, int a_stride, f32x16 (&accN)[2],
                                           const f32x16 (&accC)[2], const float (&bv)[2][16], float sc, int cbase,
                                           const DmaPlan& dma, const UnitOut& o) {
  constexpr int NP = 8;
  constexpr int KPP = (KS + NP - 1) / NP;  // k steps per part, at most
  const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
  const uint16_t* ap = A_next + j * a_stride + 8 * h;
  u32x4 bcur[KPP], bnext[KPP];
  if (NEXT) {
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
      for (int t = 0; t < 16; t++) accN[p][t] = 0.f;
#pragma unroll
    for (int i = 0; i < KPP; i++)
      if (i < KS / NP) bcur[i] = *reinterpret_cast<const u32x4*>(ap + i * 16);
  }
  // the later unit's row loads, all at once: issued while the memory
  // pipeline has room (one per part stalled the wave at each part instead)
#pragma unroll
  for (int q = 0; q < NP; q++) dma_row(dma, q);
  float ml = -INFINITY, mw = 0.f, mref = 0.f;
  float s[8];
  float gv = -INFINITY;
  int gi = 0x7fffffff;
  bool bad = false;
#pragma unroll
  for (int p = 0; p < NP; p++) {
    if (NEXT) {
      const int k0 = p * KS / NP, k1 = (p + 1) * KS / NP;
      if (p + 1 < NP) {
        const int n0 = k1, n1 = (p + 2) * KS / NP;
#pragma unroll
        for (int i = 0; i < KPP; i++)
          if (n0 + i < n1) bnext[i] = *reinterpret_cast<const u32x4*>(ap + (n0 + i) * 16);
      }
#pragma unroll
      for (int i = 0; i < KPP; i++) {
        if (k0 + i < k1) {
          const int ks = k0 + i;
          const bf16x8 bb = __builtin_bit_cast(bf16x8, bcur[i]);
          const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][0], F.w[ks][1], F.w[ks][2], F.w[ks][3]});
          const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][4], F.w[ks][5], F.w[ks][6], F.w[ks][7]});
          accN[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bb, accN[0], 0, 0, 0);
          accN[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bb, accN[1], 0, 0, 0);
        }
      }
    }
    if (GREEDY) {
      if (p < 4) {
#pragma unroll
        for (int t = 4 * p; t < 4 * p + 4; t++)
#pragma unroll
          for (int q = 0; q < 2; q++) {
            const float z = bv[q][t] + accC[q][t];
            bad |= (z != z);
            if (z > gv) { gv = z; gi = cbase + elem_col(q, t, h); }
          }
      } else if (p == 4) {
        if (bad) raise_err(o.err, DSPARK_DERR_NONFINITE);
        argmax_xor32(gv, gi);
      } else if (p == 5) {
        if (h == 0) { o.m[o.wave][o.rl] = gv; o.i[o.wave][o.rl] = gi; }
      }
    } else {
      if (p < 2) {
#pragma unroll
        for (int t = 8 * p; t < 8 * p + 8; t++)
#pragma unroll
          for (int q = 0; q < 2; q++) ml = fmaxf(ml, bv[q][t] + accC[q][t]);
        if (p == 1) {
          mw = max_xor32(ml);
          mref = (mw == -INFINITY) ? 0.f : mw;
        }
      } else if (p < 6) {
        // pair sums s_t = e[0][t] + e[1][t], and the first level of the
        // fixed tree (s_t + s_{t+8}) as soon as both terms exist
#pragma unroll
        for (int t = 4 * (p - 2); t < 4 * (p - 2) + 4; t++) {
          const float st = exp2_scaled((bv[0][t] - mref) + accC[0][t], sc) +
                           exp2_scaled((bv[1][t] - mref) + accC[1][t], sc);
          if (t < 8)
            s[t] = st;
          else
            s[t - 8] = s[t - 8] + st;
        }
      } else if (p == 6) {
#pragma unroll
        for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
          for (int t = 0; t < w; t++) s[t] = s[t] + s[t + w];
      } else {
        const float sw = sum_xor32(s[0]);
        if (h == 0) { o.m[o.wave][o.rl] = mw; o.s[o.wave][o.rl] = sw; }
      }
    }
    if (NEXT) {
#pragma unroll
      for (int i = 0; i < KPP; i++) bcur[i] = bnext[i];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 472 of the 512 registers per lane: a 40-register wave of a kernel on another
// stream (verify's target-row stream, the scheduler) still fits beside every
// wave of this one.
// Built with MFMA results in VGPRs (-amdgpu-mfma-vgpr-form): the AGPRs hold
// the resident W2 fragments.
template <int KS, bool GREEDY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1), amdgpu_num_vgpr(236))) void k_draft_fused(FusedArgs P) {
  using WT = uint16_t;
  using BB = BiasBlock<WT>;
  constexpr int APAD = BB::APAD;
  constexpr int CH = RCH;
  constexpr int GPER = CH * (KS * 16 / 8) / 256;
  __shared__ __align__(16) WT A_lds[CH * (DSPARK_MAX_RANK + APAD)];
  __shared__ __align__(16) float X[2][32 * BSTRIDE];
  __shared__ float red_m[4][CH];
  __shared__ float red_s[4][CH];
  __shared__ int red_i[4][CH];
  __shared__ int s_tok[FUSED_MAX_R];
  __shared__ BlockSelectSmem sm;
  __shared__ float w1s[DSPARK_MAX_RANK];
  __shared__ float part[16][WCOLS];
  __shared__ float gm[4];
  __shared__ int gi[4];
  __shared__ uint32_t s_E;
  __shared__ int s_ok;

  // the waves of a kernel beside this one (verify's target-row stream) share
  // every SIMD: let this kernel's wave issue first when both are ready
  __builtin_amdgcn_s_setprio(3);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, h = lane >> 5;
  const int G = gridDim.x, b = blockIdx.x;
  const int nt = ceil_div(P.V, TILE);
  const int ntl = (b < nt ? 1 : 0) + (b + G < nt ? 1 : 0);
  const bool t_one = (P.T == 1.0f);
  const uint32_t row_bytes = (uint32_t)(P.gamma * P.V) * 4u;
  const int a_stride = P.r + APAD;
  const int nch = ceil_div(P.R, CH);
  const int last_rows = P.R - (nch - 1) * CH;
  const int nrb_last = ceil_div(last_rows, 32);
  const int ups = ntl * ((nch - 1) * (CH / 32) + nrb_last);  // units per step
  const int total = ups * P.gamma;
  const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + P.spin_ticks;

  if (tid == 0) {
    s_E = ld_dev(P.epoch);
    s_ok = 1;
  }
  for (int q = tid; q < P.R; q += 256) s_tok[q] = checked_token(P.anchor[q], P.V, P.err);

  // unit q of a step -> (chunk, tile slot, row block)
  auto decode = [&](int q, int& c, int& ti, int& rb) {
    const int full = (nch - 1) * ntl * (CH / 32);
    if (q < full) {
      c = q / (ntl * (CH / 32));
      const int rem = q - c * ntl * (CH / 32);
      ti = rem / (CH / 32);
      rb = rem - ti * (CH / 32);
    } else {
      c = nch - 1;
      const int rem = q - full;
      ti = rem / nrb_last;
      rb = rem - ti * nrb_last;
    }
  };
  // base rows of global unit g (step g / ups) into X[g & 1]
  auto issue = [&](int g) {
    if (g >= total) return;
    const int k = g / ups + 1;
    int c, ti, rb;
    decode(g - (k - 1) * ups, c, ti, rb);
    const int c0 = c * CH, nrows = min(CH, P.R - c0);
    const size_t first = (size_t)c0 * P.gamma + (k - 1);
    const rsrc_t brs = make_rsrc(P.base + first * P.V, ((size_t)P.R * P.gamma - first) * P.V * 4);
    stage_dma(brs, row_bytes, rb, nrows, (b + ti * G) * TILE, X[g & 1]);
  };

  // resident W2 fragments of this workgroup's tiles, loaded once.  Most of
  // them live in the accumulation registers (AGPRs), which the MFMAs read
  // their A operand from directly, so the VGPRs stay free for the unit
  // pipeline; the register budget (472 of the 512 per lane, so that a
  // 40-register wave of a kernel on another stream still fits beside every
  // wave of this one) leaves the last two k steps in VGPRs.
  typename BB::template Frag<KS> F0, F1;
  if (ntl > 0) BB::template load<KS>(F0, P.W2, P.V, P.r, b * TILE + wave * WCOLS);
  if (ntl > 1) BB::template load<KS>(F1, P.W2, P.V, P.r, (b + G) * TILE + wave * WCOLS);
  issue(0);
  issue(1);
  if (ntl > 0) BB::template to_operands<KS>(F0);
  if (ntl > 1) BB::template to_operands<KS>(F1);
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
#pragma unroll
    for (int e = 0; e < 8; e++)
      if (ks < 14) asm volatile("" : "+a"(F0.w[ks][e]), "+a"(F1.w[ks][e]));
  __syncthreads();
  const uint32_t E = s_E;

  const float sc = t_one ? LOG2E_F : LOG2E_F * P.invT;
  const double invTd = t_one ? 1.0 : 1.0 / (double)P.T;
  const rsrc_t rec_rs = make_rsrc(P.frec, (size_t)P.R * nt * FREC_BYTES);
  bool ok = true;

  // One unit (tile slot ti, row block rb of chunk c) of step k at a time,
  // software-pipelined: the MFMA chain of the next unit runs interleaved with
  // the epilogue of the current one (unit_block); the base rows of a unit
  // arrive by direct-to-LDS loads issued two units ahead.
  auto records = [&](int k, int c0, int nrows, int tile) {
    // tile records of this chunk: two sealed 16-byte words per request,
    // stored device-coherent (written through to memory); the word w of
    // request q is stored by thread q + 128 w (greedy: one word, by
    // threads q < nrows), so the stores are spread over the four waves
    const int nwords = GREEDY ? 1 : 2;
    if (tid < nwords * CH && (tid & (CH - 1)) < nrows) {
      const int q = tid & (CH - 1), word = tid / CH;
      const uint32_t tag = E + (uint32_t)k;
      const uint32_t roff = (uint32_t)(((size_t)(c0 + q) * nt + tile) * FREC_BYTES);
      uint32_t x0, x1, x2, y0 = 0u, y1 = 0u, y2 = 0u;
      if (GREEDY) {
        float v = red_m[0][q];
        int i = red_i[0][q];
#pragma unroll
        for (int w = 1; w < 4; w++) argmax_merge(v, i, red_m[w][q], red_i[w][q]);
        x0 = __float_as_uint(v);
        x1 = (uint32_t)i;
        x2 = 0u;
      } else {
        const float m0 = red_m[0][q], m1 = red_m[1][q], m2 = red_m[2][q], m3 = red_m[3][q];
        const float mt = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
        auto rescale = [&](float swv, float mwv) {
          const float d = t_one ? (mwv - mt) : (mwv - mt) * P.invT;
          return (mwv == -INFINITY) ? 0.f : swv * exp_acc(d);
        };
        const float s0 = rescale(red_s[0][q], m0), s1 = rescale(red_s[1][q], m1);
        const float s2 = rescale(red_s[2][q], m2), s3 = rescale(red_s[3][q], m3);
        const float st = (s0 + s1) + (s2 + s3);
        x0 = __float_as_uint(mt);
        x1 = __float_as_uint(st);
        x2 = __float_as_uint(s0);
        y0 = __float_as_uint(s1);
        y1 = __float_as_uint(s2);
        y2 = __float_as_uint(s3);
        if (word == 0 && (is_bad(st) || !(mt == mt) || mt == INFINITY)) raise_err(P.err, DSPARK_DERR_NONFINITE);
      }
      if (word == 0)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{x0, x1, x2, seal(tag, x0, x1, x2)}, rec_rs, (int)roff, 0,
                                               AUX_DEV);
      else
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{y0, y1, y2, seal(tag, y0, y1, y2)}, rec_rs,
                                               (int)roff + 16, 0, AUX_DEV);
    }
  };
  // direct-to-LDS rows of global unit g (into X[g & 1]), issued one row
  // piece per part of a unit block; off when g is past the step
  auto dma_plan = [&](int g, int step_end) {
    DmaPlan d;
    const bool on = g < step_end;
    d.on = on;
    const int gg = on ? g : 0;
    const int k = gg / ups + 1;
    int c, ti, rb;
    decode(gg - (k - 1) * ups, c, ti, rb);
    const int c0 = c * CH;
    d.nrows = min(CH, P.R - c0);
    d.rb = rb;
    d.row_bytes = row_bytes;
    const size_t first = (size_t)c0 * P.gamma + (k - 1);
    d.rs = make_rsrc(P.base + first * P.V, ((size_t)P.R * P.gamma - first) * P.V * 4);
    d.coff = (uint32_t)((b + ti * G) * TILE + 4 * lane) * 4u;
    d.X = X[g & 1];
    return d;
  };

  for (int k = 1; k <= P.gamma && ok; k++) {
    int g = (k - 1) * ups;
    const int step_end = k * ups;
    for (int c = 0; c < nch && ntl > 0; c++) {
      const int c0 = c * CH, nrows = min(CH, P.R - c0), nrb = ceil_div(nrows, 32);
      const int n_u = ntl * nrb;  // units of this chunk: tile-major, then row block
      lds_barrier();  // the previous chunk is done with A_lds and red_*
      {
        // W1 rows of the chunk's tokens (r = 16 KS: 2 KS pieces of 16 bytes per
        // row), recomputing every per-thread index here: an opaque thread id
        // keeps them from living in registers across the whole step loop
        constexpr int PIECES = 2 * KS;
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const rsrc_t w1rs = make_rsrc(P.W1, (size_t)P.V * P.r * 2);
        u32x4 wv[GPER];
#pragma unroll
        for (int i = 0; i < GPER; i++) {
          const int idx = t + 256 * i, row = idx / PIECES, pc = idx % PIECES;
          const int tk = (row < nrows) ? s_tok[c0 + row] : -1;
          const u32x4 x = buf_u32x4<0>(w1rs, (uint32_t)(max(tk, 0) * P.r + pc * 8) * 2u, 0u);
          wv[i] = (tk >= 0) ? x : u32x4{0u, 0u, 0u, 0u};
        }
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int i = 0; i < GPER; i++) {
          const int idx = t + 256 * i, row = idx / PIECES, pc = idx % PIECES;
          *reinterpret_cast<u32x4*>(A_lds + row * a_stride + pc * 8) = wv[i];
        }
      }
      lds_barrier();  // A_lds complete
      f32x16 accA[2], accB[2];
      // the chunk's first MFMA chain (unit 0: tile slot 0, row block 0), alone
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int t = 0; t < 16; t++) accA[p][t] = 0.f;
      mma_resident<KS>(F0, A_lds, a_stride, accA);
      auto iter = [&](auto& accC, auto& accN, int u) {
        const int ti = u / nrb, rb = u - ti * nrb;
        const int tile = b + ti * G;
        const int cbase = tile * TILE + wave * WCOLS;
        // unit g's rows were issued two units earlier, so the next unit's 8
        // loads may still be in flight behind them, unless the next unit is
        // of the next step (issued after the draws)
        if (g + 1 < step_end)
          wait_vmcnt<8>();
        else
          wait_vmcnt<0>();
        lds_barrier();
        float bv2[2][16];
        if ((tile + 1) * TILE <= P.V)
          stage_read_full(X[g & 1], wave * WCOLS, bv2);
        else
          stage_read(X[g & 1], true, P.V, cbase, wave * WCOLS, bv2);
        lds_barrier();  // every wave has its base values out of X[g & 1]
        const DmaPlan dp = dma_plan(g + 2, step_end);
        const int rl = rb * 32 + j;
        const UnitOut o{red_m, red_s, red_i, wave, rl, P.err};
        if (u + 1 < n_u) {
          const int tn = (u + 1) / nrb, rbn = (u + 1) - tn * nrb;
          if (tn == 0)
            unit_block<KS, GREEDY, true>(F0, A_lds + rbn * 32 * a_stride, a_stride, accN, accC, bv2, sc, cbase,
                                         dp, o);
          else
            unit_block<KS, GREEDY, true>(F1, A_lds + rbn * 32 * a_stride, a_stride, accN, accC, bv2, sc, cbase,
                                         dp, o);
        } else {
          unit_block<KS, GREEDY, false>(F0, A_lds, a_stride, accN, accC, bv2, sc, cbase, dp, o);
        }
        if (rb == nrb - 1) {
          lds_barrier();  // red_* of the tile's units complete
          records(k, c0, nrows, tile);
        }
        g++;
      };
      for (int u = 0; u < n_u;) {
        iter(accA, accB, u++);
        if (u >= n_u) break;
        iter(accB, accA, u++);
      }
    }

    // draws of the requests this workgroup serves: the request's records from
    // every workgroup, polled until every word carries this step's seal
    for (int row = b; row < P.R && ok; row += G) {
      const size_t ev = (size_t)row * P.gamma + (k - 1);
      const int prev = s_tok[row];
      const uint32_t want = E + (uint32_t)k;
      const rsrc_t rrs = make_rsrc(P.frec + (size_t)row * nt * (FREC_BYTES / 4), (size_t)nt * FREC_BYTES);
      float u = 0.f;
      if (!GREEDY) {  // independent of the records: in flight with them
        for (int i = tid; i < P.r; i += 256) w1s[i] = to_f32(P.W1[(size_t)prev * P.r + i]);
        u = checked_uniform(P.u_draft[ev], P.err);
      }
      int t0, t1;
      block_tile_range(nt, t0, t1);
      // all words of the thread's tiles are loaded before any is checked (one
      // memory round trip per poll); a poll that finds a stale word loads
      // them all again
      u32x4 wa[FUSED_TPL], wb[FUSED_TPL];
      bool timed_out = false;
      while (true) {
#pragma unroll
        for (int i = 0; i < FUSED_TPL; i++) {
          const uint32_t off = (uint32_t)min(t0 + i, nt - 1) * (uint32_t)FREC_BYTES;
          wa[i] = buf_u32x4<AUX_DEV>(rrs, off, 0u);
          if (!GREEDY) wb[i] = buf_u32x4<AUX_DEV>(rrs, off + 16u, 0u);
        }
        bool have = true;
#pragma unroll
        for (int i = 0; i < FUSED_TPL; i++) {
          if (t0 + i < t1) {
            have = have && wa[i][3] == seal(want, wa[i][0], wa[i][1], wa[i][2]);
            if (!GREEDY) have = have && wb[i][3] == seal(want, wb[i][0], wb[i][1], wb[i][2]);
          }
        }
        if (have) break;
        if (__builtin_amdgcn_s_memrealtime() > deadline) { timed_out = true; break; }
      }
      if (timed_out) {
        s_ok = 0;
        raise_err(P.err, DSPARK_DERR_SYNC);
      }
      float m[FUSED_TPL], s[FUSED_TPL];
      float4 sw[FUSED_TPL];
#pragma unroll
      for (int i = 0; i < FUSED_TPL; i++) {
        const bool mine = t0 + i < t1;
        m[i] = mine ? __uint_as_float(wa[i][0]) : -INFINITY;
        s[i] = mine ? (GREEDY ? __int_as_float((int)wa[i][1]) : __uint_as_float(wa[i][1])) : 0.f;
        sw[i] = (mine && !GREEDY) ? make_float4(__uint_as_float(wa[i][2]), __uint_as_float(wb[i][0]),
                                                __uint_as_float(wb[i][1]), __uint_as_float(wb[i][2]))
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      lds_barrier();  // w1s, s_ok
      ok = s_ok != 0;
      if (!ok) break;
      int x;
      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < FUSED_TPL; i++)
          if (t0 + i < t1) argmax_merge(bv, bi, m[i], __float_as_int(s[i]));
        wave_argmax(bv, bi);
        if (lane == 0) { gm[wave] = bv; gi[wave] = bi; }
        __syncthreads();
        if (tid == 0) {
          for (int w = 1; w < 4; w++) argmax_merge(bv, bi, gm[w], gi[w]);
          x = bi;
          if (x < 0 || x >= P.V) x = 0;  // only with non-finite logits (flagged)
          P.tokens[ev] = x;
          P.probs[ev] = 1.0f;
          P.stats[2 * ev] = bv;
          P.stats[2 * ev + 1] = 1.0f;
          st_dev64(P.tokw + row, ((uint64_t)(E + (uint32_t)k) << 32) | (uint32_t)x);
        }
      } else {
        const TilePick S = block_select_tile_vals<FUSED_TPL>(m, s, sw, nt, true, invTd, (double)u, sm);
        const int cb = S.t * TILE + S.w * WCOLS;
        const int col = cb + lane;
        float bval = 0.f;
        if (wave == 0) bval = (col < P.V) ? P.base[ev * P.V + col] : -INFINITY;
        const float bias = chunk_bias<WT, KS>(P.W2, P.V, P.r, cb, w1s, part);
        if (wave == 0) {
          const float ec = exp2_scaled((bval - S.mt) + bias, sc);
          const int cpos = wave_pick64(ec, S.scale, S.rem);
          const float ex = __shfl(ec, cpos);
          if (lane == 0) {
            x = min(cb + cpos, P.V - 1);
            P.tokens[ev] = x;
            P.probs[ev] = (float)((double)ex * S.scale / S.Z);
            P.stats[2 * ev] = S.M;
            P.stats[2 * ev + 1] = (float)S.Z;
            if (!(S.Z > 0.0) || is_bad(S.M)) raise_err(P.err, DSPARK_DERR_NONFINITE);
            st_dev64(P.tokw + row, ((uint64_t)(E + (uint32_t)k) << 32) | (uint32_t)x);
          }
        }
      }
      __syncthreads();  // select scratch is reused by the next request
    }

    // the next step's first base rows, issued after the draws: a load that
    // returns to registers waits for every earlier load of its wave,
    // direct-to-LDS ones included, and the draws' loads are on the critical
    // path (the token polls below wait for the slowest draw anyway)
    if (k < P.gamma) {
      issue(k * ups);
      issue(k * ups + 1);
    }

    // tokens x_k of every request, for the next step's W1 gather
    if (k < P.gamma && ok) {
      const uint32_t want = E + (uint32_t)k;
      bool timed_out = false;
      for (int q = tid; q < P.R; q += 256) {
        uint64_t v;
        while (true) {
          v = ld_dev64(P.tokw + q);
          if ((uint32_t)(v >> 32) == want) break;
          if (__builtin_amdgcn_s_memrealtime() > deadline) { timed_out = true; break; }
        }
        if (timed_out) break;
        s_tok[q] = checked_token((int)(uint32_t)v, P.V, P.err);
      }
      if (timed_out) {
        s_ok = 0;
        raise_err(P.err, DSPARK_DERR_SYNC);
      }
      lds_barrier();
      ok = s_ok != 0;
    }
  }

  // no direct-to-LDS load may outlive the workgroup
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0) {
    const uint32_t ticket = __hip_atomic_fetch_add(P.done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket == (uint32_t)G - 1) {
      // every workgroup has read the epoch and finished: advance it for the next call
      st_dev(P.done, 0u);
      st_dev(P.epoch, E + (uint32_t)P.gamma);
    }
  }
}

// Occupancy check, once per process and device: the fused launch needs one
// resident workgroup on every compute unit.
template <int KS, bool GREEDY>
static bool fused_fits() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_draft_fused<KS, GREEDY>, 256, 0) != hipSuccess)
    return false;
  return n >= 1;
}

template <int KS>
static bool fused_fits_t(float T) {
  static const bool f_samp = fused_fits<KS, false>();
  static const bool f_greedy = fused_fits<KS, true>();
  return T == 0.f ? f_greedy : f_samp;
}

// Real-time limit of the kernel's waits: FUSED_SPIN_TICKS, or the value of
// DSPARK_FUSED_SPIN_TICKS (read on every call; the tests of the time-out path
// set it to 0, so that every wait that does not succeed at once gives up).
static uint64_t fused_spin_ticks() {
  const char* e = getenv("DSPARK_FUSED_SPIN_TICKS");
  if (e == nullptr || *e == '\0') return FUSED_SPIN_TICKS;
  char* end = nullptr;
  const unsigned long long v = strtoull(e, &end, 10);
  return (end != nullptr && *end == '\0') ? (uint64_t)v : FUSED_SPIN_TICKS;
}

bool draft_fused_supported(int R, int gamma, int V, int r, float T) {
  (void)gamma;
  const int G = device_cu_count();
  if (R > FUSED_MAX_R) return false;
  if (r != 16 * ks_bucket(r)) return false;  // rank 16, 32, 64, 128 or 256
  if (ceil_div(V, TILE) > 2 * G || ceil_div(V, TILE) > FUSED_MAX_NT) return false;
  bool fits = false;
  DSPARK_DISPATCH_KS(r, { fits = fused_fits_t<KS>(T); });
  return fits;
}

int draft_fused_launch(const float* base, const void* W1, const void* W2, const int32_t* anchor,
                       const float* u_draft, int R, int gamma, int V, int r, float T, int32_t* tokens,
                       float* probs, float* stats, const DraftWs& dw, hipStream_t stream) {
  FusedArgs A;
  A.base = base;
  A.W1 = static_cast<const uint16_t*>(W1);
  A.W2 = static_cast<const uint16_t*>(W2);
  A.anchor = anchor;
  A.u_draft = u_draft;
  A.R = R; A.gamma = gamma; A.V = V; A.r = r;
  A.T = T;
  A.invT = (T > 0.f) ? 1.0f / T : 0.f;
  A.tokens = tokens; A.probs = probs; A.stats = stats;
  A.frec = dw.frec;
  A.err = dw.err;
  A.epoch = reinterpret_cast<uint32_t*>(dw.sync + SYNC_EPOCH);
  A.done = reinterpret_cast<uint32_t*>(dw.sync + SYNC_DONE);
  A.tokw = reinterpret_cast<uint64_t*>(dw.sync + SYNC_TOKW);
  A.spin_ticks = fused_spin_ticks();
  const int G = device_cu_count();
  prof_before(DSPARK_KID_DRAFT_FUSED, stream);
  for (int rep = prof_repeat(DSPARK_KID_DRAFT_FUSED); rep > 0; rep--) {
    DSPARK_DISPATCH_KS(r, {
      if (T == 0.f)
        hipLaunchKernelGGL((k_draft_fused<KS, true>), dim3(G), dim3(256), 0, stream, A);
      else
        hipLaunchKernelGGL((k_draft_fused<KS, false>), dim3(G), dim3(256), 0, stream, A);
    });
  }
  prof_after(DSPARK_KID_DRAFT_FUSED, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

}  // namespace dspark
