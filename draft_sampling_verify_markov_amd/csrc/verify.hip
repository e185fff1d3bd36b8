// Lossless rejection-sampling verification (dspark_verify).
//
// Sources: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), "Definição do problema" (the target verifies a drafted
// block in one pass and, by rejection sampling, keeps the longest prefix that
// matches the target distribution, so decoding is lossless) and the decode
// cycle in "Arquitetura" (E and F accepted, G rejected, a corrected token G*
// emitted).  "DSpark: la apuesta de DeepSeek ..." (aitalk.it), first section:
// the output is statistically identical to the target model's.
//
// Kernels, in stream order (no kernel waits on another workgroup):
//   stream    grid = (gamma+1) x R x ceil(V / 8192) (greedy: 4096),
//             position-major.  Streams target rows j = 0..L_r of request r
//             (non-temporal loads) and writes per-1024-column softmax partials;
//             it reads no drafted token, so it can run before or beside the
//             draft.
//   decide    one workgroup per request, one wave per position: fp64 row
//             statistics, the target logit at the drafted token x_{j+1} and
//             p_{j+1}(x_{j+1}), the accept tests u < p/q, and the first
//             rejected position.
//   residual  persistent, one workgroup per compute unit over the 256-column
//             tiles (T > 0 only).  For requests that rejected at k*,
//             recomputes the draft logits of position k* with the MFMA bias
//             block and writes tile records of max(0, p - pi).  Over more
//             than 128 requests with bf16 factors the workgroup keeps its
//             tiles' W2 fragments in registers for the whole call.
//   (dspark_accept_rates reuses the stream and the residual pipeline over
//   every request and position to form c*_k = 1 - |q_k - p_k|_1 / 2.)
//   finalize  one workgroup per request: residual or bonus inverse-CDF sample
//             (fp64 scan over tiles, recompute of one chunk or tile), emitted
//             tokens and the p_k(x_k) output.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "select.h"

namespace dspark {

template <typename WT>
struct VerifyArgs {
  const float* target;
  const float* base;
  const WT* W1;
  const WT* W2;
  const int32_t* anchor;
  const int32_t* dtok;
  const float* dprob;
  const float* dstats;
  const int32_t* vlen;
  const float* u_acc;
  const float* u_fin;
  int R, gamma, V, r;
  float T, invT;
  int32_t* out_tokens;
  int32_t* accept_len;
  float* target_probs;
  double2* rowstat;
  int32_t* rej;
  float2* vpart;
  float* tp;
  float4* rrec;
  float* tvpart;  // [R*gamma][V/256] per-tile sums of max(0, p - q) (acceptance labels)
  int32_t* err;
  // Draft bias rows: W1 by previous token, or (dense) the RNN head's state
  // table of a_rows = R * gamma rows, row r * gamma + k - 1 = s_k of request r.
  bool dense;
  int a_rows;

  __device__ int L_of(int row, bool report = false) const {
    if (!vlen) return gamma;
    const int l = vlen[row];
    if (l < 0 || l > gamma) {
      if (report) raise_err(err, DSPARK_DERR_LENGTH);
      return l < 0 ? 0 : gamma;
    }
    return l;
  }
  // token before position k (1-based) of request row
  __device__ int prev_of(int row, int k) const {
    if (dense) return row * gamma + k - 1;
    const int t = (k == 1) ? anchor[row] : dtok[(size_t)row * gamma + k - 2];
    return checked_token(t, V, err);
  }
};

// fp64 butterfly sum over the wave without LDS shuffles (DPP row moves, then
// the permlane swaps between rows); every lane gets the same bits.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_f64<DPP_QUAD_XOR1>(v);
  v += dpp_f64<DPP_QUAD_XOR2>(v);
  v += dpp_f64<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f64<DPP_ROW_MIRROR>(v);
  auto join = [](uint32_t hi, uint32_t lo) { return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo); };
  const uint64_t b1 = __builtin_bit_cast(uint64_t, v);
  const LanePair h1 = swap16((uint32_t)(b1 >> 32)), l1 = swap16((uint32_t)b1);
  v = join(h1.a, l1.a) + join(h1.b, l1.b);
  const uint64_t b2 = __builtin_bit_cast(uint64_t, v);
  const LanePair h2 = swap32((uint32_t)(b2 >> 32)), l2 = swap32((uint32_t)b2);
  return join(h2.a, l2.a) + join(h2.b, l2.b);
}

// ---------------------------------------------------------------------------
// target-row stream

// One 1024-column tile of a target row already in registers: lane l holds
// columns col0 + f*256 + 4l + e (f, e < 4) in v[4f + e], -inf past V.  Writes
// the tile's partial (max, sum of exp((x - max)/T)) or (max, arg-max).
template <typename WT, bool GREEDY>
__device__ __forceinline__ void stream_tile(const VerifyArgs<WT>& P, size_t rowj, int nvt, int tt,
                                            const float (&v)[16]) {
  const int lane = threadIdx.x & 63;
  const int col0 = tt * VTILE;
  bool bad = false;
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int f = 0; f < 4; f++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float x = v[4 * f + e];
        bad |= (x != x);
        if (x > bv) { bv = x; bi = col0 + f * 256 + lane * 4 + e; }
      }
    wave_argmax(bv, bi);
    if (lane == 0) P.vpart[rowj * nvt + tt] = make_float2(bv, __int_as_float(bi));
  } else {
    const bool t_one = (P.T == 1.0f);
    float m = v[0];
#pragma unroll
    for (int i = 1; i < 16; i++) m = fmaxf(m, v[i]);
    m = wave_max(m);
    // pair sums exp(v_i) + exp(v_{i+8}), the fixed tree's first level folded
    // in as soon as both terms exist
    float s[4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float d0 = t_one ? (v[i] - m) : (v[i] - m) * P.invT;
      const float d1 = t_one ? (v[i + 8] - m) : (v[i + 8] - m) * P.invT;
      const float pr = exp_acc(d0) + exp_acc(d1);
      if (i < 4) s[i] = pr; else s[i - 4] = s[i - 4] + pr;
    }
    s[0] = s[0] + s[2];
    s[1] = s[1] + s[3];
    const float sum = wave_sum(s[0] + s[1]);
    bad = is_bad(sum) || is_bad(m);
    if (lane == 0) P.vpart[rowj * nvt + tt] = make_float2(m, sum);
  }
  if (bad) raise_err(P.err, DSPARK_DERR_NONFINITE);
}

// Target rows 0..L_r in 8192-column segments (greedy: 4096), one workgroup
// per (row j, request, segment), position-major.  Every wave loads two
// adjacent 1024-column tiles before reducing either (two tiles in flight per
// wave), in 40 registers per lane: beside a resident one-launch draft
// workgroup (472 registers per lane) the stream gets one wave per SIMD.  The
// greedy arg-max needs more registers, so there a wave takes one tile (25
// registers).
template <typename WT, bool GREEDY>
__global__ __launch_bounds__(256) void k_verify_stream(VerifyArgs<WT> P) {
  constexpr int TPW = GREEDY ? 1 : 2;  // tiles per wave
  const int nseg = ceil_div(P.V, stream_seg(GREEDY)), nvt = ceil_div(P.V, VTILE);
  const int b = blockIdx.x;
  const int jpos = b / (P.R * nseg);
  const int rem = b - jpos * P.R * nseg;
  const int row = rem / nseg, seg = rem - row * nseg;
  const int L = P.L_of(row);
  if (jpos > L) return;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t rowj = (size_t)row * (P.gamma + 1) + jpos;
  const int tt = (seg * 4 + wave) * TPW;
  if (tt * VTILE >= P.V) return;
  // the row from tile tt on; loads past V read 0 and are replaced by -inf
  const int col0 = tt * VTILE;
  const rsrc_t rs = make_rsrc(P.target + rowj * P.V + col0, (size_t)(P.V - col0) * 4);
  const uint32_t voff = (uint32_t)lane * 16u;
  f32x4 x[TPW][4];
#pragma unroll
  for (int q = 0; q < TPW; q++)
#pragma unroll
    for (int f = 0; f < 4; f++)
      x[q][f] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, q * 4096 + f * 1024, AUX_NT));
#pragma unroll
  for (int q = 0; q < TPW; q++) {
    if (tt + q < nvt) {
      float v[16];
#pragma unroll
      for (int f = 0; f < 4; f++)
#pragma unroll
        for (int e = 0; e < 4; e++)
          v[4 * f + e] = (col0 + q * VTILE + f * 256 + lane * 4 + e < P.V) ? x[q][f][e] : -INFINITY;
      stream_tile<WT, GREEDY>(P, rowj, nvt, tt + q, v);
    }
  }
}

// ---------------------------------------------------------------------------
// accept tests: one workgroup per request, one wave per position

// Waves per decide workgroup: one per target row j = 0..gamma, at most 16.
__host__ __device__ constexpr int decide_waves(int gamma) { return gamma + 1 < 16 ? gamma + 1 : 16; }

// Every load a position needs is issued before any result is used: the verify
// length, the drafted token x_{j+1} and, as soon as it arrives, the target
// logit at it, the row's tile partials, q and u.  Positions past L are
// computed on whatever the buffers hold and discarded.
template <typename WT, bool GREEDY>
__global__ __launch_bounds__(1024) void k_verify_decide(VerifyArgs<WT> P) {
  __shared__ int s_ok[DSPARK_MAX_GAMMA + 1];
  const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nw = decide_waves(P.gamma);
  const int nvt = ceil_div(P.V, VTILE);
  const int L = P.L_of(row, tid == 0);
  const bool t_one = (P.T == 1.0f);
  const double invTd = t_one ? 1.0 : 1.0 / (double)P.T;

  for (int j = wave; j <= P.gamma; j += nw) {
    const size_t rowj = (size_t)row * (P.gamma + 1) + j;
    const float2* vp = P.vpart + rowj * nvt;
    const size_t ev = (size_t)row * P.gamma + j;
    const bool drafted = j < P.gamma;
    // lane 0: the drafted token and the target logit at it
    int x = 0;
    float tx = 0.f, q = 1.f, u = 0.f;
    if (lane == 0 && drafted) {
      x = P.dtok[ev];
      q = P.dprob[ev];
      if (!GREEDY) u = P.u_acc[ev];
      if (!GREEDY && x >= 0 && x < P.V) tx = P.target[rowj * P.V + x];
    }
    if (GREEDY) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int t = lane; t < nvt; t += 64) argmax_merge(bv, bi, vp[t].x, __float_as_int(vp[t].y));
      wave_argmax(bv, bi);
      if (lane == 0 && j <= L) {
        P.rowstat[rowj] = make_double2((double)bv, (double)bi);
        if (j < L) {
          const bool ok = (checked_token(x, P.V, P.err) == bi);
          P.tp[ev] = ok ? 1.0f : 0.0f;
          s_ok[j] = ok;
        }
      }
    } else {
      float ml = -INFINITY;
      for (int t = lane; t < nvt; t += 64) ml = fmaxf(ml, vp[t].x);
      const float M = wave_max(ml);
      double zl = 0.0;
      for (int t = lane; t < nvt; t += 64)
        zl += (double)vp[t].y * (double)exp_acc((vp[t].x - M) * (float)invTd);
      const double Z = wave_sum_d(zl);
      if (lane == 0 && j <= L) {
        P.rowstat[rowj] = make_double2((double)M, Z);
        if (j < L) {
          // the target logit at the drafted token is read here (not by the
          // row stream), so the stream does not depend on the draft
          checked_token(x, P.V, P.err);
          const double p = exp(((double)tx - (double)M) * invTd) / Z;
          bool ok;
          if (!(q > 0.f)) {
            raise_err(P.err, DSPARK_DERR_PROB);
            ok = false;
          } else {
            ok = (double)checked_uniform(u, P.err) < p / (double)q;
          }
          P.tp[ev] = (float)p;
          s_ok[j] = ok;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int ks = NO_REJECT;
    for (int j = 0; j < L; j++)
      if (!s_ok[j]) { ks = j + 1; break; }
    P.rej[row] = ks;
  }
}

// ---------------------------------------------------------------------------
// residual max(0, p - pi) tile records for rejected requests

// max(0, p - pi) of one column: p = 2^((t - Mt) sc) / Zt from the target
// logit, pi = 2^(((b - m_q) + bias) sc) / Zq from the recomputed draft logit,
// sc = log2(e) / T.  -inf logits (masked or past V) give 0.
__device__ __forceinline__ float residual_elem(float t, float b, float bias, float Mt, float invZt, float mq,
                                               float invZq, float sc) {
  const float pv = exp2_scaled(t - Mt, sc) * invZt;
  const float qv = exp2_scaled((b - mq) + bias, sc) * invZq;
  return fmaxf(0.f, pv - qv);
}

// Persistent over column tiles like the draft partials kernel.  Per chunk of
// 128 consecutive requests the rejected ones are compacted; their W1 rows at
// k* are gathered into LDS once, and the work is cut into units (tile, block
// of 32 rejected requests).  A unit's base and target rows at k* arrive in LDS
// by direct-to-LDS loads issued one unit ahead (they overlap the unit's MFMA
// chain), the epilogue forms max(0, p - pi) and per-wave sums, and the tile's
// last unit writes the residual tile records.
// TVM (acceptance labels): the items are every (request, position k) pair,
// k = 1..gamma, in chunks of CH consecutive flat indices r*gamma + k-1, and
// each (item, tile) writes the tile's sum of max(0, p - q) to tvpart.
template <typename WT, int KS, bool TVM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_residual_partials(
    VerifyArgs<WT> P) {
  constexpr int APAD = BiasBlock<WT>::APAD;
  constexpr int CH = sizeof(WT) == 2 ? 128 : 64;
  constexpr int EPV = 16 / sizeof(WT);
  constexpr int GPER = CH * (KS * 16 / EPV) / 256;
  __shared__ __align__(16) WT A_lds[CH * (DSPARK_MAX_RANK + APAD)];
  __shared__ __align__(16) float Xb[32 * BSTRIDE];
  __shared__ __align__(16) float Xt[32 * BSTRIDE];
  __shared__ float red_s[4][CH];
  __shared__ int s_list[CH], s_tok[CH], s_cnt[2];
  __shared__ uint32_t s_boff[CH], s_toff[CH];
  __shared__ float s_Mt[CH], s_iZt[CH], s_mq[CH], s_iZq[CH];

  const int a_stride = P.r + APAD;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31;
  const int nt = ceil_div(P.V, TILE);
  const int G = gridDim.x;
  if ((int)blockIdx.x >= nt) return;
  const int my_tiles = (nt - (int)blockIdx.x + G - 1) / G;
  const float sc = (P.T == 1.0f) ? LOG2E_F : LOG2E_F * P.invT;

  const int nitems = TVM ? P.R * P.gamma : P.R;
  for (int c0 = 0; c0 < nitems; c0 += CH) {
    // request whose rows anchor the buffer resources of this chunk
    const int r0 = TVM ? c0 / P.gamma : c0;
    int nrej;
    __syncthreads();  // the previous chunk is done with every LDS array
    if (TVM) {
      nrej = min(CH, nitems - c0);
    } else {
      // compaction of the chunk's rejected requests (order kept)
      const int nrows = min(CH, P.R - c0);
      bool mine = false;
      if (tid < nrows) mine = P.rej[c0 + tid] <= P.L_of(c0 + tid);
      const uint64_t bal = __ballot(mine);
      if (tid < CH && lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      nrej = (CH > 64 ? s_cnt[0] + s_cnt[1] : s_cnt[0]);
      if (nrej == 0) continue;  // uniform
      if (mine) {
        const int pos = (wave == 1 ? s_cnt[0] : 0) + __popcll(bal & ((1ull << lane) - 1ull));
        s_list[pos] = tid;
      }
      __syncthreads();
    }
    if (tid < nrej) {
      int row, ks;  // request and 1-based position of the item
      if (TVM) {
        const int item = c0 + tid;
        row = item / P.gamma;
        ks = item - row * P.gamma + 1;
        s_list[tid] = tid;
      } else {
        row = c0 + s_list[tid];
        ks = P.rej[row];  // k*
      }
      const double2 rs = P.rowstat[(size_t)row * (P.gamma + 1) + ks - 1];
      const size_t ev = (size_t)row * P.gamma + ks - 1;
      s_Mt[tid] = (float)rs.x;
      s_iZt[tid] = (float)(1.0 / rs.y);
      s_mq[tid] = P.dstats[2 * ev];
      s_iZq[tid] = (float)(1.0 / (double)P.dstats[2 * ev + 1]);
      const uint32_t rl = (uint32_t)(row - r0);
      s_boff[tid] = (rl * (uint32_t)P.gamma + (uint32_t)(ks - 1)) * (uint32_t)P.V * 4u;
      s_toff[tid] = (rl * (uint32_t)(P.gamma + 1) + (uint32_t)(ks - 1)) * (uint32_t)P.V * 4u;
      s_tok[tid] = P.prev_of(row, ks);
    }
    __syncthreads();

    const int nrb = ceil_div(nrej, 32);
    const int nunits = my_tiles * nrb;
    const size_t R_left = (size_t)(P.R - r0);
    const rsrc_t brs = make_rsrc(P.base + (size_t)r0 * P.gamma * P.V, R_left * P.gamma * P.V * 4);
    const rsrc_t trs = make_rsrc(P.target + (size_t)r0 * (P.gamma + 1) * P.V, R_left * (P.gamma + 1) * P.V * 4);
    // unit u's rows: wave w loads compacted rows 4i + w of the block (8 base,
    // 8 target loads per wave).  Rows past nrej are not loaded: their staged
    // values are stale, and the sums formed from them are never read.
    auto issue = [&](int u) {
      if (u >= nunits) return;
      const int ti = u / nrb, rb = u - ti * nrb;
      const int tile0 = ((int)blockIdx.x + ti * G) * TILE;
      const int w = __builtin_amdgcn_readfirstlane(wave);
      const uint32_t coff = (uint32_t)(tile0 + 4 * lane) * 4u;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int q = rb * 32 + 4 * i + w;
        if (q >= nrej) break;  // wave-uniform; the waits below are for all loads
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            brs, (__attribute__((address_space(3))) void*)(Xb + (4 * i + w) * BSTRIDE), 16,
            (int)(s_boff[q] + coff), 0, 0, AUX_NT);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            trs, (__attribute__((address_space(3))) void*)(Xt + (4 * i + w) * BSTRIDE), 16,
            (int)(s_toff[q] + coff), 0, 0, AUX_NT);
      }
    };

    W1Gather<WT, GPER> g;
    g.load(P.W1, P.a_rows, P.r, nrej, CH, a_stride, [&](int i) { return s_tok[i]; });
    issue(0);
    typename BiasBlock<WT>::template Frag<KS> F;
    BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, (int)blockIdx.x * TILE + wave * WCOLS);
    g.store(A_lds);
    lds_barrier();  // A_lds complete; the base/target rows and W2 stay in flight

    int u = 0;
    for (int ti = 0; ti < my_tiles; ti++) {
      const int tile = (int)blockIdx.x + ti * G;
      const int cbase = tile * TILE + wave * WCOLS;
      BiasBlock<WT>::template to_operands<KS>(F);
      for (int rb = 0; rb < nrb; rb++, u++) {
        f32x16 acc[2];
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int t = 0; t < 16; t++) acc[p][t] = 0.f;
        BiasBlock<WT>::template mma_rb_op<KS>(F, P.r, A_lds + rb * 32 * a_stride, a_stride, acc);
        wait_vmcnt<0>();  // this unit's rows (the only loads in flight)
        lds_barrier();
        if (rb == nrb - 1 && tile + G < nt)
          BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, (tile + G) * TILE + wave * WCOLS);
        const int q = rb * 32 + j;
        float b[2][16], t[2][16];
        if ((tile + 1) * TILE <= P.V) {
          stage_read_full(Xb, wave * WCOLS, b);
          stage_read_full(Xt, wave * WCOLS, t);
        } else {
          stage_read(Xb, true, P.V, cbase, wave * WCOLS, b);
          stage_read(Xt, true, P.V, cbase, wave * WCOLS, t);
        }
        const int qc = q < nrej ? q : 0;
        const float Mt = s_Mt[qc], iZt = s_iZt[qc], mq = s_mq[qc], iZq = s_iZq[qc];
        // every wave has its rows out of Xb / Xt: the next unit's rows are
        // loaded while this unit's residual is formed
        lds_barrier();
        issue(u + 1);
        float d[2][16];
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int i = 0; i < 16; i++) d[p][i] = residual_elem(t[p][i], b[p][i], acc[p][i], Mt, iZt, mq, iZq, sc);
        const float sl = tree_sum32(d);
        const float sw = sum_xor32(sl);
        if ((lane >> 5) == 0) red_s[wave][q] = sw;
        if (rb == nrb - 1) lds_barrier();  // red_s of the tile's units complete
        if (rb == nrb - 1 && tid < nrej) {
          const float s0 = red_s[0][tid], s1 = red_s[1][tid], s2 = red_s[2][tid], s3 = red_s[3][tid];
          if (TVM) {
            P.tvpart[(size_t)(c0 + tid) * nt + tile] = (s0 + s1) + (s2 + s3);
          } else {
            float4* rec = P.rrec + ((size_t)(c0 + s_list[tid]) * nt + tile) * 2;
            rec[0] = make_float4(0.f, (s0 + s1) + (s2 + s3), s0, s1);
            rec[1] = make_float4(s2, s3, 0.f, 0.f);
          }
        }
      }
    }
  }
}

// Acceptance-label pass with bf16 factors and at most two tiles per
// workgroup: the W2 fragments of both tiles stay in registers for the whole
// launch, so W2 is read from memory once per call instead of once per chunk
// of items (k_residual_partials reloads a tile's fragment for every chunk).
// Chunks of 96 items (the LDS then holds two base-row buffers and one
// target-row buffer); units are taken row block first, tile second.  A unit's
// base rows arrive by direct-to-LDS loads two units ahead, its target rows
// one unit ahead; a unit's records are written after the next unit's first
// barrier.  Same per-element arithmetic and sums as k_residual_partials.  Also
// verify's residual when more than 128 requests would make the per-tile kernel
// reload W2 for each chunk (R = 512, gamma = 16, V = 131072: 1.573 -> 1.558 ms
// per round); for a single chunk of at most 128 requests, loading both tiles'
// fragments up front measured slower than the per-tile kernel.
template <int KS>
__device__ __forceinline__ void mma_rows(const typename BiasBlock<uint16_t>::template Frag<KS>& F, int r,
                                         const uint16_t* A_rows, int a_stride, f32x16 (&acc)[2]) {
  const int lane = threadIdx.x & 63, j = lane & 31, h = lane >> 5;
  const int nks = r / 16;
  const uint16_t* ap = A_rows + j * a_stride + 8 * h;
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    if (ks < nks) {
      const bf16x8 bb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ap + ks * 16));
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][0], F.w[ks][1], F.w[ks][2], F.w[ks][3]});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{F.w[ks][4], F.w[ks][5], F.w[ks][6], F.w[ks][7]});
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bb, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bb, acc[1], 0, 0, 0);
    }
  }
}

template <int KS, bool TVM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_residual_resident(
    VerifyArgs<uint16_t> P) {
  using WT = uint16_t;
  using BB = BiasBlock<WT>;
  constexpr int APAD = BB::APAD;
  constexpr int CH = 96;
  __shared__ __align__(16) WT A_lds[CH * (DSPARK_MAX_RANK + APAD)];
  __shared__ __align__(16) float Xb[2][32 * BSTRIDE];
  __shared__ __align__(16) float Xt[32 * BSTRIDE];
  __shared__ float red_s[2][4][32];
  __shared__ int s_list[CH], s_tok[CH], s_cnt[2];
  __shared__ uint32_t s_boff[CH], s_toff[CH];
  __shared__ float s_Mt[CH], s_iZt[CH], s_mq[CH], s_iZq[CH];

  const int a_stride = P.r + APAD;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, h = lane >> 5;
  const int nt = ceil_div(P.V, TILE);
  const int G = gridDim.x, b = blockIdx.x;
  if (b >= nt) return;
  const int ntl = (b + G < nt) ? 2 : 1;
  const float sc = (P.T == 1.0f) ? LOG2E_F : LOG2E_F * P.invT;

  // the fragments, in MFMA operand form, held in the accumulation registers
  // (AGPRs, which the MFMAs read their A operand from); the MFMA results go to
  // VGPRs (this file is built with -amdgpu-mfma-vgpr-form)
  typename BB::template Frag<KS> F0, F1;
  BB::template load<KS>(F0, P.W2, P.V, P.r, b * TILE + wave * WCOLS);
  if (ntl > 1) BB::template load<KS>(F1, P.W2, P.V, P.r, (b + G) * TILE + wave * WCOLS);
  BB::template to_operands<KS>(F0);
  if (ntl > 1) BB::template to_operands<KS>(F1);
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
#pragma unroll
    for (int e = 0; e < 8; e++) asm volatile("" : "+a"(F0.w[ks][e]), "+a"(F1.w[ks][e]));

  const int nitems = TVM ? P.R * P.gamma : P.R;
  for (int c0 = 0; c0 < nitems; c0 += CH) {
    const int r0 = TVM ? c0 / P.gamma : c0;
    int nrej;
    __syncthreads();  // the previous chunk is done with every LDS array
    if (TVM) {
      nrej = min(CH, nitems - c0);
    } else {
      // compaction of the chunk's rejected requests (order kept)
      const int nrows = min(CH, P.R - c0);
      bool mine = false;
      if (tid < nrows) mine = P.rej[c0 + tid] <= P.L_of(c0 + tid);
      const uint64_t bal = __ballot(mine);
      if (tid < CH && lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      nrej = s_cnt[0] + s_cnt[1];
      if (nrej == 0) continue;  // uniform
      if (mine) {
        const int pos = (wave == 1 ? s_cnt[0] : 0) + __popcll(bal & ((1ull << lane) - 1ull));
        s_list[pos] = tid;
      }
      __syncthreads();
    }
    if (tid < nrej) {
      int row, ks;  // request and 1-based position of the item
      if (TVM) {
        const int item = c0 + tid;
        row = item / P.gamma;
        ks = item - row * P.gamma + 1;
        s_list[tid] = tid;
      } else {
        row = c0 + s_list[tid];
        ks = P.rej[row];  // k*
      }
      const double2 rs = P.rowstat[(size_t)row * (P.gamma + 1) + ks - 1];
      const size_t ev = (size_t)row * P.gamma + ks - 1;
      s_Mt[tid] = (float)rs.x;
      s_iZt[tid] = (float)(1.0 / rs.y);
      s_mq[tid] = P.dstats[2 * ev];
      s_iZq[tid] = (float)(1.0 / (double)P.dstats[2 * ev + 1]);
      const uint32_t rl = (uint32_t)(row - r0);
      s_boff[tid] = (rl * (uint32_t)P.gamma + (uint32_t)(ks - 1)) * (uint32_t)P.V * 4u;
      s_toff[tid] = (rl * (uint32_t)(P.gamma + 1) + (uint32_t)(ks - 1)) * (uint32_t)P.V * 4u;
      s_tok[tid] = P.prev_of(row, ks);
    }
    __syncthreads();

    const int nrb = ceil_div(nrej, 32);
    const int nunits = nrb * ntl;
    const size_t R_left = (size_t)(P.R - r0);
    const rsrc_t brs = make_rsrc(P.base + (size_t)r0 * P.gamma * P.V, R_left * P.gamma * P.V * 4);
    const rsrc_t trs = make_rsrc(P.target + (size_t)r0 * (P.gamma + 1) * P.V, R_left * (P.gamma + 1) * P.V * 4);
    // base rows of unit u: wave w loads compacted rows 4i + w of the block
    // (8 loads per wave; rows past nrej re-read row 0)
    auto issue_b = [&](int u) {
      if (u >= nunits) return;
      const int rb = u / ntl, ti = u - rb * ntl;
      const int tile0 = (b + ti * G) * TILE;
      const int w = __builtin_amdgcn_readfirstlane(wave);
      const uint32_t coff = (uint32_t)(tile0 + 4 * lane) * 4u;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int q = rb * 32 + 4 * i + w;
        const int qc = q < nrej ? q : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            brs, (__attribute__((address_space(3))) void*)(Xb[u & 1] + (4 * i + w) * BSTRIDE), 16,
            (int)(s_boff[qc] + coff), 0, 0, AUX_NT);
      }
    };
    // target rows of unit u into Xt (one buffer: issued once the previous
    // unit has read it)
    auto issue_t = [&](int u) {
      if (u >= nunits) return;
      const int rb = u / ntl, ti = u - rb * ntl;
      const int tile0 = (b + ti * G) * TILE;
      const int w = __builtin_amdgcn_readfirstlane(wave);
      const uint32_t coff = (uint32_t)(tile0 + 4 * lane) * 4u;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int q = rb * 32 + 4 * i + w;
        const int qc = q < nrej ? q : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            trs, (__attribute__((address_space(3))) void*)(Xt + (4 * i + w) * BSTRIDE), 16,
            (int)(s_toff[qc] + coff), 0, 0, AUX_NT);
      }
    };
    // records of unit u (its 32 rows, its tile) from the four waves' sums
    auto records = [&](int u) {
      const int rb = u / ntl, ti = u - rb * ntl;
      const int tile = b + ti * G;
      const int q = rb * 32 + tid;
      if (tid < 32 && q < nrej) {
        const float s0 = red_s[u & 1][0][tid], s1 = red_s[u & 1][1][tid];
        const float s2 = red_s[u & 1][2][tid], s3 = red_s[u & 1][3][tid];
        if (TVM) {
          P.tvpart[(size_t)(c0 + q) * nt + tile] = (s0 + s1) + (s2 + s3);
        } else {
          float4* rec = P.rrec + ((size_t)(c0 + s_list[q]) * nt + tile) * 2;
          rec[0] = make_float4(0.f, (s0 + s1) + (s2 + s3), s0, s1);
          rec[1] = make_float4(s2, s3, 0.f, 0.f);
        }
      }
    };

    // W1 rows of the chunk's items straight to LDS: one 16-byte piece per
    // lane, one row per load (r / 8 lanes), wave w takes items w, w + 4, ...
    {
      const rsrc_t wrs = make_rsrc(P.W1, (size_t)P.a_rows * P.r * 2);
      const int w = __builtin_amdgcn_readfirstlane(wave);
      for (int i = w; i < nrej; i += 4) {
        const int tk = __builtin_amdgcn_readfirstlane(s_tok[i]);
        if (8 * lane < P.r)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              wrs, (__attribute__((address_space(3))) void*)(A_lds + i * a_stride), 16,
              (int)((uint32_t)(tk * P.r + 8 * lane) * 2u), 0, 0, 0);
      }
    }
    issue_b(0);
    issue_t(0);
    issue_b(1);
    // the W1 rows (issued before unit 0's and unit 1's loads) have landed
    if (nunits > 1)
      wait_vmcnt<24>();
    else
      wait_vmcnt<16>();
    lds_barrier();  // A_lds complete; unit 0's and unit 1's rows in flight

    auto unit = [&](int u) {
      const int rb = u / ntl, ti = u - rb * ntl;
      const int tile = b + ti * G, cbase = tile * TILE + wave * WCOLS;
      f32x16 acc[2];
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int t = 0; t < 16; t++) acc[p][t] = 0.f;
      if (ti == 0)
        mma_rows<KS>(F0, P.r, A_lds + rb * 32 * a_stride, a_stride, acc);
      else
        mma_rows<KS>(F1, P.r, A_lds + rb * 32 * a_stride, a_stride, acc);
      // this unit's base rows and target values; the next unit's base rows
      // (8 loads, issued after them) may stay in flight
      if (u + 1 < nunits)
        wait_vmcnt<8>();
      else
        wait_vmcnt<0>();
      lds_barrier();
      if (u > 0) records(u - 1);
      float bv[2][16], tc[2][16];
      if ((tile + 1) * TILE <= P.V) {
        stage_read_full(Xb[u & 1], wave * WCOLS, bv);
        stage_read_full(Xt, wave * WCOLS, tc);
      } else {
        stage_read(Xb[u & 1], true, P.V, cbase, wave * WCOLS, bv);
        stage_read(Xt, true, P.V, cbase, wave * WCOLS, tc);
      }
      lds_barrier();  // every wave has its rows out of Xb[u & 1] and Xt
      issue_t(u + 1);
      issue_b(u + 2);
      const int q = rb * 32 + j;
      const int qc = q < nrej ? q : 0;
      const float Mt = s_Mt[qc], iZt = s_iZt[qc], mq = s_mq[qc], iZq = s_iZq[qc];
      // the residual in place of the target values
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int i = 0; i < 16; i++) tc[p][i] = residual_elem(tc[p][i], bv[p][i], acc[p][i], Mt, iZt, mq, iZq, sc);
      const float sl = tree_sum32(tc);
      const float sw = sum_xor32(sl);
      if (h == 0) red_s[u & 1][wave][j] = sw;
    };
    for (int u = 0; u < nunits; u++) unit(u);
    lds_barrier();  // the last unit's sums
    records(nunits - 1);
  }
}

// ---------------------------------------------------------------------------
// finalize: one wave per request

// Inverse-CDF sample of softmax(target row / T) from its 1024-column tile
// partials: fp64 scan over tiles, then the recomputed tile (same per-element
// arithmetic and lane mapping as the stream kernel).
template <typename WT>
__device__ __forceinline__ int wave_sample_target_row(const VerifyArgs<WT>& P, size_t rowj, double u) {
  const int lane = threadIdx.x & 63;
  const int nvt = ceil_div(P.V, VTILE);
  const float2* vp = P.vpart + rowj * nvt;
  const bool t_one = (P.T == 1.0f);
  const double invTd = t_one ? 1.0 : 1.0 / (double)P.T;
  const int per = ceil_div(nvt, 64);
  const int t0 = min(nvt, lane * per), t1 = min(nvt, t0 + per);
  float mloc = -INFINITY;
  for (int t = t0; t < t1; t++) mloc = fmaxf(mloc, vp[t].x);
  const float M = wave_max(mloc);
  double loc = 0.0;
  for (int t = t0; t < t1; t++) loc += (double)vp[t].y * (double)exp_acc((vp[t].x - M) * (float)invTd);
  double incl_unused;
  const double ex = wave_excl_scan_d(loc, &incl_unused);
  const double Z = __shfl(ex + loc, (nvt - 1) / per);
  const double target = u * Z;
  int found = 0x7fffffff, lastpos = -1;
  double before = 0.0, cum = 0.0;
  for (int t = t0; t < t1; t++) {
    const double w = (double)vp[t].y * (double)exp_acc((vp[t].x - M) * (float)invTd);
    const double pp = cum;
    cum += w;
    if (found == 0x7fffffff && target < ex + cum) { found = t; before = ex + pp; }
    if (vp[t].y > 0.f) lastpos = t;
  }
  int tstar = wave_min_i(found);
  double rem;
  if (tstar != 0x7fffffff) {
    rem = __shfl(target - before, tstar / per);
  } else {
    tstar = max(wave_max_i(lastpos), 0);
    rem = INFINITY;
  }
  const float mt = vp[tstar].x;
  const double scale = (double)exp_acc((mt - M) * (float)invTd);
  const float* trow = P.target + rowj * P.V;
  // lane l holds columns tstar*1024 + f*256 + 4l + e (the stream kernel's mapping)
  double carry = 0.0;
  int pick = -1;
  int lastc = -1;
#pragma unroll
  for (int f = 0; f < 4; f++) {
    const int c = tstar * VTILE + f * 256 + lane * 4;
    f32x4 x = (c < P.V) ? ld_stream4(trow + c) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    double w4[4], s4 = 0.0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float d = t_one ? (x[e] - mt) : (x[e] - mt) * P.invT;
      const float ev = exp_acc(d);
      w4[e] = (double)ev * scale;
      s4 += w4[e];
      if (ev > 0.f) lastc = c + e;
    }
    double incl;
    const double exl = wave_excl_scan_d(s4, &incl);
    const double tot = __shfl(incl, 63);
    if (pick < 0 && rem < carry + tot) {
      double run = carry + exl;
      int hit = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        run += w4[e];
        if (hit == 0x7fffffff && rem < run) hit = c + e;
      }
      const int hmin = wave_min_i(hit);
      pick = (hmin != 0x7fffffff) ? hmin : -1;
    }
    carry += tot;
  }
  if (pick < 0) pick = max(wave_max_i(lastc), 0);
  return min(pick, P.V - 1);
}

// One workgroup per request.  Residual sample: the four waves choose the tile
// and chunk from the residual records, recompute that chunk's draft bias with
// vector FMAs (chunk_bias), and wave 0 does the in-chunk search.  Bonus sample
// (or a residual with no mass): wave 0 samples the target row.
template <typename WT>
struct FinalizeSmem {
  BlockSelectSmem sm;
  float w1s[DSPARK_MAX_RANK];
  float part[32 / sizeof(WT)][WCOLS];
};

// The finalize of one request (one workgroup), from its residual tile records
// `rrec` (global, or LDS in the small-problem kernel).
template <typename WT, bool GREEDY, int KS>
__device__ __forceinline__ void finalize_request(const VerifyArgs<WT>& P, int row, const float4* rrec,
                                                 FinalizeSmem<WT>& fs) {
  BlockSelectSmem& sm = fs.sm;
  float* w1s = fs.w1s;
  auto& part = fs.part;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = P.L_of(row);
  const int ks = P.rej[row];
  const bool rejected = ks <= L;
  const int A = rejected ? ks - 1 : L;
  const size_t rowA = (size_t)row * (P.gamma + 1) + A;
  int y = 0;
  // the outputs' accepted tokens and probabilities, loaded before the sample
  // is drawn so that the final stores wait on no load
  int dt = -1;
  float tpv = -1.0f;
  if (wave == 0 && lane < P.gamma) {
    if (lane < A) dt = P.dtok[(size_t)row * P.gamma + lane];
    if (P.target_probs && lane + 1 <= min(L, A + 1)) tpv = P.tp[(size_t)row * P.gamma + lane];
  }

  if (GREEDY) {
    if (wave != 0) return;
    y = (int)P.rowstat[rowA].y;
    if (y < 0 || y >= P.V) y = 0;
  } else {
    const double u = (double)checked_uniform(P.u_fin[row], P.err);
    bool use_p = !rejected;
    if (rejected) {  // uniform over the workgroup
      const int prev = P.prev_of(row, ks);
      for (int k = tid; k < P.r; k += 256) w1s[k] = to_f32(P.W1[(size_t)prev * P.r + k]);
      // position k*'s target row statistics and draft normaliser, loaded
      // before the tile and chunk picks that precede their use
      const size_t ev = (size_t)row * P.gamma + ks - 1;
      const double2 rs = P.rowstat[(size_t)row * (P.gamma + 1) + ks - 1];
      const float dq_m = P.dstats[2 * ev], dq_z = P.dstats[2 * ev + 1];
      const int nt = ceil_div(P.V, TILE);
      const TilePick S = block_select_tile(rrec, nt, false, 1.0, u, sm);
      if (!(S.Z > 0.0)) {
        use_p = true;  // no residual mass: sample p itself
      } else {
        const int cb = S.t * TILE + S.w * WCOLS;
        const int col = cb + lane;
        float b = -INFINITY, t = -INFINITY;
        if (wave == 0 && col < P.V) {
          b = P.base[ev * P.V + col];
          t = P.target[((size_t)row * (P.gamma + 1) + ks - 1) * P.V + col];
        }
        const float bias = chunk_bias<WT, KS>(P.W2, P.V, P.r, cb, w1s, part);
        if (wave != 0) return;
        const float sc = (P.T == 1.0f) ? LOG2E_F : LOG2E_F * P.invT;
        const float d = residual_elem(t, b, bias, (float)rs.x, (float)(1.0 / rs.y), dq_m,
                                      (float)(1.0 / (double)dq_z), sc);
        y = min(cb + wave_pick64(d, 1.0, S.rem), P.V - 1);
      }
    }
    if (wave != 0) return;
    if (use_p) y = wave_sample_target_row(P, rowA, u);
  }

  // outputs (wave 0): lane i writes slot i
  int32_t* out = P.out_tokens + (size_t)row * (P.gamma + 1);
  if (lane <= P.gamma) out[lane] = (lane < A) ? dt : ((lane == A) ? y : -1);
  if (lane == 0) P.accept_len[row] = A;
  if (P.target_probs && lane < P.gamma) P.target_probs[(size_t)row * P.gamma + lane] = tpv;
}

template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) void k_verify_finalize(VerifyArgs<WT> P) {
  __shared__ FinalizeSmem<WT> fs;
  const int row = blockIdx.x;
  finalize_request<WT, GREEDY, KS>(P, row, P.rrec + (size_t)row * ceil_div(P.V, TILE) * 2, fs);
}

// Small problems (at most 16 column tiles): verify's residual and finalize in
// one workgroup per request.  A rejected request's residual tile records are
// formed in LDS with the arithmetic of k_residual_partials on block row 0 (bf16
// factors through the same fragment and MFMA chain with the request's bias row
// read by all 32 block rows, fp32 factors through the same fmaf chain per
// column, one column per thread; the base and target values of block rows
// 1..31 are zero and go unused), then the request is finalized from them as
// k_verify_finalize would: the outputs are bit-identical to the two kernels'.
constexpr int VROWS_MAX_TILES = 16;
constexpr size_t VROWS_MAX_W2_BYTES = size_t(32) << 20;  // R * r * V * sizeof(WT), W2 read per request

template <typename WT, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_verify_tail_rows(
    VerifyArgs<WT> P) {
  constexpr int APAD = BiasBlock<WT>::APAD;
  constexpr bool FP32 = std::is_same<WT, float>::value;
  __shared__ __align__(16) WT A_row[DSPARK_MAX_RANK + APAD];
  __shared__ __align__(16) float Xb[33 * BSTRIDE];  // row 0 base values, row 1 (fp32) the bias, rest 0
  __shared__ __align__(16) float Xt[32 * BSTRIDE];  // row 0 target values, rest 0
  __shared__ float red_s[4];
  __shared__ __align__(16) float4 recs[2 * VROWS_MAX_TILES];
  __shared__ FinalizeSmem<WT> fs;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x;
  const int nt = ceil_div(P.V, TILE);
  const int L = P.L_of(row);
  const int ks = P.rej[row];
  if (ks <= L) {  // uniform
    for (int i = tid; i < 33 * BSTRIDE; i += 256) Xb[i] = 0.f;
    for (int i = tid; i < 32 * BSTRIDE; i += 256) Xt[i] = 0.f;
    const float sc = (P.T == 1.0f) ? LOG2E_F : LOG2E_F * P.invT;
    const double2 rs = P.rowstat[(size_t)row * (P.gamma + 1) + ks - 1];
    const size_t ev = (size_t)row * P.gamma + ks - 1;
    const float Mt = (float)rs.x, iZt = (float)(1.0 / rs.y);
    const float mq = P.dstats[2 * ev], iZq = (float)(1.0 / (double)P.dstats[2 * ev + 1]);
    const int prev = P.prev_of(row, ks);
    for (int e = tid; e < P.r; e += 256) A_row[e] = P.W1[(size_t)prev * P.r + e];
    const float* brow = P.base + ev * P.V;
    const float* trow = P.target + ((size_t)row * (P.gamma + 1) + ks - 1) * P.V;
    __syncthreads();
    for (int t = 0; t < nt; t++) {
      const int cbase = t * TILE + wave * WCOLS;
      const int c = t * TILE + tid;
      Xb[tid] = (c < P.V) ? brow[c] : 0.f;
      Xt[tid] = (c < P.V) ? trow[c] : 0.f;
      f32x16 acc[2];
      if constexpr (FP32) {
        float a = 0.f;
        for (int kk = 0; kk < P.r; kk++)
          a = fmaf(to_f32(A_row[kk]), (c < P.V) ? to_f32(P.W2[(size_t)kk * P.V + c]) : 0.f, a);
        Xb[BSTRIDE + tid] = a;
        __syncthreads();
        float av[2][16];
        stage_read_full(Xb + BSTRIDE, wave * WCOLS, av);
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) acc[p][q] = av[p][q];
      } else {
        typename BiasBlock<WT>::template Frag<KS> F;
        BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, cbase);
        __syncthreads();
        BiasBlock<WT>::template to_operands<KS>(F);
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) acc[p][q] = 0.f;
        BiasBlock<WT>::template mma_rb_op<KS>(F, P.r, A_row, 0, acc);
      }
      float b[2][16], tv[2][16];
      if ((t + 1) * TILE <= P.V) {
        stage_read_full(Xb, wave * WCOLS, b);
        stage_read_full(Xt, wave * WCOLS, tv);
      } else {
        stage_read(Xb, true, P.V, cbase, wave * WCOLS, b);
        stage_read(Xt, true, P.V, cbase, wave * WCOLS, tv);
      }
      float d[2][16];
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int i = 0; i < 16; i++) d[p][i] = residual_elem(tv[p][i], b[p][i], acc[p][i], Mt, iZt, mq, iZq, sc);
      const float sl = tree_sum32(d);
      const float sw = sum_xor32(sl);
      if (lane == 0) red_s[wave] = sw;
      __syncthreads();
      if (tid == 0) {
        const float s0 = red_s[0], s1 = red_s[1], s2 = red_s[2], s3 = red_s[3];
        recs[2 * t] = make_float4(0.f, (s0 + s1) + (s2 + s3), s0, s1);
        recs[2 * t + 1] = make_float4(s2, s3, 0.f, 0.f);
      }
      __syncthreads();  // Xb, Xt and red_s are rewritten by the next tile; recs complete
    }
  }
  finalize_request<WT, false, KS>(P, row, recs, fs);
}

// ---------------------------------------------------------------------------
// acceptance labels c*_k = 1 - |q_k - p_k|_1 / 2 (dspark_accept_rates)

// Target row statistics (M, Z) of rows j < gamma: one workgroup per request,
// one wave per row, from the stream kernel's 1024-column partials.
template <typename WT>
__global__ __launch_bounds__(256) void k_target_rowstats(VerifyArgs<WT> P) {
  const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nvt = ceil_div(P.V, VTILE);
  const double invTd = (P.T == 1.0f) ? 1.0 : 1.0 / (double)P.T;
  for (int j = wave; j < P.gamma; j += 4) {
    const size_t rowj = (size_t)row * (P.gamma + 1) + j;
    const float2* vp = P.vpart + rowj * nvt;
    float ml = -INFINITY;
    for (int t = lane; t < nvt; t += 64) ml = fmaxf(ml, vp[t].x);
    const float M = wave_max(ml);
    double zl = 0.0;
    for (int t = lane; t < nvt; t += 64) zl += (double)vp[t].y * (double)exp_acc((vp[t].x - M) * (float)invTd);
    const double Z = wave_sum_d(zl);
    if (lane == 0) P.rowstat[rowj] = make_double2((double)M, Z);
  }
}

// c* of one item (one wave): 1 - sum over tiles of the residual sums, the
// per-lane strided sums added in a fixed order (fp64).
template <typename WT>
__global__ __launch_bounds__(256) void k_accept_finalize(VerifyArgs<WT> P, float* __restrict__ out) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= P.R * P.gamma) return;
  const int nt = ceil_div(P.V, TILE);
  const float* tp = P.tvpart + (size_t)item * nt;
  double s = 0.0;
  for (int t = lane; t < nt; t += 64) s += (double)tp[t];
  const double D = wave_sum_d(s);
  if (lane == 0) {
    out[item] = (float)(1.0 - D);
    if (!(D == D)) raise_err(P.err, DSPARK_DERR_NONFINITE);
  }
}

// Residual tile records: the per-tile kernel, which reads a tile's W2
// fragment once per chunk of 128 requests; with bf16 factors and at most two
// tiles per workgroup, the resident-W2 kernel (W2 read once per call) for the
// acceptance labels and for verify's residual over more than 128 requests.
template <typename WT, bool TVM>
static void launch_residual(const VerifyArgs<WT>& P, hipStream_t stream) {
  const int nt = ceil_div(P.V, TILE), G = device_cu_count();
  const int grid_r = min(nt, G);
  if constexpr (std::is_same<WT, uint16_t>::value) {
    if (nt <= 2 * G && (TVM || P.R > 128)) {
      DSPARK_DISPATCH_KS(P.r, hipLaunchKernelGGL((k_residual_resident<KS, TVM>), dim3(grid_r), dim3(256), 0,
                                                 stream, P));
      return;
    }
  }
  DSPARK_DISPATCH_KS(P.r, hipLaunchKernelGGL((k_residual_partials<WT, KS, TVM>), dim3(grid_r), dim3(256), 0,
                                             stream, P));
}

template <typename WT>
static int launch_accept_rates(const VerifyArgs<WT>& P, float* out, hipStream_t stream) {
  const int nseg = ceil_div(P.V, stream_seg(false));
  const long long nblk = (long long)(P.gamma + 1) * P.R * nseg;
  hipLaunchKernelGGL((k_verify_stream<WT, false>), dim3((unsigned)nblk), dim3(256), 0, stream, P);
  hipLaunchKernelGGL((k_target_rowstats<WT>), dim3(P.R), dim3(256), 0, stream, P);
  launch_residual<WT, true>(P, stream);
  hipLaunchKernelGGL((k_accept_finalize<WT>), dim3(ceil_div(P.R * P.gamma, 4)), dim3(256), 0, stream, P, out);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

// Target rows 0..L_r of every request: per-1024-column partials.  Reads only
// target and the verify lengths, so it can run before the draft is known.
template <typename WT>
static void launch_verify_stream(const VerifyArgs<WT>& P, hipStream_t stream) {
  const bool greedy = (P.T == 0.f);
  const int nseg = ceil_div(P.V, stream_seg(greedy));
  const long long nblk = (long long)(P.gamma + 1) * P.R * nseg;
  prof_before(DSPARK_KID_VERIFY_STREAM, stream);
  for (int rep = prof_repeat(DSPARK_KID_VERIFY_STREAM); rep > 0; rep--) {
    if (greedy)
      hipLaunchKernelGGL((k_verify_stream<WT, true>), dim3((unsigned)nblk), dim3(256), 0, stream, P);
    else
      hipLaunchKernelGGL((k_verify_stream<WT, false>), dim3((unsigned)nblk), dim3(256), 0, stream, P);
  }
  prof_after(DSPARK_KID_VERIFY_STREAM, stream);
}

// Accept tests, residual and emission from the stream's partials.

// DSPARK_VERIFY_KERNEL=split keeps the residual and finalize kernels apart
// even where the small-problem kernel applies; both compute the same outputs.
static bool split_requested() {
  const char* e = getenv("DSPARK_VERIFY_KERNEL");
  return e != nullptr && strcmp(e, "split") == 0;
}

template <typename WT>
static bool verify_rows_fits(const VerifyArgs<WT>& P) {
  return !split_requested() && ceil_div(P.V, TILE) <= VROWS_MAX_TILES &&
         (size_t)P.R * (size_t)P.r * (size_t)P.V * sizeof(WT) <= VROWS_MAX_W2_BYTES;
}

template <typename WT>
static int launch_verify_finish(const VerifyArgs<WT>& P, hipStream_t stream) {
  const bool greedy = (P.T == 0.f);
  prof_before(DSPARK_KID_VERIFY_DECIDE, stream);
  for (int rep = prof_repeat(DSPARK_KID_VERIFY_DECIDE); rep > 0; rep--) {
    if (greedy)
      hipLaunchKernelGGL((k_verify_decide<WT, true>), dim3(P.R), dim3(64 * decide_waves(P.gamma)), 0, stream, P);
    else
      hipLaunchKernelGGL((k_verify_decide<WT, false>), dim3(P.R), dim3(64 * decide_waves(P.gamma)), 0, stream, P);
  }
  prof_after(DSPARK_KID_VERIFY_DECIDE, stream);
  if (!greedy && verify_rows_fits(P)) {
    prof_before(DSPARK_KID_VERIFY_FINALIZE, stream);
    for (int rep = prof_repeat(DSPARK_KID_VERIFY_FINALIZE); rep > 0; rep--)
      DSPARK_DISPATCH_KS(P.r, hipLaunchKernelGGL((k_verify_tail_rows<WT, KS>), dim3(P.R), dim3(256), 0, stream, P));
    prof_after(DSPARK_KID_VERIFY_FINALIZE, stream);
    return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
  }
  if (!greedy) {
    prof_before(DSPARK_KID_RESIDUAL, stream);
    for (int rep = prof_repeat(DSPARK_KID_RESIDUAL); rep > 0; rep--) {
      launch_residual<WT, false>(P, stream);
    }
    prof_after(DSPARK_KID_RESIDUAL, stream);
  }
  prof_before(DSPARK_KID_VERIFY_FINALIZE, stream);
  for (int rep = prof_repeat(DSPARK_KID_VERIFY_FINALIZE); rep > 0; rep--) {
    if (greedy)
      hipLaunchKernelGGL((k_verify_finalize<WT, true, 1>), dim3(P.R), dim3(256), 0, stream, P);
    else
      DSPARK_DISPATCH_KS(P.r, hipLaunchKernelGGL((k_verify_finalize<WT, false, KS>), dim3(P.R), dim3(256), 0,
                                                 stream, P));
  }
  prof_after(DSPARK_KID_VERIFY_FINALIZE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

template <typename WT>
static int launch_verify(const VerifyArgs<WT>& P, hipStream_t stream, int part) {
  if (part != VERIFY_FINISH) launch_verify_stream(P, stream);
  if (part == VERIFY_STREAM) return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
  return launch_verify_finish(P, stream);
}

int verify_impl(const float* target, const float* base, const void* W1, const void* W2,
                dspark_wtype w_type, const int32_t* anchor, const int32_t* dtok, const float* dprob,
                const float* dstats, const int32_t* vlen, const float* u_acc, const float* u_fin,
                int R, int gamma, int V, int r, float T, int32_t* out_tokens, int32_t* accept_len,
                float* target_probs, void* ws, hipStream_t stream, bool dense_rows = false,
                int part = VERIFY_ALL) {
  const WsLayout Lw = ws_layout(R, gamma, V);
  auto fill = [&](auto& P) {
    P.dense = dense_rows;
    P.a_rows = dense_rows ? R * gamma : V;
    P.target = target; P.base = base;
    P.anchor = anchor; P.dtok = dtok; P.dprob = dprob; P.dstats = dstats; P.vlen = vlen;
    P.u_acc = u_acc; P.u_fin = u_fin;
    P.R = R; P.gamma = gamma; P.V = V; P.r = r;
    P.T = T; P.invT = (T > 0.f) ? 1.0f / T : 0.f;
    P.out_tokens = out_tokens; P.accept_len = accept_len; P.target_probs = target_probs;
    P.rowstat = ws_ptr<double2>(ws, Lw.rowstat);
    P.rej = ws_ptr<int32_t>(ws, Lw.rej);
    P.vpart = ws_ptr<float2>(ws, Lw.vpart);
    P.tp = ws_ptr<float>(ws, Lw.tp);
    P.rrec = ws_ptr<float4>(ws, Lw.rrec);
    P.tvpart = ws_ptr<float>(ws, Lw.tvpart);
    P.err = ws_ptr<int32_t>(ws, Lw.err);
  };
  if (w_type == DSPARK_W_BF16) {
    VerifyArgs<uint16_t> P;
    fill(P);
    P.W1 = static_cast<const uint16_t*>(W1);
    P.W2 = static_cast<const uint16_t*>(W2);
    return launch_verify(P, stream, part);
  }
  VerifyArgs<float> P;
  fill(P);
  P.W1 = static_cast<const float*>(W1);
  P.W2 = static_cast<const float*>(W2);
  return launch_verify(P, stream, part);
}

int accept_rates_impl(const float* target, const float* base, const void* W1, const void* W2,
                      dspark_wtype w_type, const int32_t* anchor, const int32_t* dtok, const float* dstats,
                      int R, int gamma, int V, int r, float T, float* out, void* ws, hipStream_t stream) {
  const WsLayout Lw = ws_layout(R, gamma, V);
  auto fill = [&](auto& P) {
    P = {};
    P.dense = false;
    P.a_rows = V;
    P.target = target; P.base = base;
    P.anchor = anchor; P.dtok = dtok; P.dstats = dstats; P.vlen = nullptr;
    P.R = R; P.gamma = gamma; P.V = V; P.r = r;
    P.T = T; P.invT = 1.0f / T;
    P.rowstat = ws_ptr<double2>(ws, Lw.rowstat);
    P.vpart = ws_ptr<float2>(ws, Lw.vpart);
    P.tvpart = ws_ptr<float>(ws, Lw.tvpart);
    P.err = ws_ptr<int32_t>(ws, Lw.err);
  };
  if (w_type == DSPARK_W_BF16) {
    VerifyArgs<uint16_t> P;
    fill(P);
    P.W1 = static_cast<const uint16_t*>(W1);
    P.W2 = static_cast<const uint16_t*>(W2);
    return launch_accept_rates(P, out, stream);
  }
  VerifyArgs<float> P;
  fill(P);
  P.W1 = static_cast<const float*>(W1);
  P.W2 = static_cast<const float*>(W2);
  return launch_accept_rates(P, out, stream);
}

}  // namespace dspark
