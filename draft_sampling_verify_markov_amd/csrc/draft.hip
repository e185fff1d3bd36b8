// Markov-head sequential drafting (dspark_draft).
//
// Source: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), section "Arquitetura": Semi-Autoregressive Generation
// (the sequential stage adds a prefix-dependent transition bias B_k to the
// parallel stage's base logits and samples position by position) and the
// Markov head (first-order bias from the immediately preceding token, low-rank
// B = W1 W2, default rank 256).  The anchor is the first prediction position,
// so the token before position 1 is the anchor.
//
// Per step k (sequential in k, data-parallel over requests and vocabulary):
//   K1 draft_partials  grid = V / 256 column tiles, 4 waves each.
//        Gathers W1[x_{k-1}] for a block of 128 requests into LDS, runs the
//        (R x r) . (r x 256) bias product on bf16 MFMA 32x32x16 with fp32
//        accumulation, adds the base logits in the epilogue and writes per
//        (request, tile) softmax partials (max, sum exp) plus the four per-wave
//        sums.  z is never written to memory.
//   K2 draft_select    one wave per request (4 per workgroup).
//        Combines the tile records in fp64 (wave shuffles), finds the tile and
//        then the 64-column chunk holding u * Z, recomputes that chunk's logits
//        with the same MFMA instruction sequence and does the in-chunk
//        inverse-CDF search.
#include "select.h"

namespace dspark {

template <typename WT>
struct DraftStep {
  const float* base;
  const WT* W1;
  const WT* W2;
  const int32_t* anchor;
  const float* u_draft;
  int R, gamma, V, r, k;  // k: 1-based step
  float T, invT;
  int32_t* tokens;
  float* probs;
  float* stats;
  float4* trec;  // [R][nt][2] tile records
  int32_t* err;

  __device__ int prev_token(int row) const {
    const int t = (k == 1) ? anchor[row] : tokens[(size_t)row * gamma + k - 2];
    return checked_token(t, V, err);
  }
  __device__ const float* base_row(int row) const {
    return base + ((size_t)row * gamma + (k - 1)) * V;
  }
};

// Scaled, max-shifted logit: ((b - m) + bias) / T.  Subtracting the fp32 max
// from the fp32 base value first keeps the argument accurate near the top of
// the distribution, where the probability mass is.
__device__ __forceinline__ float shifted(float b, float m, float bias, float invT, bool t_one) {
  float d = (b - m) + bias;
  return t_one ? d : d * invT;
}

template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) void k_draft_partials(DraftStep<WT> P) {
  constexpr int APAD = BiasBlock<WT>::APAD;
  constexpr int A_ELEMS = RCH * (DSPARK_MAX_RANK + APAD);
  static_assert(A_ELEMS * sizeof(WT) >= 2 * 32 * BSTRIDE * sizeof(float), "staging fits the W1 block");
  // The gathered W1 block; after the MFMA the same bytes stage base rows.
  __shared__ __align__(16) WT A_lds[A_ELEMS];
  __shared__ float red_m[4][RCH];
  __shared__ float red_s[4][RCH];
  __shared__ int red_i[4][RCH];
  float* const X0 = reinterpret_cast<float*>(A_lds);
  float* const X1 = X0 + 32 * BSTRIDE;

  const int a_stride = P.r + APAD;
  const int tile = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int tile0 = tile * TILE;
  const int cbase = tile0 + wave * WCOLS;
  const int nt = gridDim.x;
  const bool t_one = (P.T == 1.0f);
  const uint32_t row_bytes = (uint32_t)(P.gamma * P.V) * 4u;

  for (int c0 = 0; c0 < P.R; c0 += RCH) {
    const int nrows = min(RCH, P.R - c0), nrb = ceil_div(nrows, 32);
    // W2 slice of this wave for the whole k range (re-read per 128-row chunk so
    // the fragment registers are free after each chunk's MFMA).
    typename BiasBlock<WT>::template Frag<KS> F;
    BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, cbase);
    __syncthreads();
    gather_w1_rows<WT, KS * sizeof(WT) / 2>(P.W1, P.V, P.r, nrows, nrb * 32, A_lds, a_stride,
                                            [&](int i) { return P.prev_token(c0 + i); });
    // base rows of this chunk, addressed from its first row: blocks 0-1 in
    // flight during the MFMA, 2-3 during the first two epilogues
    const size_t first = (size_t)c0 * P.gamma + (P.k - 1);
    const rsrc_t brs = make_rsrc(P.base + first * P.V, ((size_t)P.R * P.gamma - first) * P.V * 4);
    u32x4 va[8], vb[8];
    stage_load(va, brs, row_bytes, 0, nrows, P.V, tile0);
    stage_load(vb, brs, row_bytes, 1, nrows, P.V, tile0);
    __syncthreads();

    f32x16 acc[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; rb++)
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int t = 0; t < 16; t++) acc[rb][p][t] = 0.f;
    BiasBlock<WT>::template mma<KS>(F, P.r, A_lds, a_stride, nrb, acc);
    __syncthreads();  // the W1 block is dead: reuse its bytes for staging
    stage_store(va, X0);
    stage_store(vb, X1);
    stage_load(va, brs, row_bytes, 2, nrows, P.V, tile0);
    stage_load(vb, brs, row_bytes, 3, nrows, P.V, tile0);
    __syncthreads();

#pragma unroll
    for (int rb = 0; rb < 4; rb++) {
      if (rb >= nrb) break;
      if (rb == 2) {
        __syncthreads();
        stage_store(va, X0);
        stage_store(vb, X1);
        __syncthreads();
      }
      const int rl = rb * 32 + j, row = c0 + rl;
      const bool rowv = rl < nrows;
      float b[2][16];
      stage_read((rb & 1) ? X1 : X0, rowv, P.V, cbase, wave * WCOLS, b);
      float4* rec = P.trec + ((size_t)row * nt + tile) * 2;

      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        bool bad = false;
#pragma unroll
        for (int t = 0; t < 16; t++)
#pragma unroll
          for (int p = 0; p < 2; p++) {
            const float z = b[p][t] + acc[rb][p][t];
            bad |= (z != z);
            if (z > bv) { bv = z; bi = cbase + elem_col(p, t, h); }
          }
        if (bad) raise_err(P.err, DSPARK_DERR_NONFINITE);
        argmax_merge(bv, bi, __shfl_xor(bv, 32), __shfl_xor(bi, 32));
        if (h == 0) { red_m[wave][rl] = bv; red_i[wave][rl] = bi; }
        __syncthreads();
        if (wave == 0 && h == 0 && rowv) {
          float v = red_m[0][rl];
          int i = red_i[0][rl];
#pragma unroll
          for (int w = 1; w < 4; w++) argmax_merge(v, i, red_m[w][rl], red_i[w][rl]);
          rec[0] = make_float4(v, __int_as_float(i), 0.f, 0.f);
        }
      } else {
        float ml = -INFINITY;
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int t = 0; t < 16; t++) ml = fmaxf(ml, b[p][t] + acc[rb][p][t]);
        const float mw = fmaxf(ml, __shfl_xor(ml, 32));
        if (h == 0) red_m[wave][rl] = mw;
        __syncthreads();
        const float mt = fmaxf(fmaxf(red_m[0][rl], red_m[1][rl]), fmaxf(red_m[2][rl], red_m[3][rl]));
        float e[2][16];
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int t = 0; t < 16; t++) e[p][t] = exp_acc(shifted(b[p][t], mt, acc[rb][p][t], P.invT, t_one));
        const float sl = tree_sum32(e);
        const float sw = sl + __shfl_xor(sl, 32);
        if (h == 0) red_s[wave][rl] = sw;
        __syncthreads();
        if (wave == 0 && h == 0 && rowv) {
          const float s0 = red_s[0][rl], s1 = red_s[1][rl], s2 = red_s[2][rl], s3 = red_s[3][rl];
          const float st = (s0 + s1) + (s2 + s3);
          rec[0] = make_float4(mt, st, s0, s1);
          rec[1] = make_float4(s2, s3, 0.f, 0.f);
          if (is_bad(st) || is_bad(mt)) raise_err(P.err, DSPARK_DERR_NONFINITE);
        }
      }
    }
  }
}

// One wave per request: tile selection over the records, recompute of the
// chosen 64-column chunk, in-chunk inverse CDF.
template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) void k_draft_select(DraftStep<WT> P) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int row = blockIdx.x * 4 + wave;
  if (row >= P.R) return;  // waves are independent: no block-level barrier below
  const int nt = ceil_div(P.V, TILE);
  const float4* recs = P.trec + (size_t)row * nt * 2;
  const size_t ev = (size_t)row * P.gamma + (P.k - 1);

  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = lane; t < nt; t += 64) {
      const float4 r0 = recs[2 * t];
      argmax_merge(bv, bi, r0.x, __float_as_int(r0.y));
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
      int x = bi;
      if (x < 0 || x >= P.V) x = 0;  // only with non-finite logits (flagged)
      P.tokens[ev] = x;
      P.probs[ev] = 1.0f;
      P.stats[2 * ev] = bv;
      P.stats[2 * ev + 1] = 1.0f;
    }
    return;
  }

  const bool t_one = (P.T == 1.0f);
  const double invTd = t_one ? 1.0 : 1.0 / (double)P.T;
  const int prev = P.prev_token(row);
  const float u = checked_uniform(P.u_draft[ev], P.err);
  const TilePick S = wave_select_tile(recs, nt, true, invTd, (double)u);
  const int cb = S.t * TILE + S.w * WCOLS;

  typename BiasBlock<WT>::template Frag<KS> F;
  BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, cb);
  typename BiasBlock<WT>::template Row<KS> w1;
  BiasBlock<WT>::template load_row<KS>(w1, P.W1, P.r, prev);
  float bvals[2][16];
  load_row_cols(make_rsrc(P.base_row(row), (size_t)P.V * 4), 0u, j == 0, P.V, cb, bvals);
  f32x16 acc[2];
#pragma unroll
  for (int p = 0; p < 2; p++)
#pragma unroll
    for (int t = 0; t < 16; t++) acc[p][t] = 0.f;
  BiasBlock<WT>::template mma_row<KS>(F, P.r, w1, acc);
  float e[2][16];
#pragma unroll
  for (int p = 0; p < 2; p++)
#pragma unroll
    for (int t = 0; t < 16; t++) e[p][t] = exp_acc(shifted(bvals[p][t], S.mt, acc[p][t], P.invT, t_one));
  const float ec = chunk_to_lanes(e);
  const int c = wave_pick64(ec, S.scale, S.rem);
  const float ex = __shfl(ec, c);
  if (lane == 0) {
    const int x = min(cb + c, P.V - 1);
    P.tokens[ev] = x;
    P.probs[ev] = (float)((double)ex * S.scale / S.Z);
    P.stats[2 * ev] = S.M;
    P.stats[2 * ev + 1] = (float)S.Z;
    if (!(S.Z > 0.0) || is_bad(S.M)) raise_err(P.err, DSPARK_DERR_NONFINITE);
  }
}

template <typename WT>
static int launch_draft(const float* base, const void* W1, const void* W2, const int32_t* anchor,
                        const float* u_draft, int R, int gamma, int V, int r, float T,
                        int32_t* tokens, float* probs, float* stats, void* ws, hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, V);
  DraftStep<WT> P;
  P.base = base;
  P.W1 = static_cast<const WT*>(W1);
  P.W2 = static_cast<const WT*>(W2);
  P.anchor = anchor;
  P.u_draft = u_draft;
  P.R = R; P.gamma = gamma; P.V = V; P.r = r;
  P.T = T;
  P.invT = (T > 0.f) ? 1.0f / T : 0.f;
  P.tokens = tokens; P.probs = probs; P.stats = stats;
  P.trec = ws_ptr<float4>(ws, L.trec);
  P.err = ws_ptr<int32_t>(ws, L.err);
  const int nt = ceil_div(V, TILE);
  for (int k = 1; k <= gamma; k++) {
    P.k = k;
    prof_before(DSPARK_KID_DRAFT_PARTIALS, stream);
    DSPARK_DISPATCH_KS(r, {
      if (T == 0.f)
        hipLaunchKernelGGL((k_draft_partials<WT, true, KS>), dim3(nt), dim3(256), 0, stream, P);
      else
        hipLaunchKernelGGL((k_draft_partials<WT, false, KS>), dim3(nt), dim3(256), 0, stream, P);
    });
    prof_after(DSPARK_KID_DRAFT_PARTIALS, stream);
    prof_before(DSPARK_KID_DRAFT_SELECT, stream);
    DSPARK_DISPATCH_KS(r, {
      if (T == 0.f)
        hipLaunchKernelGGL((k_draft_select<WT, true, 1>), dim3(ceil_div(R, 4)), dim3(256), 0, stream, P);
      else
        hipLaunchKernelGGL((k_draft_select<WT, false, KS>), dim3(ceil_div(R, 4)), dim3(256), 0, stream, P);
    });
    prof_after(DSPARK_KID_DRAFT_SELECT, stream);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int draft_impl(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
               const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r, float T,
               int32_t* tokens, float* probs, float* stats, void* ws, hipStream_t stream) {
  if (w_type == DSPARK_W_BF16)
    return launch_draft<uint16_t>(base, W1, W2, anchor, u_draft, R, gamma, V, r, T, tokens, probs,
                                  stats, ws, stream);
  return launch_draft<float>(base, W1, W2, anchor, u_draft, R, gamma, V, r, T, tokens, probs, stats,
                             ws, stream);
}

}  // namespace dspark
