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
//   K1 draft_partials  persistent, one workgroup (4 waves) per compute unit,
//        looping over 256-column tiles.  Gathers W1[x_{k-1}] for a chunk of
//        128 requests into LDS once, runs the (R x r) . (r x 256) bias product
//        on bf16 MFMA 32x32x16 with fp32 accumulation one 32-request block at
//        a time, adds the base logits (brought into LDS by direct-to-LDS loads
//        two blocks ahead) in the epilogue and writes per (request, tile)
//        softmax partials (max, sum exp) plus the four per-wave sums.  z is
//        never written to memory.
//   K2 draft_select    one workgroup per request.
//        Combines the tile records in fp64, finds the tile and then the
//        64-column chunk holding u * Z, recomputes that chunk's logits (the
//        bias with vector FMAs over all 256 threads and a fixed-order sum of
//        their partials, so its rounding differs from the MFMA sums behind
//        the records by fp32 accumulation error only) and does the in-chunk
//        inverse-CDF search.
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "rnn.h"
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
  // Bias rows: W1 indexed by the previous token (Markov head), or, with dense
  // set, a table of a_rows = R * gamma rows where row r * gamma + k - 1 holds
  // the RNN head's state s_k of request r.
  bool dense;
  int a_rows;

  __device__ int prev_token(int row) const {
    if (dense) return row * gamma + k - 1;
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

// Requests per chunk (rows of the gathered W1 block held in LDS).
template <typename WT>
struct DraftChunk {
  static constexpr int ROWS = sizeof(WT) == 2 ? 128 : 64;
};

// Persistent over column tiles: workgroup g handles tiles g, g + G, ... of the
// vocabulary.  Per request chunk the W1 rows are gathered into LDS once.  The
// work is cut into units (tile, 32-row block); a unit's base rows arrive in
// LDS by direct-to-LDS loads issued two units ahead (ring of two buffers), the
// unit's bias block is one MFMA chain per wave, and the epilogue adds the base
// logits and reduces per wave.  The next tile's W2 fragment is loaded into
// registers during the last unit of the current tile.
template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_draft_partials(DraftStep<WT> P) {
  constexpr int APAD = BiasBlock<WT>::APAD;
  constexpr int CH = DraftChunk<WT>::ROWS;
  constexpr int EPV = 16 / sizeof(WT);
  constexpr int GPER = CH * (KS * 16 / EPV) / 256;
  __shared__ __align__(16) WT A_lds[CH * (DSPARK_MAX_RANK + APAD)];
  __shared__ __align__(16) float X[2][32 * BSTRIDE];
  __shared__ float red_m[4][CH];
  __shared__ float red_s[4][CH];
  __shared__ int red_i[4][CH];
  __shared__ int s_tok[CH];

  const int a_stride = P.r + APAD;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, h = lane >> 5;
  const int nt = ceil_div(P.V, TILE);
  const int G = gridDim.x;
  const bool t_one = (P.T == 1.0f);
  const uint32_t row_bytes = (uint32_t)(P.gamma * P.V) * 4u;
  if ((int)blockIdx.x >= nt) return;
  const int my_tiles = (nt - (int)blockIdx.x + G - 1) / G;

  for (int c0 = 0; c0 < P.R; c0 += CH) {
    const int nrows = min(CH, P.R - c0), nrb = ceil_div(nrows, 32);
    const int nunits = my_tiles * nrb;
    const size_t first = (size_t)c0 * P.gamma + (P.k - 1);
    const rsrc_t brs = make_rsrc(P.base + first * P.V, ((size_t)P.R * P.gamma - first) * P.V * 4);
    auto issue = [&](int u) {
      if (u < nunits) {
        const int ti = u / nrb, rb = u - ti * nrb;
        stage_dma(brs, row_bytes, rb, nrows, ((int)blockIdx.x + ti * G) * TILE, X[u & 1]);
      }
    };

    __syncthreads();  // the previous chunk is done with A_lds, X, red_* and s_tok
    if ((int)threadIdx.x < CH) s_tok[threadIdx.x] = (int)threadIdx.x < nrows ? P.prev_token(c0 + threadIdx.x) : -1;
    __syncthreads();
    // issue order: W1 rows, the first unit's base rows, the W2 fragment, the
    // second unit's rows -- the same order (fragment, then one unit of rows)
    // as at every later tile start, which the waits below count on
    W1Gather<WT, GPER> g;
    g.load(P.W1, P.a_rows, P.r, nrows, CH, a_stride, [&](int i) { return s_tok[i]; });
    issue(0);
    typename BiasBlock<WT>::template Frag<KS> F;
    BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, (int)blockIdx.x * TILE + wave * WCOLS);
    issue(1);
    g.store(A_lds);

    const float sc = t_one ? LOG2E_F : LOG2E_F * P.invT;
    int u = 0;
    // One unit: wait for its base rows, MFMA, epilogue, then refill the
    // freed buffer two units ahead.  CONVERT: first unit of a tile (turns
    // the loaded fragment into operand form); RELOAD: last unit of a tile
    // (loads the next tile's fragment once the MFMA chain has used it).
    auto unit = [&](int tile, int rb, auto convert, auto reload) {
      const int cbase = tile * TILE + wave * WCOLS;
      if (u + 1 < nunits)
        wait_vmcnt<8>();  // this unit's rows are in; the next unit's may be in flight
      else
        wait_vmcnt<0>();
      lds_barrier();
      if constexpr (decltype(convert)::value) BiasBlock<WT>::template to_operands<KS>(F);

      f32x16 acc[2];
#pragma unroll
      for (int p = 0; p < 2; p++)
#pragma unroll
        for (int t = 0; t < 16; t++) acc[p][t] = 0.f;
      BiasBlock<WT>::template mma_rb_op<KS>(F, P.r, A_lds + rb * 32 * a_stride, a_stride, acc);
      if constexpr (decltype(reload)::value) {
        if (tile + G < nt) BiasBlock<WT>::template load<KS>(F, P.W2, P.V, P.r, (tile + G) * TILE + wave * WCOLS);
      }

      const int rl = rb * 32 + j;
      float b[2][16];
      if ((tile + 1) * TILE <= P.V)
        stage_read_full(X[u & 1], wave * WCOLS, b);
      else
        stage_read(X[u & 1], true, P.V, cbase, wave * WCOLS, b);
      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        bool bad = false;
#pragma unroll
        for (int t = 0; t < 16; t++)
#pragma unroll
          for (int p = 0; p < 2; p++) {
            const float z = b[p][t] + acc[p][t];
            bad |= (z != z);
            if (z > bv) { bv = z; bi = cbase + elem_col(p, t, h); }
          }
        if (bad) raise_err(P.err, DSPARK_DERR_NONFINITE);
        argmax_xor32(bv, bi);
        if (h == 0) { red_m[wave][rl] = bv; red_i[wave][rl] = bi; }
      } else {
        float ml = -INFINITY;
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int t = 0; t < 16; t++) ml = fmaxf(ml, b[p][t] + acc[p][t]);
        const float mw = max_xor32(ml);
        // a wave whose columns are all past V (or all -inf) has mass 0
        const float mref = (mw == -INFINITY) ? 0.f : mw;
        float e[2][16];
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int t = 0; t < 16; t++) e[p][t] = exp2_scaled((b[p][t] - mref) + acc[p][t], sc);
        const float sl = tree_sum32(e);
        const float sw = sum_xor32(sl);
        if (h == 0) { red_m[wave][rl] = mw; red_s[wave][rl] = sw; }
      }
      lds_barrier();  // X[u & 1] is free again; red_* of this unit complete
      issue(u + 2);
      u++;
    };

    // tile records, one thread per request, after the tile's last row block
    auto finalize = [&](int tile) {
      if ((int)threadIdx.x >= nrows) return;
      const int q = threadIdx.x;
      float4* rec = P.trec + ((size_t)(c0 + q) * nt + tile) * 2;
      if (GREEDY) {
        float v = red_m[0][q];
        int i = red_i[0][q];
#pragma unroll
        for (int w = 1; w < 4; w++) argmax_merge(v, i, red_m[w][q], red_i[w][q]);
        rec[0] = make_float4(v, __int_as_float(i), 0.f, 0.f);
      } else {
        const float m0 = red_m[0][q], m1 = red_m[1][q], m2 = red_m[2][q], m3 = red_m[3][q];
        const float mt = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
        auto rescale = [&](float sw, float mw) {
          const float d = t_one ? (mw - mt) : (mw - mt) * P.invT;
          return (mw == -INFINITY) ? 0.f : sw * exp_acc(d);
        };
        const float s0 = rescale(red_s[0][q], m0), s1 = rescale(red_s[1][q], m1);
        const float s2 = rescale(red_s[2][q], m2), s3 = rescale(red_s[3][q], m3);
        const float st = (s0 + s1) + (s2 + s3);
        rec[0] = make_float4(mt, st, s0, s1);
        rec[1] = make_float4(s2, s3, 0.f, 0.f);
        // a fully -inf tile (masked vocabulary) is valid: mass 0
        if (is_bad(st) || !(mt == mt) || mt == INFINITY) raise_err(P.err, DSPARK_DERR_NONFINITE);
      }
    };

    using T_ = std::true_type;
    using F_ = std::false_type;
    for (int ti = 0; ti < my_tiles; ti++) {
      const int tile = (int)blockIdx.x + ti * G;
      if (nrb == 1) {
        unit(tile, 0, T_{}, T_{});
      } else {
        unit(tile, 0, T_{}, F_{});
        for (int rb = 1; rb < nrb - 1; rb++) unit(tile, rb, F_{}, F_{});
        unit(tile, nrb - 1, F_{}, T_{});
      }
      finalize(tile);
    }
  }
}

// One workgroup per request.  The four waves read the row's tile records
// together and choose the tile and then the 64-column chunk holding u * Z.
// The chunk's bias W1[x_{k-1}] . W2[:, chunk] is then recomputed on the
// vector ALUs: thread (c, q) forms the fp32 dot product over k = q, q+4, ...
// for column c (exact bf16 products, fp32 sums), the four partials are added
// in a fixed order, and wave 0 does the in-chunk inverse-CDF search with one
// column per lane.
template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) void k_draft_select(DraftStep<WT> P) {
  constexpr int KQ = KS * 4;  // k values per thread (r <= 16 KS)
  __shared__ BlockSelectSmem sm;
  __shared__ float w1s[DSPARK_MAX_RANK];
  __shared__ float part[32 / sizeof(WT)][WCOLS];  // [k groups][columns]
  __shared__ float gm[4];
  __shared__ int gi[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row = blockIdx.x;
  const int nt = ceil_div(P.V, TILE);
  const float4* recs = P.trec + (size_t)row * nt * 2;
  const size_t ev = (size_t)row * P.gamma + (P.k - 1);

  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = tid; t < nt; t += 256) {
      const float4 r0 = recs[2 * t];
      argmax_merge(bv, bi, r0.x, __float_as_int(r0.y));
    }
    wave_argmax(bv, bi);
    if (lane == 0) { gm[wave] = bv; gi[wave] = bi; }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < 4; w++) argmax_merge(bv, bi, gm[w], gi[w]);
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
  // W1 row of the previous token into LDS (published by the select's barriers)
  const int prev = P.prev_token(row);
  for (int k = tid; k < P.r; k += 256) w1s[k] = to_f32(P.W1[(size_t)prev * P.r + k]);
  const float u = checked_uniform(P.u_draft[ev], P.err);
  const TilePick S = block_select_tile(recs, nt, true, invTd, (double)u, sm);
  const int cb = S.t * TILE + S.w * WCOLS;

  // base logit of column cb + lane (wave 0), issued before the W2 loads
  const int col = cb + lane;
  float bval = 0.f;
  if (wave == 0) bval = (col < P.V) ? P.base_row(row)[col] : -INFINITY;

  const float bias = chunk_bias<WT, KS>(P.W2, P.V, P.r, cb, w1s, part);
  if (wave != 0) return;
  const float sc = t_one ? LOG2E_F : LOG2E_F * P.invT;
  const float ec = exp2_scaled((bval - S.mt) + bias, sc);
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

// Small problems: one workgroup per request runs all gamma steps.  A
// request's draw depends only on its own previous token, so no workgroup
// waits on another.  Per step and tile the workgroup computes the bias block
// of its single request with the arithmetic of k_draft_partials: bf16 factors
// through the same fragment and MFMA chain (the request's W1 row read by all
// 32 block rows, a zero row stride), fp32 factors through the same fmaf chain
// per column, one column per thread; then the same epilogue on block row 0.
// It keeps the tile records in LDS and draws with the selection of
// k_draft_select, so its outputs are bit-identical to the per-step kernels'.  The step's base row
// sits in LDS (the next step's is loaded during the current one); with fp32
// factors W2 is staged in LDS once, with bf16 factors every workgroup reads
// W2 once per step, which bounds the sizes this path takes (draft_rows_fits).
constexpr int ROWS_MAX_TILES = 16;
constexpr int ROWS_MAX_V = ROWS_MAX_TILES * TILE;
constexpr int ROWS_W2_LDS_FLOATS = 16384;                // fp32 factors: r * V at most
constexpr size_t ROWS_MAX_W2_BYTES = size_t(32) << 20;  // bf16: R * gamma * r * V * 2 at most

template <typename WT>
static bool draft_rows_fits(int R, int gamma, int V, int r) {
  if (ceil_div(V, TILE) > ROWS_MAX_TILES) return false;
  if (std::is_same<WT, float>::value) return (size_t)r * (size_t)V <= (size_t)ROWS_W2_LDS_FLOATS;
  return (size_t)R * (size_t)gamma * (size_t)r * (size_t)V * sizeof(WT) <= ROWS_MAX_W2_BYTES;
}

template <typename WT, bool GREEDY, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_draft_rows(DraftStep<WT> P) {
  constexpr int APAD = BiasBlock<WT>::APAD;
  constexpr bool W2_LDS = std::is_same<WT, float>::value;
  constexpr int PF = ROWS_MAX_V / 256;  // base values per thread of a prefetched row
  __shared__ __align__(16) WT A_row[DSPARK_MAX_RANK + APAD];
  // block rows of the tile's base values: row 0 the request's; with fp32
  // factors row 1 holds its bias (read as block row 0 from X + BSTRIDE); the
  // rest zero
  __shared__ __align__(16) float X[33 * BSTRIDE];
  __shared__ __align__(16) float Bs[2][ROWS_MAX_V];
  __shared__ __align__(16) WT W2s[W2_LDS ? ROWS_W2_LDS_FLOATS : 1];
  __shared__ float red_m[4], red_s[4];
  __shared__ int red_i[4];
  __shared__ __align__(16) float4 recs[2 * ROWS_MAX_TILES];
  __shared__ BlockSelectSmem sm;
  __shared__ float w1s[DSPARK_MAX_RANK];
  __shared__ float part[32 / sizeof(WT)][WCOLS];
  __shared__ float gm[4];
  __shared__ int gi[4];
  __shared__ int s_x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int row = blockIdx.x;
  const int nt = ceil_div(P.V, TILE);
  const bool t_one = (P.T == 1.0f);
  const float sc = t_one ? LOG2E_F : LOG2E_F * P.invT;
  const double invTd = t_one ? 1.0 : 1.0 / (double)P.T;
  const WT* W2 = W2_LDS ? W2s : P.W2;

  auto load_base = [&](int k, float (&v)[PF]) {  // base row of step k, in registers
    const float* brow = P.base + ((size_t)row * P.gamma + (k - 1)) * P.V;
#pragma unroll
    for (int i = 0; i < PF; i++) {
      const int c = tid + 256 * i;
      v[i] = (c < P.V) ? brow[c] : 0.f;
    }
  };
  auto store_base = [&](float* dst, const float (&v)[PF]) {
#pragma unroll
    for (int i = 0; i < PF; i++) dst[tid + 256 * i] = v[i];
  };
  {
    float v[PF];
    load_base(1, v);
    if (W2_LDS)
      for (int i = tid; i < P.r * P.V; i += 256) W2s[i] = P.W2[i];
    for (int i = tid; i < 33 * BSTRIDE; i += 256) X[i] = 0.f;
    if (tid == 0) s_x = checked_token(P.anchor[row], P.V, P.err);
    store_base(Bs[0], v);
  }
  __syncthreads();

  for (int k = 1; k <= P.gamma; k++) {
    const int prev = s_x;
    const size_t ev = (size_t)row * P.gamma + (k - 1);
    const float* bl = Bs[(k - 1) & 1];
    float nxt[PF];
    if (k < P.gamma) load_base(k + 1, nxt);
    // the previous token's W1 row (the MMA operand of every block row) and,
    // widened, the chunk recompute's copy
    for (int e = tid; e < P.r; e += 256) {
      const WT w = P.W1[(size_t)prev * P.r + e];
      A_row[e] = w;
      w1s[e] = to_f32(w);
    }
    if (W2_LDS) __syncthreads();  // A_row complete before the per-column sums read it
    for (int t = 0; t < nt; t++) {
      const int cbase = t * TILE + wave * WCOLS;
      f32x16 acc[2];
      X[tid] = bl[t * TILE + tid];  // block row 0 (past V: 0, masked by the reader)
      if constexpr (W2_LDS) {
        // fp32 factors: the request's bias at column t TILE + tid, the fmaf
        // chain of the block's MMA (ascending k from 0); columns past V have
        // W2 = 0 there
        const int c = t * TILE + tid;
        float a = 0.f;
        for (int kk = 0; kk < P.r; kk++)
          a = fmaf(to_f32(A_row[kk]), (c < P.V) ? to_f32(W2s[(size_t)kk * P.V + c]) : 0.f, a);
        X[BSTRIDE + tid] = a;
        __syncthreads();
        float av[2][16];
        stage_read_full(X + BSTRIDE, wave * WCOLS, av);
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) acc[p][q] = av[p][q];
      } else {
        typename BiasBlock<WT>::template Frag<KS> F;
        BiasBlock<WT>::template load<KS>(F, W2, P.V, P.r, t * TILE + wave * WCOLS);
        __syncthreads();
        BiasBlock<WT>::template to_operands<KS>(F);
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) acc[p][q] = 0.f;
        BiasBlock<WT>::template mma_rb_op<KS>(F, P.r, A_row, 0, acc);
      }
      float b[2][16];
      if ((t + 1) * TILE <= P.V)
        stage_read_full(X, wave * WCOLS, b);
      else
        stage_read(X, true, P.V, cbase, wave * WCOLS, b);
      if (GREEDY) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        bool bad = false;
#pragma unroll
        for (int q = 0; q < 16; q++)
#pragma unroll
          for (int p = 0; p < 2; p++) {
            const float z = b[p][q] + acc[p][q];
            bad |= (z != z);
            if (z > bv) { bv = z; bi = cbase + elem_col(p, q, h); }
          }
        if (bad) raise_err(P.err, DSPARK_DERR_NONFINITE);
        argmax_xor32(bv, bi);
        if (lane == 0) { red_m[wave] = bv; red_i[wave] = bi; }
      } else {
        float ml = -INFINITY;
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) ml = fmaxf(ml, b[p][q] + acc[p][q]);
        const float mw = max_xor32(ml);
        const float mref = (mw == -INFINITY) ? 0.f : mw;
        float e[2][16];
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
          for (int q = 0; q < 16; q++) e[p][q] = exp2_scaled((b[p][q] - mref) + acc[p][q], sc);
        const float sl = tree_sum32(e);
        const float sw = sum_xor32(sl);
        if (lane == 0) { red_m[wave] = mw; red_s[wave] = sw; }
      }
      __syncthreads();
      if (tid == 0) {
        if (GREEDY) {
          float v = red_m[0];
          int i = red_i[0];
#pragma unroll
          for (int w = 1; w < 4; w++) argmax_merge(v, i, red_m[w], red_i[w]);
          recs[2 * t] = make_float4(v, __int_as_float(i), 0.f, 0.f);
        } else {
          const float m0 = red_m[0], m1 = red_m[1], m2 = red_m[2], m3 = red_m[3];
          const float mt = fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
          auto rescale = [&](float swv, float mwv) {
            const float d = t_one ? (mwv - mt) : (mwv - mt) * P.invT;
            return (mwv == -INFINITY) ? 0.f : swv * exp_acc(d);
          };
          const float s0 = rescale(red_s[0], m0), s1 = rescale(red_s[1], m1);
          const float s2 = rescale(red_s[2], m2), s3 = rescale(red_s[3], m3);
          const float st = (s0 + s1) + (s2 + s3);
          recs[2 * t] = make_float4(mt, st, s0, s1);
          recs[2 * t + 1] = make_float4(s2, s3, 0.f, 0.f);
          if (is_bad(st) || !(mt == mt) || mt == INFINITY) raise_err(P.err, DSPARK_DERR_NONFINITE);
        }
      }
      __syncthreads();  // X and red_* are rewritten by the next tile; recs complete
    }

    // the draw from the records (k_draft_select's selection)
    if (GREEDY) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int t = tid; t < nt; t += 256) {
        const float4 r0 = recs[2 * t];
        argmax_merge(bv, bi, r0.x, __float_as_int(r0.y));
      }
      wave_argmax(bv, bi);
      if (lane == 0) { gm[wave] = bv; gi[wave] = bi; }
      __syncthreads();
      if (tid == 0) {
        for (int w = 1; w < 4; w++) argmax_merge(bv, bi, gm[w], gi[w]);
        int x = bi;
        if (x < 0 || x >= P.V) x = 0;  // only with non-finite logits (flagged)
        P.tokens[ev] = x;
        P.probs[ev] = 1.0f;
        P.stats[2 * ev] = bv;
        P.stats[2 * ev + 1] = 1.0f;
        s_x = x;
      }
    } else {
      const float u = checked_uniform(P.u_draft[ev], P.err);
      const TilePick S = block_select_tile(recs, nt, true, invTd, (double)u, sm);
      const int cb = S.t * TILE + S.w * WCOLS;
      const int col = cb + lane;
      const float bval = (wave == 0 && col < P.V) ? bl[col] : -INFINITY;
      const float bias = chunk_bias<WT, KS>(W2, P.V, P.r, cb, w1s, part);
      if (wave == 0) {
        const float ec = exp2_scaled((bval - S.mt) + bias, sc);
        const int c = wave_pick64(ec, S.scale, S.rem);
        const float ex = __shfl(ec, c);
        if (lane == 0) {
          const int x = min(cb + c, P.V - 1);
          P.tokens[ev] = x;
          P.probs[ev] = (float)((double)ex * S.scale / S.Z);
          P.stats[2 * ev] = S.M;
          P.stats[2 * ev + 1] = (float)S.Z;
          if (!(S.Z > 0.0) || is_bad(S.M)) raise_err(P.err, DSPARK_DERR_NONFINITE);
          s_x = x;
        }
      }
    }
    if (k < P.gamma) store_base(Bs[k & 1], nxt);
    __syncthreads();  // s_x, the next base row, w1s, A_row and the selection's LDS are reused by the next step
  }
}

bool draft_fused_supported(int R, int gamma, int V, int r, float T);
int draft_fused_launch(const float* base, const void* W1, const void* W2, const int32_t* anchor,
                       const float* u_draft, int R, int gamma, int V, int r, float T, int32_t* tokens,
                       float* probs, float* stats, const DraftWs& dw, hipStream_t stream);

// DSPARK_DRAFT_KERNEL=stepwise selects the per-step kernels below even where
// the one-launch draft (draft_fused.hip) applies; both compute the same draw.
static bool stepwise_requested() {
  const char* e = getenv("DSPARK_DRAFT_KERNEL");
  return e != nullptr && strcmp(e, "stepwise") == 0;
}

template <typename WT>
static int launch_draft(const float* base, const void* W1, const void* W2, const int32_t* anchor,
                        const float* u_draft, int R, int gamma, int V, int r, float T,
                        int32_t* tokens, float* probs, float* stats, const DraftWs& dw, hipStream_t stream,
                        const RnnHead* rnn = nullptr) {
  if (std::is_same<WT, uint16_t>::value && rnn == nullptr && !stepwise_requested() &&
      draft_fused_supported(R, gamma, V, r, T))
    return draft_fused_launch(base, W1, W2, anchor, u_draft, R, gamma, V, r, T, tokens, probs, stats, dw,
                              stream);
  const bool rows = rnn == nullptr && !stepwise_requested() && draft_rows_fits<WT>(R, gamma, V, r);
  DraftStep<WT> P;
  P.base = base;
  P.W1 = static_cast<const WT*>(rnn ? rnn->states : W1);
  P.dense = rnn != nullptr;
  P.a_rows = rnn ? R * gamma : V;
  P.W2 = static_cast<const WT*>(W2);
  P.anchor = anchor;
  P.u_draft = u_draft;
  P.R = R; P.gamma = gamma; P.V = V; P.r = r;
  P.T = T;
  P.invT = (T > 0.f) ? 1.0f / T : 0.f;
  P.tokens = tokens; P.probs = probs; P.stats = stats;
  P.trec = dw.trec;
  P.err = dw.err;
  if (rows) {
    P.k = 1;
    prof_before(DSPARK_KID_DRAFT_ROWS, stream);
    for (int rep = prof_repeat(DSPARK_KID_DRAFT_ROWS); rep > 0; rep--) {
      DSPARK_DISPATCH_KS(r, {
        if (T == 0.f)
          hipLaunchKernelGGL((k_draft_rows<WT, true, KS>), dim3(R), dim3(256), 0, stream, P);
        else
          hipLaunchKernelGGL((k_draft_rows<WT, false, KS>), dim3(R), dim3(256), 0, stream, P);
      });
    }
    prof_after(DSPARK_KID_DRAFT_ROWS, stream);
    return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
  }
  const int nt = ceil_div(V, TILE);
  const int grid1 = min(nt, device_cu_count());
  for (int k = 1; k <= gamma; k++) {
    P.k = k;
    if (rnn) launch_rnn_state<WT>(*rnn, static_cast<const WT*>(W1), anchor, tokens, R, gamma, V, r, k, P.err, stream);
    prof_before(DSPARK_KID_DRAFT_PARTIALS, stream);
    for (int rep = prof_repeat(DSPARK_KID_DRAFT_PARTIALS); rep > 0; rep--) {
      DSPARK_DISPATCH_KS(r, {
        if (T == 0.f)
          hipLaunchKernelGGL((k_draft_partials<WT, true, KS>), dim3(grid1), dim3(256), 0, stream, P);
        else
          hipLaunchKernelGGL((k_draft_partials<WT, false, KS>), dim3(grid1), dim3(256), 0, stream, P);
      });
    }
    prof_after(DSPARK_KID_DRAFT_PARTIALS, stream);
    prof_before(DSPARK_KID_DRAFT_SELECT, stream);
    for (int rep = prof_repeat(DSPARK_KID_DRAFT_SELECT); rep > 0; rep--) {
      DSPARK_DISPATCH_KS(r, {
        if (T == 0.f)
          hipLaunchKernelGGL((k_draft_select<WT, true, 1>), dim3(R), dim3(256), 0, stream, P);
        else
          hipLaunchKernelGGL((k_draft_select<WT, false, KS>), dim3(R), dim3(256), 0, stream, P);
      });
    }
    prof_after(DSPARK_KID_DRAFT_SELECT, stream);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int draft_impl(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
               const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r, float T,
               int32_t* tokens, float* probs, float* stats, const DraftWs& dw, hipStream_t stream,
               const RnnHead* rnn = nullptr) {
  if (w_type == DSPARK_W_BF16)
    return launch_draft<uint16_t>(base, W1, W2, anchor, u_draft, R, gamma, V, r, T, tokens, probs,
                                  stats, dw, stream, rnn);
  return launch_draft<float>(base, W1, W2, anchor, u_draft, R, gamma, V, r, T, tokens, probs, stats,
                             dw, stream, rnn);
}

}  // namespace dspark
