// RNN head: the gated recurrent state of the sequential stage.
//
// Source: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), "Arquitetura" > Semi-Autoregressive Generation, RNN head:
// a recurrent state s_k accumulates the whole in-block prefix with a gated
// update, so the bias can use tokens before the immediately previous one;
// "Experimentos": it adds a small gain at long blocks, and the Markov head is
// the default.  The pages give no equations; the update is the GRU form:
//   e = W1[x_{k-1}] (x_0 = anchor), s_0 = 0
//   u = sigmoid(e Wx[0] + s Ws[0] + b[0]),  g = sigmoid(e Wx[1] + s Ws[1] + b[1])
//   h = tanh(e Wx[2] + (g * s) Ws[2] + b[2]),  s_k = (1 - u) * s + u * h
// and the transition bias at position k is s_k . W2.  s_k is stored in the
// weights' type, rounded once from fp64 (nearest, ties to even), and
// feeds the same bias contraction as a gathered W1 row.  The gate arithmetic
// is fp64: products of stored values are exact there, so the stored state is
// reproducible to the last bit (6 r^2 multiply-adds per request and step).
//
// Per draft step two launches, each tiled over (16 requests x 8 state units)
// with the tile's weight columns and input rows staged in LDS as fp64:
// k_rnn_gates (update and reset gates, the candidate's input part, g * s) and
// k_rnn_update (the candidate's recurrent part, which needs g * s of every
// unit, and the new state).
#pragma once
#include "common.h"

namespace dspark {

__device__ __forceinline__ double w_to_f64(float x) { return (double)x; }
__device__ __forceinline__ double w_to_f64(uint16_t b) { return (double)__uint_as_float((uint32_t)b << 16); }

template <typename WT>
__device__ __forceinline__ WT store_state(double x);
template <>
__device__ __forceinline__ float store_state<float>(double x) {
  return (float)x;
}
// One rounding from fp64 to bf16, nearest with ties to even: the fp64
// significand is cut to bf16's 8 significant bits, then the value (now exact
// in fp32) is narrowed.  Below 2^-126 (bf16 subnormals) the spacing is
// 2^-133, so the value is rounded on that grid instead (exact scalings).
// |x| <= 1 here, so nothing overflows.
template <>
__device__ __forceinline__ uint16_t store_state<uint16_t>(double x) {
  double q;
  if (fabs(x) < 0x1p-126) {
    q = rint(x * 0x1p133) * 0x1p-133;
  } else {
    uint64_t u = __builtin_bit_cast(uint64_t, x);
    constexpr uint64_t DROP = (1ull << 45) - 1;  // 52 - 7 significand bits go
    u += (DROP >> 1) + ((u >> 45) & 1ull);
    q = __builtin_bit_cast(double, u & ~DROP);
  }
  return (uint16_t)(__float_as_uint((float)q) >> 16);
}

// Eight consecutive weights of one row of a gate matrix (one or two 16-byte
// loads), widened exactly to fp32.
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, float (&w)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; e++) {
    w[2 * e] = __uint_as_float(x[e] << 16);
    w[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* __restrict__ p, float (&w)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Tiling of the per-step gate products: a workgroup of RNN_W waves takes
// RNN_RB requests and RNN_UB consecutive state units, with the tile's weight
// columns and its requests' input rows staged in LDS as fp64 (exact
// widenings, converted once).  Wave w sums the inputs [w r / RNN_W,
// (w + 1) r / RNN_W) in order; lane l owns unit l % 8 and requests 2 (l / 8),
// 2 (l / 8) + 1: ten fp64 sums in the gates kernel (five gate products, two
// requests), two in the update kernel.  The waves' partial sums are then
// added in a fixed pairwise order, ((w0 + w1) + (w2 + w3)) + ((w4 + w5) +
// (w6 + w7)): deterministic, and no lane shuffles.  Two waves per SIMD and
// an unrolled input loop keep LDS reads in flight behind the fp64 FMAs.
constexpr int RNN_RB = 16;
constexpr int RNN_UB = 8;
constexpr int RNN_W = 8;
constexpr int RNN_T = 64 * RNN_W;
constexpr int RNN_XPAD = 2;  // row padding of the staged inputs (conflict-free reads)

template <typename WT>
struct RnnStep {
  const WT* W1;
  const WT* Wx;
  const WT* Ws;
  const float* bias;
  const int32_t* anchor;
  const int32_t* tokens;
  WT* S;            // state table [R][gamma][r]
  double* gates;    // [3][R][r]
  int R, gamma, V, r, k;
  int32_t* err;
};

// Staging of a request block's input rows into LDS as fp64, in pieces of 8
// consecutive values: piece p = thread + RNN_T m is row p / (r / 8), values
// [8 (p % (r / 8)), + 8).  Every global load of a thread is issued before the
// first LDS store, so the staging costs one memory latency, not one per value.
constexpr int RNN_PIECES = RNN_RB * DSPARK_MAX_RANK / 8 / RNN_T;  // per thread, at most
__device__ __forceinline__ void piece_of(int m, int r, int& q, int& c) {
  const int idx = threadIdx.x + RNN_T * m, per_row = r / 8;
  q = idx / per_row;
  c = idx - q * per_row;
}

// Sum of the RNN_W partial sums x[w * stride], w = 0..7, in the fixed order.
__device__ __forceinline__ double wave_sum8(const double* x, int stride) {
  return ((x[0] + x[stride]) + (x[2 * stride] + x[3 * stride])) +
         ((x[4 * stride] + x[5 * stride]) + (x[6 * stride] + x[7 * stride]));
}

// Update gate, reset gate and the candidate's input part for a tile of
// (requests, units); writes u, e.Wx[2] and g * s to the gate buffer.
template <typename WT>
__global__ __launch_bounds__(RNN_T) void k_rnn_gates(RnnStep<WT> P) {
  __shared__ double s_w[5][DSPARK_MAX_RANK][RNN_UB];  // Wx[0..2], Ws[0..1] columns of the tile
  // e rows, then s rows; after the products the partial sums reuse this space
  __shared__ double s_x[2][RNN_RB][DSPARK_MAX_RANK + RNN_XPAD];
  const int t = threadIdx.x;
  const int u0 = blockIdx.x * RNN_UB, row0 = blockIdx.y * RNN_RB;
  const int r = P.r;
  const size_t rr = (size_t)r * r;
  {
    // every global load first: weight pieces of input row t % 256 (gates 0-2
    // by the first 256 threads, 3-4 by the others), the previous tokens of
    // this thread's input pieces, then their W1 and state rows
    const int wi = t & 255, g0 = t < 256 ? 0 : 3, ng = t < 256 ? 3 : 2;
    float w[3][8];
    if (wi < r)
#pragma unroll
      for (int gg = 0; gg < 3; gg++)
        if (gg < ng) {
          const int g = g0 + gg;
          load8((g < 3 ? P.Wx + g * rr : P.Ws + (g - 3) * rr) + u0 + (size_t)wi * r, w[gg]);
        }
    int prev[RNN_PIECES];
#pragma unroll
    for (int m = 0; m < RNN_PIECES; m++) {
      int q, c;
      piece_of(m, r, q, c);
      const int row = row0 + q;
      prev[m] = -1;
      if (q < RNN_RB && row < P.R)
        prev[m] = (P.k == 1) ? P.anchor[row] : P.tokens[(size_t)row * P.gamma + P.k - 2];
    }
    float ev[RNN_PIECES][8], sv8[RNN_PIECES][8];
#pragma unroll
    for (int m = 0; m < RNN_PIECES; m++) {
      int q, c;
      piece_of(m, r, q, c);
      const bool ok = prev[m] >= 0;
      const int tok = ok ? checked_token(prev[m], P.V, P.err) : 0;
#pragma unroll
      for (int e = 0; e < 8; e++) ev[m][e] = sv8[m][e] = 0.f;
      if (ok) load8(P.W1 + (size_t)tok * r + 8 * c, ev[m]);
      if (ok && P.k > 1) load8(P.S + ((size_t)(row0 + q) * P.gamma + P.k - 2) * r + 8 * c, sv8[m]);
    }
    if (wi < r)
#pragma unroll
      for (int gg = 0; gg < 3; gg++)
        if (gg < ng)
#pragma unroll
          for (int e = 0; e < 8; e++) s_w[g0 + gg][wi][e] = (double)w[gg][e];
#pragma unroll
    for (int m = 0; m < RNN_PIECES; m++) {
      int q, c;
      piece_of(m, r, q, c);
      if (q < RNN_RB)
#pragma unroll
        for (int e = 0; e < 8; e++) {
          s_x[0][q][8 * c + e] = (double)ev[m][e];
          s_x[1][q][8 * c + e] = (double)sv8[m][e];
        }
    }
  }
  __syncthreads();
  const int wave = t >> 6, l = t & 63, n = l & 7, mq = l >> 3;
  const int qa = 2 * mq, qb = qa + 1;
  double acc[5][2];
#pragma unroll
  for (int g = 0; g < 5; g++) acc[g][0] = acc[g][1] = 0.0;
  const int kw = r / RNN_W, i1 = (wave + 1) * kw;
#pragma unroll 4
  for (int i = wave * kw; i < i1; i++) {
    const double ea = s_x[0][qa][i], eb = s_x[0][qb][i];
    const double sa = s_x[1][qa][i], sb = s_x[1][qb][i];
#pragma unroll
    for (int g = 0; g < 5; g++) {
      const double w = s_w[g][i][n];
      acc[g][0] = fma(g < 3 ? ea : sa, w, acc[g][0]);  // the products are exact in fp64
      acc[g][1] = fma(g < 3 ? eb : sb, w, acc[g][1]);
    }
  }
  // output thread t < 128: request t / 8, unit u0 + t % 8; its s value is read
  // before the partial sums overwrite the staged rows
  const int oq = t >> 3, on = t & 7, j = u0 + on;
  const double sv = (t < RNN_RB * RNN_UB) ? s_x[1][oq][j] : 0.0;
  __syncthreads();
  double* red = &s_x[0][0][0];  // [wave][gate][request parity][lane]
#pragma unroll
  for (int g = 0; g < 5; g++)
#pragma unroll
    for (int q = 0; q < 2; q++) red[((wave * 5 + g) * 2 + q) * 64 + l] = acc[g][q];
  __syncthreads();
  const int row = row0 + oq;
  if (t < RNN_RB * RNN_UB && row < P.R) {
    const int ol = (oq >> 1) * 8 + on, op = oq & 1;
    double p[5];
#pragma unroll
    for (int g = 0; g < 5; g++) p[g] = wave_sum8(red + (g * 2 + op) * 64 + ol, 5 * 2 * 64);
    const double u = 1.0 / (1.0 + exp(-((p[0] + p[3]) + (double)P.bias[j])));
    const double gr = 1.0 / (1.0 + exp(-((p[1] + p[4]) + (double)P.bias[r + j])));
    const size_t o = (size_t)row * r + j, plane = (size_t)P.R * r;
    P.gates[o] = u;
    P.gates[plane + o] = p[2];
    P.gates[2 * plane + o] = gr * sv;
  }
}

// Candidate h = tanh(e.Wx[2] + (g * s).Ws[2] + b[2]) and the new state.
template <typename WT>
__global__ __launch_bounds__(RNN_T) void k_rnn_update(RnnStep<WT> P) {
  __shared__ double s_w[DSPARK_MAX_RANK][RNN_UB];
  __shared__ double s_gs[RNN_RB][DSPARK_MAX_RANK + RNN_XPAD];
  __shared__ double red[RNN_W][2][64];
  const int t = threadIdx.x;
  const int u0 = blockIdx.x * RNN_UB, row0 = blockIdx.y * RNN_RB;
  const int r = P.r;
  const size_t rr = (size_t)r * r, plane = (size_t)P.R * r;
  {
    // every global load first (weight piece of input row t, the g * s pieces)
    float w[8];
    if (t < r) load8(P.Ws + 2 * rr + (size_t)t * r + u0, w);
    double gv[RNN_PIECES][8];
#pragma unroll
    for (int m = 0; m < RNN_PIECES; m++) {
      int q, c;
      piece_of(m, r, q, c);
      const int row = row0 + q;
      const bool ok = q < RNN_RB && row < P.R;
      double4 a{0.0, 0.0, 0.0, 0.0}, b{0.0, 0.0, 0.0, 0.0};
      if (ok) {
        const double4* src = reinterpret_cast<const double4*>(P.gates + 2 * plane + (size_t)row * r + 8 * c);
        a = src[0];
        b = src[1];
      }
      gv[m][0] = a.x; gv[m][1] = a.y; gv[m][2] = a.z; gv[m][3] = a.w;
      gv[m][4] = b.x; gv[m][5] = b.y; gv[m][6] = b.z; gv[m][7] = b.w;
    }
    if (t < r)
#pragma unroll
      for (int e = 0; e < 8; e++) s_w[t][e] = (double)w[e];
#pragma unroll
    for (int m = 0; m < RNN_PIECES; m++) {
      int q, c;
      piece_of(m, r, q, c);
      if (q < RNN_RB)
#pragma unroll
        for (int e = 0; e < 8; e++) s_gs[q][8 * c + e] = gv[m][e];
    }
  }
  __syncthreads();
  const int wave = t >> 6, l = t & 63, n = l & 7, mq = l >> 3;
  const int qa = 2 * mq, qb = qa + 1;
  double acc0 = 0.0, acc1 = 0.0;
  const int kw = r / RNN_W, i1 = (wave + 1) * kw;
#pragma unroll 4
  for (int i = wave * kw; i < i1; i++) {
    const double w = s_w[i][n];
    acc0 = fma(s_gs[qa][i], w, acc0);
    acc1 = fma(s_gs[qb][i], w, acc1);
  }
  red[wave][0][l] = acc0;
  red[wave][1][l] = acc1;
  __syncthreads();
  const int oq = t >> 3, on = t & 7, row = row0 + oq, j = u0 + on;
  if (t < RNN_RB * RNN_UB && row < P.R) {
    const int ol = (oq >> 1) * 8 + on, op = oq & 1;
    const double hs = wave_sum8(&red[0][op][ol], 2 * 64);
    const size_t o = (size_t)row * r + j;
    const double u = P.gates[o];
    const double h = tanh((P.gates[plane + o] + hs) + (double)P.bias[2 * r + j]);
    const double sp = (P.k == 1) ? 0.0 : w_to_f64(P.S[((size_t)row * P.gamma + P.k - 2) * r + j]);
    P.S[((size_t)row * P.gamma + P.k - 1) * r + j] = store_state<WT>((1.0 - u) * sp + u * h);
  }
}

template <typename WT>
inline void launch_rnn_state(const RnnHead& h, const WT* W1, const int32_t* anchor, const int32_t* tokens, int R,
                             int gamma, int V, int r, int k, int32_t* err, hipStream_t stream) {
  RnnStep<WT> P;
  P.W1 = W1;
  P.Wx = static_cast<const WT*>(h.Wx);
  P.Ws = static_cast<const WT*>(h.Ws);
  P.bias = h.bias;
  P.anchor = anchor;
  P.tokens = tokens;
  P.S = static_cast<WT*>(h.states);
  P.gates = h.gates;
  P.R = R; P.gamma = gamma; P.V = V; P.r = r; P.k = k;
  P.err = err;
  const dim3 grid((unsigned)(r / RNN_UB), (unsigned)ceil_div(R, RNN_RB));
  hipLaunchKernelGGL(k_rnn_gates<WT>, grid, dim3(RNN_T), 0, stream, P);
  hipLaunchKernelGGL(k_rnn_update<WT>, grid, dim3(RNN_T), 0, stream, P);
}

}  // namespace dspark
