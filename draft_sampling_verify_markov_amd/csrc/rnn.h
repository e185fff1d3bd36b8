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
// with the tile's weight columns and input rows staged in LDS: k_rnn_gates
// (update and reset gates, the candidate's input part, g * s) and
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

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __shfl_xor((uint32_t)u, m), hi = __shfl_xor((uint32_t)(u >> 32), m);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Tiling of the per-step gate products: a workgroup takes RNN_RB requests and
// RNN_UB consecutive state units; thread t = (request t / 16, input lane
// t % 16) sums the inputs i = 16 m + lane, and the 16 lanes of a request are
// combined by a fixed xor butterfly (deterministic; the 16 lanes of a request
// are consecutive lanes of one wave).
constexpr int RNN_RB = 16;
constexpr int RNN_UB = 8;
constexpr int RNN_LANES = 16;

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

// Update gate, reset gate and the candidate's input part for a tile of
// (requests, units); writes u, e.Wx[2] and g * s to the gate buffer.
template <typename WT>
__global__ __launch_bounds__(256) void k_rnn_gates(RnnStep<WT> P) {
  __shared__ float s_w[5][DSPARK_MAX_RANK][RNN_UB];           // Wx[0..2], Ws[0..1] columns of the tile
  // rows padded by 16 floats: the four requests of a wave read distinct banks
  __shared__ float s_e[RNN_RB][DSPARK_MAX_RANK + 16], s_s[RNN_RB][DSPARK_MAX_RANK + 16];
  const int t = threadIdx.x, rl = t / RNN_LANES, ln = t % RNN_LANES;
  const int u0 = blockIdx.x * RNN_UB, row0 = blockIdx.y * RNN_RB;
  const int r = P.r;
  const size_t rr = (size_t)r * r;
#pragma unroll
  for (int g = 0; g < 5; g++) {
    const WT* src = (g < 3 ? P.Wx + g * rr : P.Ws + (g - 3) * rr) + u0;
    for (int i = t; i < r; i += 256) {
      float w[8];
      load8(src + (size_t)i * r, w);
#pragma unroll
      for (int e = 0; e < 8; e++) s_w[g][i][e] = w[e];
    }
  }
  {
    // request q = t / 16 of the tile, r / 16 consecutive input units per thread
    const int q = t / RNN_LANES, per = r / RNN_LANES, i0 = (t % RNN_LANES) * per, row = row0 + q;
    const bool ok = row < P.R;
    int prev = 0;
    if (ok) prev = checked_token((P.k == 1) ? P.anchor[row] : P.tokens[(size_t)row * P.gamma + P.k - 2], P.V, P.err);
    const WT* erow = P.W1 + (size_t)prev * r + i0;
    const WT* srow = P.S + ((size_t)row * P.gamma + P.k - 2) * r + i0;
    for (int e = 0; e < per; e++) {
      s_e[q][i0 + e] = ok ? to_f32(erow[e]) : 0.f;
      s_s[q][i0 + e] = (ok && P.k > 1) ? to_f32(srow[e]) : 0.f;
    }
  }
  __syncthreads();
  double acc[5][RNN_UB];
#pragma unroll
  for (int g = 0; g < 5; g++)
#pragma unroll
    for (int e = 0; e < RNN_UB; e++) acc[g][e] = 0.0;
  for (int i = ln; i < r; i += RNN_LANES) {
    const double ev = s_e[rl][i], sv = s_s[rl][i];
#pragma unroll
    for (int g = 0; g < 5; g++) {
      const double x = g < 3 ? ev : sv;
#pragma unroll
      for (int e = 0; e < RNN_UB; e++) acc[g][e] += x * (double)s_w[g][i][e];
    }
  }
#pragma unroll
  for (int m = RNN_LANES / 2; m >= 1; m >>= 1)
#pragma unroll
    for (int g = 0; g < 5; g++)
#pragma unroll
      for (int e = 0; e < RNN_UB; e++) acc[g][e] += shfl_xor_f64(acc[g][e], m);
  // lane ln < 8 finishes unit u0 + ln of its request
  const int row = row0 + rl, j = u0 + ln;
  if (ln < RNN_UB && row < P.R) {
    double p[5];
#pragma unroll
    for (int g = 0; g < 5; g++) {
      double v = acc[g][0];
#pragma unroll
      for (int e = 1; e < RNN_UB; e++) v = (ln == e) ? acc[g][e] : v;
      p[g] = v;
    }
    const double u = 1.0 / (1.0 + exp(-((p[0] + p[3]) + (double)P.bias[j])));
    const double gr = 1.0 / (1.0 + exp(-((p[1] + p[4]) + (double)P.bias[r + j])));
    const size_t o = (size_t)row * r + j, plane = (size_t)P.R * r;
    P.gates[o] = u;
    P.gates[plane + o] = p[2];
    P.gates[2 * plane + o] = gr * (double)s_s[rl][j];
  }
}

// Candidate h = tanh(e.Wx[2] + (g * s).Ws[2] + b[2]) and the new state.
template <typename WT>
__global__ __launch_bounds__(256) void k_rnn_update(RnnStep<WT> P) {
  __shared__ float s_w[DSPARK_MAX_RANK][RNN_UB];
  __shared__ double s_gs[RNN_RB][DSPARK_MAX_RANK];
  const int t = threadIdx.x, rl = t / RNN_LANES, ln = t % RNN_LANES;
  const int u0 = blockIdx.x * RNN_UB, row0 = blockIdx.y * RNN_RB;
  const int r = P.r;
  const size_t rr = (size_t)r * r, plane = (size_t)P.R * r;
  for (int i = t; i < r; i += 256) {
    float w[8];
    load8(P.Ws + 2 * rr + (size_t)i * r + u0, w);
#pragma unroll
    for (int e = 0; e < 8; e++) s_w[i][e] = w[e];
  }
  {
    const int q = t / RNN_LANES, per = r / RNN_LANES, i0 = (t % RNN_LANES) * per, row = row0 + q;
    const double* src = P.gates + 2 * plane + (size_t)row * r + i0;
    for (int e = 0; e < per; e++) s_gs[q][i0 + e] = (row < P.R) ? src[e] : 0.0;
  }
  __syncthreads();
  double acc[RNN_UB];
#pragma unroll
  for (int e = 0; e < RNN_UB; e++) acc[e] = 0.0;
  for (int i = ln; i < r; i += RNN_LANES) {
    const double gv = s_gs[rl][i];
#pragma unroll
    for (int e = 0; e < RNN_UB; e++) acc[e] += gv * (double)s_w[i][e];
  }
#pragma unroll
  for (int m = RNN_LANES / 2; m >= 1; m >>= 1)
#pragma unroll
    for (int e = 0; e < RNN_UB; e++) acc[e] += shfl_xor_f64(acc[e], m);
  const int row = row0 + rl, j = u0 + ln;
  if (ln < RNN_UB && row < P.R) {
    double hs = acc[0];
#pragma unroll
    for (int e = 1; e < RNN_UB; e++) hs = (ln == e) ? acc[e] : hs;
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
  hipLaunchKernelGGL(k_rnn_gates<WT>, grid, dim3(256), 0, stream, P);
  hipLaunchKernelGGL(k_rnn_update<WT>, grid, dim3(256), 0, stream, P);
}

}  // namespace dspark
