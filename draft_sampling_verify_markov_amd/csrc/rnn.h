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
// weights' type (fp32, then bf16 round-to-nearest-even for bf16 weights) and
// feeds the same bias contraction as a gathered W1 row.  The gate arithmetic
// is fp64: products of stored values are exact there, so the stored state is
// reproducible to the last bit (3 * 2 * r^2 multiply-adds per request and step).
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
template <>
__device__ __forceinline__ uint16_t store_state<uint16_t>(double x) {
  uint32_t u = __float_as_uint((float)x);
  u += 0x7FFFu + ((u >> 16) & 1u);  // |x| < 1: no overflow into the exponent's top
  return (uint16_t)(u >> 16);
}

// One workgroup per request, one thread per state unit (r <= 256).
template <typename WT>
__global__ __launch_bounds__(256) void k_rnn_state(const WT* __restrict__ W1, const WT* __restrict__ Wx,
                                                   const WT* __restrict__ Ws, const float* __restrict__ bias,
                                                   const int32_t* anchor, const int32_t* tokens, WT* S, int gamma,
                                                   int V, int r, int k, int32_t* err) {
  __shared__ double s_e[DSPARK_MAX_RANK], s_s[DSPARK_MAX_RANK], s_gs[DSPARK_MAX_RANK];
  const int row = blockIdx.x, j = threadIdx.x;
  const int t = (k == 1) ? anchor[row] : tokens[(size_t)row * gamma + k - 2];
  const int prev = checked_token(t, V, err);
  const size_t rr = (size_t)r * r;
  if (j < r) {
    s_e[j] = w_to_f64(W1[(size_t)prev * r + j]);
    s_s[j] = (k == 1) ? 0.0 : w_to_f64(S[((size_t)row * gamma + k - 2) * r + j]);
  }
  __syncthreads();
  double u = 0.0, hx = 0.0;
  if (j < r) {
    double ue = 0.0, ge = 0.0, he = 0.0, us = 0.0, gs = 0.0;
    for (int i = 0; i < r; i++) {
      const double e = s_e[i], sv = s_s[i];
      const size_t o = (size_t)i * r + j;
      ue += e * w_to_f64(Wx[o]);
      ge += e * w_to_f64(Wx[rr + o]);
      he += e * w_to_f64(Wx[2 * rr + o]);
      us += sv * w_to_f64(Ws[o]);
      gs += sv * w_to_f64(Ws[rr + o]);
    }
    u = 1.0 / (1.0 + exp(-((ue + us) + (double)bias[j])));
    const double g = 1.0 / (1.0 + exp(-((ge + gs) + (double)bias[r + j])));
    hx = he;
    s_gs[j] = g * s_s[j];
  }
  __syncthreads();
  if (j < r) {
    double hs = 0.0;
    for (int i = 0; i < r; i++) hs += s_gs[i] * w_to_f64(Ws[2 * rr + (size_t)i * r + j]);
    const double h = tanh((hx + hs) + (double)bias[2 * r + j]);
    S[((size_t)row * gamma + k - 1) * r + j] = store_state<WT>((1.0 - u) * s_s[j] + u * h);
  }
}

template <typename WT>
inline void launch_rnn_state(const RnnHead& h, const WT* W1, const int32_t* anchor, const int32_t* tokens, int R,
                             int gamma, int V, int r, int k, int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(k_rnn_state<WT>, dim3(R), dim3(256), 0, stream, W1, static_cast<const WT*>(h.Wx),
                     static_cast<const WT*>(h.Ws), h.bias, anchor, tokens, static_cast<WT*>(h.states), gamma, V, r,
                     k, err);
}

}  // namespace dspark
