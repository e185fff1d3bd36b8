// Sequential temperature scaling of the confidence head (dspark_sts_fit,
// dspark_sts_apply).
//
// Source: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), "Arquitetura" > Confidence-Scheduled Verification: the
// head outputs c_k = sigmoid(linear(h_k)); each c_k is a conditional
// probability, so the survival estimate of a prefix is the cumulative product
// of the c's; post-hoc calibration (Sequential Temperature Scaling) runs a 1-D
// grid search position by position, left to right, on a held-out set, and
// keeps the temperature that minimises the ECE of that product.
// "Análise dos experimentos": the head is over-confident before calibration
// and the calibrated survival estimates are what the scheduler consumes.
//
// Calibration map: c' = sigmoid(logit(c) / tau_k), logit(c) = log c - log1p(-c)
// (c = 0 and 1 are fixed points).  Score of candidate g at position k:
//   ECE_g = sum_b |sum_{i in b} (a'_i - y_i)| / N,   b = min(floor(a'_i * bins), bins - 1)
//   a'_i = A_i * c'_{i,k}   (A_i = product of the already-calibrated c'_{i,j<k})
//   y_i  = Y_i * l_{i,k}    (Y_i = product of the conditional labels l_{i,j<k})
// tau_k = grid[first minimiser], then A and Y advance by position k.
//
// Per position three launches:
//   k_sts_bins     grid (N / 1024, G / 16), 256 threads: thread (g, lane) owns
//                  one grid value and one sample lane; samples are staged 256 at
//                  a time in LDS (logit, A, y as fp64) and every thread folds
//                  16 of them (four at a time) into its own LDS bin column with ds_add_u64 of a
//                  2^-40 fixed-point difference (exact, order-independent
//                  sums, so the score and the arg-min are deterministic);
//                  per-(chunk, g, bin) sums go to the workspace.
//   k_sts_score    one wave per grid value: bin sums over chunks, |.|, total.
//   k_sts_advance  one workgroup per 256 samples: first arg-min of the scores
//                  (every workgroup reduces the G scores itself), outputs,
//                  then A *= c'(tau_k), Y *= l_k.
// The arithmetic is fp64 throughout (the scores feed an arg-min).
#include "common.h"

namespace dspark {

constexpr int STS_CHUNK = 1024;  // samples per workgroup of k_sts_bins
constexpr int STS_GPW = 16;      // grid values per workgroup
constexpr int STS_SUB = 256;     // samples staged in LDS at a time
constexpr int STS_LANES = 256 / STS_GPW;
constexpr int STS_ILP = 4;       // samples per thread per step of k_sts_bins

struct StsLayout {
  size_t err, A, Y, table, part, total;
};

inline StsLayout sts_layout(int N, int gamma, int G, int bins) {
  StsLayout L;
  const size_t nchunk = (size_t)ceil_div(N, STS_CHUNK);
  size_t o = 0;
  L.err = o;    o = ws_align(o + 256);
  L.A = o;      o = ws_align(o + (size_t)N * 8);
  L.Y = o;      o = ws_align(o + (size_t)N * 8);
  L.table = o;  o = ws_align(o + (size_t)gamma * G * 8);
  L.part = o;   o = ws_align(o + nchunk * G * bins * 8);
  L.total = o;
  return L;
}

struct StsArgs {
  const float* conf;    // [N, gamma]
  const float* labels;  // [N, gamma]
  const float* grid;    // [G]
  int N, gamma, G, bins, nchunk;
  double* A;            // [N]
  double* Y;            // [N]
  double* table;        // [gamma, G] (workspace)
  long long* part;      // [nchunk, G, bins]
  float* tau_out;       // [gamma]
  int32_t* idx_out;     // [gamma] or null
  double* ece_out;      // [gamma]
  double* table_out;    // [gamma, G] or null
  int32_t* err;
};

// A value in [0, 1]; NaN and out-of-range values are clamped and flagged.
__device__ __forceinline__ double unit_in(float v, int32_t* err) {
  if (v >= 0.f && v <= 1.f) return (double)v;
  if (err) raise_err(err, DSPARK_DERR_CALIB);
  return v > 1.f ? 1.0 : 0.0;
}
__device__ __forceinline__ bool tau_ok(float t) { return t > 0.f && !__builtin_isinf(t); }
__device__ __forceinline__ double logit_of(double c) { return log(c) - log1p(-c); }
// c' for a logit and the reciprocal temperature (the one expression every
// kernel of this file uses, so fit, advance and apply agree bit for bit).
__device__ __forceinline__ double calibrated(double ell, double inv_tau) {
  return 1.0 / (1.0 + exp(-(ell * inv_tau)));
}

__global__ void k_sts_init(StsArgs P) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < P.N) {
    P.A[i] = 1.0;
    P.Y[i] = 1.0;
  }
}

template <int MAXB>
__global__ __launch_bounds__(256) void k_sts_bins(StsArgs P, int k) {
  __shared__ unsigned long long s_bins[MAXB * 256];
  __shared__ double s_l[STS_SUB], s_a[STS_SUB], s_y[STS_SUB];
  const int t = threadIdx.x, gl = t % STS_GPW, lane = t / STS_GPW;
  const int g = blockIdx.y * STS_GPW + gl;
  const int i0 = blockIdx.x * STS_CHUNK, i1 = min(P.N, i0 + STS_CHUNK);
  const int nb = P.bins;
  for (int b = 0; b < nb; b++) s_bins[b * 256 + t] = 0ull;
  bool gok = false;
  double inv = 0.0;
  if (g < P.G) {
    const float tau = P.grid[g];
    gok = tau_ok(tau);
    inv = gok ? 1.0 / (double)tau : 0.0;
  }
  const double fb = (double)nb;
  for (int s0 = i0; s0 < i1; s0 += STS_SUB) {
    const int n = min(STS_SUB, i1 - s0);
    __syncthreads();  // the previous sub-chunk is consumed
    if (t < n) {
      const size_t e = (size_t)(s0 + t) * P.gamma + k;
      s_l[t] = logit_of(unit_in(P.conf[e], P.err));
      s_a[t] = P.A[s0 + t];
      s_y[t] = P.Y[s0 + t] * unit_in(P.labels[e], P.err);
    }
    __syncthreads();
    if (gok) {
      // four independent samples per step (j0 + 16u): four exp/divide chains
      // in flight per thread; past the sub-chunk's end a slot recomputes the
      // last sample and adds nothing
      for (int j0 = lane; j0 < n; j0 += STS_ILP * STS_LANES) {
        double ah[STS_ILP], ys[STS_ILP];
#pragma unroll
        for (int u = 0; u < STS_ILP; u++) {
          const int j = min(j0 + u * STS_LANES, n - 1);
          ah[u] = s_a[j] * calibrated(s_l[j], inv);
          ys[u] = s_y[j];
        }
#pragma unroll
        for (int u = 0; u < STS_ILP; u++) {
          int b = (int)(ah[u] * fb);
          b = min(max(b, 0), nb - 1);
          const long long q = (long long)rint((ah[u] - ys[u]) * 0x1p40);
          // branch-free: a slot past the end adds 0
          atomicAdd(&s_bins[b * 256 + t], (unsigned long long)(j0 + u * STS_LANES < n ? q : 0ll));
        }
      }
    }
  }
  __syncthreads();
  for (int e = t; e < STS_GPW * nb; e += 256) {
    const int gl2 = e % STS_GPW, b = e / STS_GPW, g2 = blockIdx.y * STS_GPW + gl2;
    if (g2 < P.G) {
      unsigned long long s = 0ull;
      for (int ln = 0; ln < STS_LANES; ln++) s += s_bins[b * 256 + ln * STS_GPW + gl2];
      P.part[((size_t)blockIdx.x * P.G + g2) * nb + b] = (long long)s;
    }
  }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64s(unsigned long long v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

__global__ __launch_bounds__(64) void k_sts_score(StsArgs P, int k) {
  const int g = blockIdx.x, lane = threadIdx.x;
  long long s = 0;
  if (lane < P.bins) {
    // eight independent partial sums keep eight loads in flight
    long long p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const long long* src = P.part + (size_t)g * P.bins + lane;
    const size_t stride = (size_t)P.G * P.bins;
    int c = 0;
    for (; c + 8 <= P.nchunk; c += 8)
#pragma unroll
      for (int u = 0; u < 8; u++) p[u] += src[(size_t)(c + u) * stride];
    for (; c < P.nchunk; c++) p[0] += src[(size_t)c * stride];
    s = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  }
  unsigned long long a = (unsigned long long)(s < 0 ? -s : s);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a += shfl_xor_u64s(a, m);
  if (lane == 0) {
    double e = (double)a * 0x1p-40 / (double)P.N;
    if (!tau_ok(P.grid[g])) {
      e = INFINITY;
      raise_err(P.err, DSPARK_DERR_CALIB);
    }
    P.table[(size_t)k * P.G + g] = e;
    if (P.table_out) P.table_out[(size_t)k * P.G + g] = e;
  }
}

__global__ __launch_bounds__(256) void k_sts_advance(StsArgs P, int k) {
  __shared__ double s_v[256];
  __shared__ int s_i[256];
  const int t = threadIdx.x;
  const double* row = P.table + (size_t)k * P.G;
  double bv = INFINITY;
  int bi = 0x7fffffff;
  for (int g = t; g < P.G; g += 256) {
    const double v = row[g];
    if (v < bv || (v == bv && g < bi)) {
      bv = v;
      bi = g;
    }
  }
  s_v[t] = bv;
  s_i[t] = bi;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      const double v = s_v[t + w];
      const int i = s_i[t + w];
      if (v < s_v[t] || (v == s_v[t] && i < s_i[t])) {
        s_v[t] = v;
        s_i[t] = i;
      }
    }
    __syncthreads();
  }
  const int idx = s_i[0] < P.G ? s_i[0] : 0;  // scores are never NaN; kept in range regardless
  const float tau = P.grid[idx];
  if (blockIdx.x == 0 && t == 0) {
    P.tau_out[k] = tau;
    if (P.idx_out) P.idx_out[k] = idx;
    P.ece_out[k] = row[idx];
  }
  const int i = blockIdx.x * 256 + t;
  if (i < P.N) {
    const size_t e = (size_t)i * P.gamma + k;
    const double c = unit_in(P.conf[e], nullptr);
    // a grid of nothing but invalid temperatures leaves c unchanged
    const double cc = tau_ok(tau) ? calibrated(logit_of(c), 1.0 / (double)tau) : c;
    P.A[i] = P.A[i] * cc;
    P.Y[i] = P.Y[i] * unit_in(P.labels[e], nullptr);
  }
}

__global__ void k_sts_apply(const float* conf, const float* tau, int n, int gamma, float* out, int32_t* err) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int k = i % gamma;
  const double c = unit_in(conf[i], err);
  const float tk = tau[k];
  if (!tau_ok(tk)) {
    raise_err(err, DSPARK_DERR_CALIB);
    out[i] = (float)c;
    return;
  }
  out[i] = (float)calibrated(logit_of(c), 1.0 / (double)tk);
}

size_t sts_workspace_size_impl(int N, int gamma, int G, int bins) {
  return sts_layout(N, gamma, G, bins).total;
}

int sts_fit_impl(const float* conf, const float* labels, const float* grid, int N, int gamma, int G, int bins,
                 float* tau, int32_t* tau_index, double* ece, double* ece_table, void* ws, hipStream_t stream) {
  const StsLayout L = sts_layout(N, gamma, G, bins);
  StsArgs P{};
  P.conf = conf;
  P.labels = labels;
  P.grid = grid;
  P.N = N;
  P.gamma = gamma;
  P.G = G;
  P.bins = bins;
  P.nchunk = ceil_div(N, STS_CHUNK);
  char* w = static_cast<char*>(ws);
  P.err = reinterpret_cast<int32_t*>(w + L.err);
  P.A = reinterpret_cast<double*>(w + L.A);
  P.Y = reinterpret_cast<double*>(w + L.Y);
  P.table = reinterpret_cast<double*>(w + L.table);
  P.part = reinterpret_cast<long long*>(w + L.part);
  P.tau_out = tau;
  P.idx_out = tau_index;
  P.ece_out = ece;
  P.table_out = ece_table;
  const int nblk = ceil_div(N, 256);
  hipLaunchKernelGGL(k_sts_init, dim3(nblk), dim3(256), 0, stream, P);
  const dim3 gb((unsigned)P.nchunk, (unsigned)ceil_div(G, STS_GPW));
  for (int k = 0; k < gamma; k++) {
    if (bins <= 16)
      hipLaunchKernelGGL(k_sts_bins<16>, gb, dim3(256), 0, stream, P, k);
    else
      hipLaunchKernelGGL(k_sts_bins<DSPARK_STS_MAX_BINS>, gb, dim3(256), 0, stream, P, k);
    hipLaunchKernelGGL(k_sts_score, dim3(G), dim3(64), 0, stream, P, k);
    hipLaunchKernelGGL(k_sts_advance, dim3(nblk), dim3(256), 0, stream, P, k);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int sts_apply_impl(const float* conf, const float* tau, int R, int gamma, float* out, void* ws,
                   hipStream_t stream) {
  const int n = R * gamma;
  hipLaunchKernelGGL(k_sts_apply, dim3(ceil_div(n, 256)), dim3(256), 0, stream, conf, tau, n, gamma, out,
                     static_cast<int32_t*>(ws));
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

}  // namespace dspark
