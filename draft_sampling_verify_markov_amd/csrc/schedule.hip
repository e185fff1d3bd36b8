// Hardware-aware prefix scheduler (dspark_schedule).
//
// Sources: "DSpark: Aceleração da inferência de LLM com speculative decoding"
// (pt.news.hada.io), "Arquitetura" > Hardware-Aware Prefix Scheduler: the
// verify length is chosen to maximise global throughput Theta = tau * SPS(B)
// with a cost table SPS(B) profiled once; survival probabilities a_{r,j} are
// non-increasing in j, so a global sort with greedy admission respects each
// block's prefix; the walk stops as soon as throughput drops, so admission
// depends only on confidences (non-anticipation).  "DeepSpec ... DSpark"
// (jdon.com): one global candidate pool sorted high to low, each admitted
// token grows the verify batch by one.
//
// One workgroup of 1024 threads; the pool is padded to NS = 1024 * KPT slots
// and slot i = t + 1024 m lives in register m of thread t throughout:
//   1. a[r,j] = fp32 running product of c[r,0..j]           (one thread per request)
//   2. 64-bit keys (~bits(a) << 32 | r*gamma + j), bitonic sort ascending
//      -> a descending, flat index ascending on ties.  Exchange distances
//      below 64 use wave shuffles, 64..1023 a double-buffered LDS exchange
//      (one barrier per stage), 1024 and up stay inside a thread.
//   3. exact int64 prefix of floor(a * 2^36) in slot order (wave scans plus
//      per-wave totals): T_n = R * 2^36 + sum of the first n  (expected
//      emitted tokens)
//   4. Theta_n = double(T_n) * double(SPS(R + n)); n* = first strict drop
//   5. verify_len[r] = admitted candidates of row r (LDS counters)
#include "common.h"

namespace dspark {

constexpr int SCHED_THREADS = 1024;
constexpr int FIX_SHIFT = 36;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ long long shfl_up_i64(long long v, int d) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __shfl_up((uint32_t)u, d), hi = __shfl_up((uint32_t)(u >> 32), d);
  return (long long)(((uint64_t)hi << 32) | lo);
}

template <int KPT>
__global__ __launch_bounds__(SCHED_THREADS) void k_schedule(const float* __restrict__ conf,
                                                           const float* __restrict__ sps, int R,
                                                           int gamma, int n_table,
                                                           int32_t* __restrict__ verify_len,
                                                           int32_t* __restrict__ n_admitted,
                                                           float* __restrict__ cum_conf,
                                                           int32_t* err) {
  constexpr int NT = SCHED_THREADS, NS = NT * KPT;
  __shared__ uint64_t bufs[2][NS];
  __shared__ long long wsum[NT / 64];
  __shared__ int s_nstar;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = R * gamma;

  // 1. survival probabilities and sort keys (slot = flat index).  The
  // confidences are first read in parallel (coalesced) into LDS.
  float* cl = reinterpret_cast<float*>(&bufs[1][0]);
  for (int f = tid; f < n; f += NT) {
    float c = conf[f];
    if (!(c > 0.f && c <= 1.f)) {
      raise_err(err, DSPARK_DERR_CONF);
      c = (c > 1.f) ? 1.f : 0.f;  // NaN and non-positive values count as 0
    }
    cl[f] = c;
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) {
    float a = 1.0f;
    for (int j = 0; j < gamma; j++) {
      const int f = r * gamma + j;
      a = (j == 0) ? cl[f] : __fmul_rn(a, cl[f]);
      if (cum_conf) cum_conf[f] = a;
      bufs[0][f] = ((uint64_t)(~__float_as_uint(a)) << 32) | (uint32_t)f;
    }
  }
  for (int i = n + tid; i < NS; i += NT) bufs[0][i] = ~0ull;
  if (tid == 0) s_nstar = n;
  __syncthreads();
  uint64_t k[KPT];
#pragma unroll
  for (int m = 0; m < KPT; m++) k[m] = bufs[0][tid + NT * m];

  // 2. bitonic sort over slots
  int nb = 1;  // next exchange buffer (bufs[0] is still being read above)
  for (int kk = 2; kk <= NS; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj >= NT) {
        const int mj = jj / NT;
#pragma unroll
        for (int m = 0; m < KPT; m++) {
          if ((m & mj) == 0) {
            const int m2 = m | mj;
            const bool up = ((tid + NT * m) & kk) == 0;
            const uint64_t x = k[m], y = k[m2];
            if ((x > y) == up) {
              k[m] = y;
              k[m2] = x;
            }
          }
        }
      } else if (jj >= 64) {
        uint64_t* B = bufs[nb];
        nb ^= 1;
#pragma unroll
        for (int m = 0; m < KPT; m++) B[tid + NT * m] = k[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < KPT; m++) {
          const int i = tid + NT * m, pi = i ^ jj;
          const uint64_t y = B[pi];
          const bool up = (i & kk) == 0, lower = i < pi;
          k[m] = (lower == up) ? (k[m] < y ? k[m] : y) : (k[m] > y ? k[m] : y);
        }
      } else {
#pragma unroll
        for (int m = 0; m < KPT; m++) {
          const int i = tid + NT * m;
          const uint64_t y = shfl_xor_u64(k[m], jj);
          const bool up = (i & kk) == 0, lower = (lane & jj) == 0;
          k[m] = (lower == up) ? (k[m] < y ? k[m] : y) : (k[m] > y ? k[m] : y);
        }
      }
    }
  }

  // 3./4. exclusive fixed-point prefix in slot order and the drop test of
  // each slot (T_n before slot n, T_n + v after it)
  auto fixv = [&](int m) -> long long {
    const int i = tid + NT * m;
    const float a = __uint_as_float(~(uint32_t)(k[m] >> 32));
    return (i < n) ? (long long)floor((double)a * (double)(1LL << FIX_SHIFT)) : 0;
  };
  long long carry = 0;
  int drop = n;
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const long long vm = fixv(m);
    long long incl = vm;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = shfl_up_i64(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    long long before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) {
      const long long x = wsum[w];
      if (w < wave) before += x;
      total += x;
    }
    const int i = tid + NT * m;
    if (i < n) {
      const long long Tn = ((long long)R << FIX_SHIFT) + carry + before + (incl - vm);
      const long long Tn1 = Tn + vm;
      const int B0 = R + i, B1 = R + i + 1;
      const double S0 = (B0 <= n_table) ? (double)sps[B0 - 1] : 0.0;
      const double S1 = (B1 <= n_table) ? (double)sps[B1 - 1] : 0.0;
      if ((double)Tn1 * S1 < (double)Tn * S0) drop = min(drop, i);
    }
    carry += total;
    __syncthreads();  // wsum is rewritten for the next m
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) drop = min(drop, __shfl_xor(drop, o));
  if (lane == 0 && drop < n) atomicMin(&s_nstar, drop);
  int* cnt = reinterpret_cast<int*>(&bufs[0][0]);  // keys live in registers now
  for (int r = tid; r < R; r += NT) cnt[r] = 0;
  __syncthreads();
  const int nstar = s_nstar;

  // 5. per-request verify lengths
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const int i = tid + NT * m;
    if (i < nstar) atomicAdd(&cnt[(uint32_t)k[m] / gamma], 1);
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) verify_len[r] = cnt[r];
  if (tid == 0) *n_admitted = nstar;
}

int schedule_impl(const float* conf, const float* sps, int R, int gamma, int n_table,
                  int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                  hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, 8);
  const int n = R * gamma;
  int32_t* err = ws_ptr<int32_t>(ws, L.err);
  prof_before(DSPARK_KID_SCHEDULE, stream);
  for (int rep = prof_repeat(DSPARK_KID_SCHEDULE); rep > 0; rep--) {
    if (n <= SCHED_THREADS)
      hipLaunchKernelGGL(k_schedule<1>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma, n_table,
                         verify_len, n_admitted, cum_conf, err);
    else if (n <= 2 * SCHED_THREADS)
      hipLaunchKernelGGL(k_schedule<2>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma, n_table,
                         verify_len, n_admitted, cum_conf, err);
    else if (n <= 4 * SCHED_THREADS)
      hipLaunchKernelGGL(k_schedule<4>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma, n_table,
                         verify_len, n_admitted, cum_conf, err);
    else
      hipLaunchKernelGGL(k_schedule<8>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma, n_table,
                         verify_len, n_admitted, cum_conf, err);
  }
  prof_after(DSPARK_KID_SCHEDULE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

}  // namespace dspark
