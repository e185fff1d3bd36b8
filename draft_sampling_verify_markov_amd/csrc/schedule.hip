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
// One workgroup of 1024 threads:
//   1. a[r,j] = fp32 running product of c[r,0..j]           (one thread per request)
//   2. 64-bit keys (~bits(a) << 32 | r*gamma + j), bitonic sort in LDS
//      -> a descending, flat index ascending on ties
//   3. exact int64 prefix of floor(a * 2^36) over the sorted pool:
//      T_n = R * 2^36 + sum of the first n  (expected emitted tokens)
//   4. Theta_n = double(T_n) * double(SPS(R + n)); n* = first strict drop
//   5. verify_len[r] = admitted candidates of row r (LDS counters)
#include "common.h"

namespace dspark {

constexpr int SCHED_THREADS = 1024;
constexpr int FIX_SHIFT = 36;

__global__ __launch_bounds__(SCHED_THREADS) void k_schedule(const float* __restrict__ conf,
                                                           const float* __restrict__ sps, int R,
                                                           int gamma, int n_table,
                                                           int32_t* __restrict__ verify_len,
                                                           int32_t* __restrict__ n_admitted,
                                                           float* __restrict__ cum_conf,
                                                           int32_t* err) {
  __shared__ uint64_t keys[DSPARK_MAX_POOL];
  __shared__ int cnt[DSPARK_MAX_POOL];
  __shared__ long long scan_tmp[SCHED_THREADS];
  __shared__ int s_nstar;

  const int tid = threadIdx.x;
  const int n = R * gamma;
  int P2 = 1;
  while (P2 < n) P2 <<= 1;

  // 1. survival probabilities and sort keys
  for (int r = tid; r < R; r += SCHED_THREADS) {
    float a = 1.0f;
    for (int j = 0; j < gamma; j++) {
      const size_t f = (size_t)r * gamma + j;
      float c = conf[f];
      if (!(c > 0.f && c <= 1.f)) {
        raise_err(err, DSPARK_DERR_CONF);
        c = (c > 1.f) ? 1.f : 0.f;  // NaN and non-positive values count as 0
      }
      a = (j == 0) ? c : __fmul_rn(a, c);
      if (cum_conf) cum_conf[f] = a;
      keys[f] = ((uint64_t)(~__float_as_uint(a)) << 32) | (uint32_t)f;
    }
  }
  for (int i = n + tid; i < P2; i += SCHED_THREADS) keys[i] = ~0ull;
  __syncthreads();

  // 2. bitonic sort, ascending
  for (int k = 2; k <= P2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P2; i += SCHED_THREADS) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint64_t x = keys[i], y = keys[ixj];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }

  // 3. fixed-point prefix over the sorted pool; each thread owns a run
  const int per = ceil_div(n, SCHED_THREADS);
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  long long loc = 0;
  for (int i = i0; i < i1; i++) {
    const float a = __uint_as_float(~(uint32_t)(keys[i] >> 32));
    loc += (long long)floor((double)a * (double)(1LL << FIX_SHIFT));
  }
  // exclusive scan of the per-thread sums (exact integer arithmetic)
  scan_tmp[tid] = loc;
  __syncthreads();
  const long long shifted_v = (tid > 0) ? scan_tmp[tid - 1] : 0;
  __syncthreads();
  scan_tmp[tid] = shifted_v;
  __syncthreads();
  for (int o = 1; o < SCHED_THREADS; o <<= 1) {
    const long long add = (tid >= o) ? scan_tmp[tid - o] : 0;
    __syncthreads();
    scan_tmp[tid] += add;
    __syncthreads();
  }
  const long long excl = scan_tmp[tid];
  if (tid == 0) s_nstar = n;
  __syncthreads();

  // 4. objective and first drop
  long long Tn = ((long long)R << FIX_SHIFT) + excl;
  for (int i = i0; i < i1; i++) {
    const float a = __uint_as_float(~(uint32_t)(keys[i] >> 32));
    const long long Tn1 = Tn + (long long)floor((double)a * (double)(1LL << FIX_SHIFT));
    const int B0 = R + i, B1 = R + i + 1;
    const double S0 = (B0 <= n_table) ? (double)sps[B0 - 1] : 0.0;
    const double S1 = (B1 <= n_table) ? (double)sps[B1 - 1] : 0.0;
    const double th0 = (double)Tn * S0, th1 = (double)Tn1 * S1;
    if (th1 < th0) {
      atomicMin(&s_nstar, i);
      break;
    }
    Tn = Tn1;
  }
  for (int r = tid; r < R; r += SCHED_THREADS) cnt[r] = 0;
  __syncthreads();
  const int nstar = s_nstar;

  // 5. per-request verify lengths
  for (int i = i0; i < min(i1, nstar); i++) atomicAdd(&cnt[(uint32_t)keys[i] / gamma], 1);
  __syncthreads();
  for (int r = tid; r < R; r += SCHED_THREADS) verify_len[r] = cnt[r];
  if (tid == 0) *n_admitted = nstar;
}

int schedule_impl(const float* conf, const float* sps, int R, int gamma, int n_table,
                  int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                  hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, 8);
  prof_before(DSPARK_KID_SCHEDULE, stream);
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma,
                     n_table, verify_len, n_admitted, cum_conf, ws_ptr<int32_t>(ws, L.err));
  prof_after(DSPARK_KID_SCHEDULE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

}  // namespace dspark
