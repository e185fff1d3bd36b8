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
//
// dspark_schedule_threshold: the static-threshold baseline L_r = #{j : a_{r,j}
// >= theta} (HADA, "Análise dos experimentos": the static threshold sweep).
//
// dspark_schedule_async (HADA, "Implantação em produção", practical
// application of the scheduler): the cut length K is the first maximiser of
// Theta over the pool of the confidences of two steps earlier (steps 1-4
// without the early stop), and step 5 admits the first K candidates of the
// current pool.
#include "common.h"
#include "select.h"

namespace dspark {

constexpr int SCHED_THREADS = 1024;
constexpr int FIX_SHIFT = 36;
// The lean shape: pools of at most 1024 candidates in 256 threads.
constexpr int SCHED_LEAN_THREADS = 256;
constexpr int SCHED_LEAN_KPT = 4;

// LDS of the scheduler kernels: NB exchange buffers of NS = NT * KPT keys
// (also the per-request counters), the confidence staging (the second buffer,
// or an array of its own with one buffer), per-wave partials.
template <int NT, int KPT, int NB>
struct SchedSmem {
  uint64_t bufs[NB][NT * KPT];
  float cstage[NB == 1 ? NT * KPT : 1];
  long long wsum[NT / 64];
  double wmax[NT / 64];
  int wmin[NT / 64];
  int s_n;
};

// One bitonic stage at partner distance D < 64 (lane ^ D, DPP and permlane
// moves) of the merge of size kk; no stage when D >= kk.
template <int D, int NT, int KPT>
__device__ __forceinline__ void sort_wave_stage(uint64_t (&k)[KPT], int kk) {
  if (kk <= D) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int tk = tid & kk;  // slot i = tid + NT m: i & kk = tk | (NT m & kk)
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const uint64_t y = lane_xor_u64<D>(k[m]);
    const bool up = (tk | ((NT * m) & kk)) == 0, lower = (lane & D) == 0;
    // keep the smaller key where lower == up, else the larger (equal keys
    // are interchangeable)
    if ((lower == up) == (y < k[m])) k[m] = y;
    if (NT < SCHED_THREADS) __builtin_amdgcn_sched_barrier(0);  // one key's exchange at a time: fewer live registers
  }
}

// Steps 1-2 for one confidence array: running products (written to cum_conf
// when non-NULL), 64-bit keys, bitonic sort.  On return slot t + NT m of the
// sorted pool is k[m] of thread t.  Every thread must call it.  With NB = 2
// the LDS stages alternate between two buffers (one barrier each); with one
// buffer a stage also waits before it overwrites the buffer.
template <int NT, int KPT, int NB>
__device__ __forceinline__ void pool_sort(const float* __restrict__ conf, int R, int gamma,
                                          float* __restrict__ cum_conf, int32_t* err, SchedSmem<NT, KPT, NB>& sm,
                                          uint64_t (&k)[KPT]) {
  constexpr int NS = NT * KPT;
  const int tid = threadIdx.x;
  const int n = R * gamma;
  __syncthreads();  // a previous user of the LDS buffers is done
  // confidences read in parallel (coalesced) into LDS
  float* cl = NB == 1 ? sm.cstage : reinterpret_cast<float*>(&sm.bufs[NB - 1][0]);
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
      sm.bufs[0][f] = ((uint64_t)(~__float_as_uint(a)) << 32) | (uint32_t)f;
    }
  }
  for (int i = n + tid; i < NS; i += NT) sm.bufs[0][i] = ~0ull;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < KPT; m++) k[m] = sm.bufs[0][tid + NT * m];

  int nb = NB - 1;  // next exchange buffer (bufs[0] is still being read above)
  // unrolled: every stage's distances and directions are constants
#pragma unroll
  for (int kk = 2; kk <= NS; kk <<= 1) {
#pragma unroll
    for (int jj = kk >> 1; jj >= 64; jj >>= 1) {
      if (jj >= NT) {
        const int mj = jj / NT;
#pragma unroll
        for (int m = 0; m < KPT; m++) {
          if ((m & mj) == 0) {
            const int m2 = m | mj;
            const bool up = ((tid & kk) | ((NT * m) & kk)) == 0;
            const uint64_t x = k[m], y = k[m2];
            if ((x > y) == up) {
              k[m] = y;
              k[m2] = x;
            }
          }
        }
      } else if (jj >= 64) {
        uint64_t* B = sm.bufs[nb];
        if (NB == 2) nb ^= 1;
        else __syncthreads();  // every thread has read the previous stage's partners
#pragma unroll
        for (int m = 0; m < KPT; m++) B[tid + NT * m] = k[m];
        __syncthreads();
#pragma unroll
        for (int m = 0; m < KPT; m++) {
          // partner slot (tid ^ jj) + NT m: jj < NT leaves the m part alone
          const uint64_t y = B[(tid ^ jj) + NT * m];
          const bool up = ((tid & kk) | ((NT * m) & kk)) == 0, lower = (tid & jj) == 0;
          k[m] = (lower == up) ? (k[m] < y ? k[m] : y) : (k[m] > y ? k[m] : y);
        }
      }
    }
    // distances below 64: partners in the same wave
    sort_wave_stage<32, NT>(k, kk);
    sort_wave_stage<16, NT>(k, kk);
    sort_wave_stage<8, NT>(k, kk);
    sort_wave_stage<4, NT>(k, kk);
    sort_wave_stage<2, NT>(k, kk);
    sort_wave_stage<1, NT>(k, kk);
  }
}

// Step 3: exact fixed-point prefix in slot order.  Calls f(i, Tn, v) for every
// slot i < n of the thread, with Tn = R * 2^36 + (sum of the first i values)
// and v = floor(a_i * 2^36).  Every thread must call it.
// key(m) gives the thread's slot tid + NT m.
template <int NT, int KPT, int NB, typename Key, typename Fn>
__device__ __forceinline__ void pool_scan(Key key, int n, int R, SchedSmem<NT, KPT, NB>& sm, Fn f) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long carry = 0;
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const int i = tid + NT * m;
    const float a = __uint_as_float(~(uint32_t)(key(m) >> 32));
    const long long vm = (i < n) ? (long long)floor((double)a * (double)(1LL << FIX_SHIFT)) : 0;
    // the wave scan runs in fp64, exact here: every partial sum is an
    // integer below 64 * 2^36 < 2^53
    double incl_d;
    (void)wave_excl_scan_d((double)vm, &incl_d);
    const long long incl = (long long)incl_d;
    if (lane == 63) sm.wsum[wave] = incl;
    __syncthreads();
    long long before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; w++) {
      const long long x = sm.wsum[w];
      if (w < wave) before += x;
      total += x;
    }
    if (i < n) f(i, ((long long)R << FIX_SHIFT) + carry + before + (incl - vm), vm);
    carry += total;
    __syncthreads();  // wsum is rewritten for the next m
  }
}

// Step 3 with the sorted keys in LDS (bufs[0], slot order): thread t takes
// the KPT consecutive slots t KPT .. t KPT + KPT - 1, so one wave scan of the
// per-thread sums and one exchange of the per-wave totals give every prefix.
// Calls f as pool_scan does.  Every thread must call it.
template <int NT, int KPT, int NB, typename Fn>
__device__ __forceinline__ void pool_scan_lds(int n, int R, SchedSmem<NT, KPT, NB>& sm, Fn f) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto val = [&](int i) -> long long {
    if (i >= n) return 0;
    const float a = __uint_as_float(~(uint32_t)(sm.bufs[0][i] >> 32));
    return (long long)floor((double)a * (double)(1LL << FIX_SHIFT));
  };
  long long loc = 0;
#pragma unroll
  for (int q = 0; q < KPT; q++) loc += val(tid * KPT + q);
  // exact in fp64: every partial sum is an integer below NT * KPT * 2^36 < 2^53
  double incl_d;
  const double excl_d = wave_excl_scan_d((double)loc, &incl_d);
  if (lane == 63) sm.wsum[wave] = (long long)incl_d;
  __syncthreads();
  long long Tn = ((long long)R << FIX_SHIFT) + (long long)excl_d;
#pragma unroll
  for (int w = 0; w < NT / 64; w++)
    if (w < wave) Tn += sm.wsum[w];
#pragma unroll 1
  for (int q = 0; q < KPT; q++) {
    const int i = tid * KPT + q;
    if (i < n) {
      const long long v = val(i);
      f(i, Tn, v);
      Tn += v;
    }
  }
  __syncthreads();  // wsum may be reused
}

__device__ __forceinline__ double sps_at(const float* __restrict__ sps, int n_table, int B) {
  return (B <= n_table) ? (double)sps[B - 1] : 0.0;
}

// Step 5: verify_len[r] = admitted candidates (the first nstar slots) of row r.
template <int NT, int KPT, int NB, typename Key>
__device__ __forceinline__ void pool_admit(Key key, int nstar, int R, int gamma, SchedSmem<NT, KPT, NB>& sm,
                                           int32_t* __restrict__ verify_len) {
  const int tid = threadIdx.x;
  // with one buffer the keys stay in it and the counters take the staging array
  int* cnt = NB == 1 ? reinterpret_cast<int*>(sm.cstage) : reinterpret_cast<int*>(&sm.bufs[0][0]);
  __syncthreads();
  for (int r = tid; r < R; r += NT) cnt[r] = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const int i = tid + NT * m;
    if (i < nstar) atomicAdd(&cnt[(uint32_t)key(m) / gamma], 1);
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) verify_len[r] = cnt[r];
}

// Early-stop walk: n* = first slot whose admission lowers Theta.
template <int NT, int KPT, int NB>
__device__ __forceinline__ void schedule_body(const float* __restrict__ conf, const float* __restrict__ sps,
                                              int R, int gamma, int n_table, int32_t* __restrict__ verify_len,
                                              int32_t* __restrict__ n_admitted, float* __restrict__ cum_conf,
                                              int32_t* err) {
  __shared__ SchedSmem<NT, KPT, NB> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = R * gamma;
  if (tid == 0) sm.s_n = n;
  uint64_t k[KPT];
  pool_sort<NT, KPT, NB>(conf, R, gamma, cum_conf, err, sm, k);
  // with one buffer the sorted keys go back to LDS (fewer live registers)
  if (NB == 1) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < KPT; m++) sm.bufs[0][tid + NT * m] = k[m];
    __syncthreads();
  }
  auto key = [&](int m) { return NB == 1 ? sm.bufs[0][tid + NT * m] : k[m]; };
  int drop = n;
  auto walk = [&](int i, long long Tn, long long v) {
    const double th0 = (double)Tn * sps_at(sps, n_table, R + i);
    const double th1 = (double)(Tn + v) * sps_at(sps, n_table, R + i + 1);
    if (th1 < th0) drop = min(drop, i);
  };
  if (NB == 1) pool_scan_lds<NT, KPT, NB>(n, R, sm, walk);
  else pool_scan<NT, KPT, NB>(key, n, R, sm, walk);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) drop = min(drop, __shfl_xor(drop, o));
  if (lane == 0 && drop < n) atomicMin(&sm.s_n, drop);
  __syncthreads();
  const int nstar = sm.s_n;
  pool_admit<NT, KPT, NB>(key, nstar, R, gamma, sm, verify_len);
  if (tid == 0) *n_admitted = nstar;
}

template <int KPT>
__global__ __launch_bounds__(SCHED_THREADS) void k_schedule(const float* __restrict__ conf,
                                                           const float* __restrict__ sps, int R,
                                                           int gamma, int n_table,
                                                           int32_t* __restrict__ verify_len,
                                                           int32_t* __restrict__ n_admitted,
                                                           float* __restrict__ cum_conf,
                                                           int32_t* err) {
  schedule_body<SCHED_THREADS, KPT, 2>(conf, sps, R, gamma, n_table, verify_len, n_admitted, cum_conf, err);
}

// The same walk for pools of at most 1024 candidates in a workgroup small
// enough to share a compute unit with the one-launch draft (one wave per SIMD,
// at most 32 registers per lane, one 8 KiB exchange buffer), so that it can
// run beside the draft instead of ahead of it.
__global__ __launch_bounds__(SCHED_LEAN_THREADS) __attribute__((amdgpu_num_vgpr(32))) void k_schedule_lean(
    const float* __restrict__ conf, const float* __restrict__ sps, int R, int gamma, int n_table,
    int32_t* __restrict__ verify_len, int32_t* __restrict__ n_admitted, float* __restrict__ cum_conf,
    int32_t* err) {
  schedule_body<SCHED_LEAN_THREADS, SCHED_LEAN_KPT, 1>(conf, sps, R, gamma, n_table, verify_len, n_admitted,
                                                       cum_conf, err);
}

// Asynchronous production variant: K = the first maximiser of Theta over the
// lagged pool (no early stop), then the current pool's top K are admitted.
template <int NT, int KPT, int NB>
__device__ __forceinline__ void schedule_async_body(const float* __restrict__ conf,
                                                    const float* __restrict__ conf_lag,
                                                    const float* __restrict__ sps, int R, int gamma, int n_table,
                                                    int32_t* __restrict__ verify_len,
                                                    int32_t* __restrict__ n_admitted, float* __restrict__ cum_conf,
                                                    int32_t* err) {
  __shared__ SchedSmem<NT, KPT, NB> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = R * gamma;
  uint64_t k[KPT];
  // with one buffer the sorted keys go back to LDS (fewer live registers)
  auto to_lds = [&]() {
    if (NB == 1) {
      __syncthreads();
#pragma unroll
      for (int m = 0; m < KPT; m++) sm.bufs[0][tid + NT * m] = k[m];
      __syncthreads();
    }
  };
  auto key = [&](int m) { return NB == 1 ? sm.bufs[0][tid + NT * m] : k[m]; };
  auto scan = [&](auto f) {
    if (NB == 1) pool_scan_lds<NT, KPT, NB>(n, R, sm, f);
    else pool_scan<NT, KPT, NB>(key, n, R, sm, f);
  };
  pool_sort<NT, KPT, NB>(conf_lag, R, gamma, nullptr, err, sm, k);
  to_lds();
  // Theta_0 (no draft admitted) belongs to thread 0; slot i gives Theta_{i+1}
  const double theta0 = (double)((long long)R << FIX_SHIFT) * sps_at(sps, n_table, R);
  double best = (tid == 0) ? theta0 : -1.0;
  scan([&](int i, long long Tn, long long v) {
    best = fmax(best, (double)(Tn + v) * sps_at(sps, n_table, R + i + 1));
  });
  // block arg-max: largest Theta, then the smallest n holding it
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) best = fmax(best, __shfl_xor(best, o));
  if (lane == 0) sm.wmax[wave] = best;
  __syncthreads();
  double bmax = sm.wmax[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) bmax = fmax(bmax, sm.wmax[w]);
  int cand = 0x7fffffff;
  scan([&](int i, long long Tn, long long v) {
    const double th = (double)(Tn + v) * sps_at(sps, n_table, R + i + 1);
    if (th == bmax) cand = min(cand, i + 1);
  });
  if (tid == 0 && theta0 == bmax) cand = 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) cand = min(cand, __shfl_xor(cand, o));
  if (lane == 0) sm.wmin[wave] = cand;
  __syncthreads();
  int K = sm.wmin[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) K = min(K, sm.wmin[w]);

  pool_sort<NT, KPT, NB>(conf, R, gamma, cum_conf, err, sm, k);
  to_lds();
  pool_admit<NT, KPT, NB>(key, K, R, gamma, sm, verify_len);
  if (tid == 0) *n_admitted = K;
}

template <int KPT>
__global__ __launch_bounds__(SCHED_THREADS) void k_schedule_async(const float* __restrict__ conf,
                                                                 const float* __restrict__ conf_lag,
                                                                 const float* __restrict__ sps, int R,
                                                                 int gamma, int n_table,
                                                                 int32_t* __restrict__ verify_len,
                                                                 int32_t* __restrict__ n_admitted,
                                                                 float* __restrict__ cum_conf,
                                                                 int32_t* err) {
  schedule_async_body<SCHED_THREADS, KPT, 2>(conf, conf_lag, sps, R, gamma, n_table, verify_len, n_admitted,
                                             cum_conf, err);
}

// The asynchronous variant for pools of at most 1024 candidates, in the lean
// scheduler's shape (256 threads, at most 32 registers per lane, one 8 KiB
// exchange buffer): it shares a compute unit with the one-launch draft.
__global__ __launch_bounds__(SCHED_LEAN_THREADS) __attribute__((amdgpu_num_vgpr(32))) void k_schedule_async_lean(
    const float* __restrict__ conf, const float* __restrict__ conf_lag, const float* __restrict__ sps, int R,
    int gamma, int n_table, int32_t* __restrict__ verify_len, int32_t* __restrict__ n_admitted,
    float* __restrict__ cum_conf, int32_t* err) {
  schedule_async_body<SCHED_LEAN_THREADS, SCHED_LEAN_KPT, 1>(conf, conf_lag, sps, R, gamma, n_table, verify_len,
                                                             n_admitted, cum_conf, err);
}

// Static-threshold baseline: L_r = #{j : a_{r,j} >= theta}.  One workgroup
// of 256 threads in at most 32 registers per lane (it shares a compute unit
// with the one-launch draft); thread t handles requests t, t + 256, ...; the
// admitted total is summed in a fixed order through LDS.
constexpr int SCHED_TH_THREADS = 256;
__global__ __launch_bounds__(SCHED_TH_THREADS) __attribute__((amdgpu_num_vgpr(32))) void k_schedule_threshold(
    const float* __restrict__ conf, float theta, int R, int gamma, int32_t* __restrict__ verify_len,
    int32_t* __restrict__ n_admitted, float* __restrict__ cum_conf, int32_t* err) {
  __shared__ int wsum[SCHED_TH_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tot = 0;
  for (int r = tid; r < R; r += SCHED_TH_THREADS) {
    float a = 1.0f;
    int L = 0;
    for (int j = 0; j < gamma; j++) {
      const size_t f = (size_t)r * gamma + j;
      float c = conf[f];
      if (!(c > 0.f && c <= 1.f)) {
        raise_err(err, DSPARK_DERR_CONF);
        c = (c > 1.f) ? 1.f : 0.f;
      }
      a = (j == 0) ? c : __fmul_rn(a, c);
      if (cum_conf) cum_conf[f] = a;
      L += (a >= theta) ? 1 : 0;
    }
    verify_len[r] = L;
    tot += L;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  if (lane == 0) wsum[wave] = tot;
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int w = 0; w < SCHED_TH_THREADS / 64; w++) n += wsum[w];
    *n_admitted = n;
  }
}

int schedule_threshold_impl(const float* conf, float theta, int R, int gamma, int32_t* verify_len,
                            int32_t* n_admitted, float* cum_conf, void* ws, hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, 8);
  prof_before(DSPARK_KID_SCHEDULE, stream);
  for (int rep = prof_repeat(DSPARK_KID_SCHEDULE); rep > 0; rep--)
    hipLaunchKernelGGL(k_schedule_threshold, dim3(1), dim3(SCHED_TH_THREADS), 0, stream, conf, theta, R, gamma,
                       verify_len, n_admitted, cum_conf, ws_ptr<int32_t>(ws, L.err));
  prof_after(DSPARK_KID_SCHEDULE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int schedule_async_impl(const float* conf, const float* conf_lag, const float* sps, int R, int gamma,
                        int n_table, int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                        hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, 8);
  const int n = R * gamma;
  int32_t* err = ws_ptr<int32_t>(ws, L.err);
  prof_before(DSPARK_KID_SCHEDULE, stream);
  for (int rep = prof_repeat(DSPARK_KID_SCHEDULE); rep > 0; rep--) {
    if (n <= SCHED_LEAN_THREADS * SCHED_LEAN_KPT)
      hipLaunchKernelGGL(k_schedule_async_lean, dim3(1), dim3(SCHED_LEAN_THREADS), 0, stream, conf, conf_lag, sps,
                         R, gamma, n_table, verify_len, n_admitted, cum_conf, err);
    else if (n <= 2 * SCHED_THREADS)
      hipLaunchKernelGGL(k_schedule_async<2>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, conf_lag, sps, R,
                         gamma, n_table, verify_len, n_admitted, cum_conf, err);
    else if (n <= 4 * SCHED_THREADS)
      hipLaunchKernelGGL(k_schedule_async<4>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, conf_lag, sps, R,
                         gamma, n_table, verify_len, n_admitted, cum_conf, err);
    else
      hipLaunchKernelGGL(k_schedule_async<8>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, conf_lag, sps, R,
                         gamma, n_table, verify_len, n_admitted, cum_conf, err);
  }
  prof_after(DSPARK_KID_SCHEDULE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int schedule_impl(const float* conf, const float* sps, int R, int gamma, int n_table,
                  int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                  hipStream_t stream) {
  const WsLayout L = ws_layout(R, gamma, 8);
  const int n = R * gamma;
  int32_t* err = ws_ptr<int32_t>(ws, L.err);
  prof_before(DSPARK_KID_SCHEDULE, stream);
  for (int rep = prof_repeat(DSPARK_KID_SCHEDULE); rep > 0; rep--) {
    if (n <= SCHED_LEAN_THREADS * SCHED_LEAN_KPT)
      hipLaunchKernelGGL(k_schedule_lean, dim3(1), dim3(SCHED_LEAN_THREADS), 0, stream, conf, sps, R, gamma,
                         n_table, verify_len, n_admitted, cum_conf, err);
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
