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
__device__ __forceinline__ void sort_wave_stage(uint64_t (&k)[KPT], int kk, int tid) {
  if (kk <= D) return;
  const int lane = tid & 63;
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

// Step 1 and the keys: on return slot t + NT m (flat index order) of the
// unsorted pool is k[m] of thread t, slots past R * gamma hold ~0.
template <int NT, int KPT, int NB>
__device__ __forceinline__ void pool_keys(const float* __restrict__ conf, int R, int gamma,
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
}

// Bitonic sort, ascending, of the NT * KS keys in registers (slot t + NT m is
// k[m] of thread t; tid is threadIdx.x, passed in so that a caller in a loop
// can keep the per-stage partner indices from being hoisted out of it).  Distances of NT and up stay inside a thread, 64..NT/2
// go through the LDS exchange buffers of sm, below 64 through DPP and
// permlane moves.  The first LDS stage writes bufs[NB - 1], so bufs[0] may
// still be read by other threads when this starts (with NB = 2).
template <int NT, int KS, int NB, typename SM>
__device__ __forceinline__ void pool_bitonic(SM& sm, uint64_t (&k)[KS], int tid) {
  constexpr int NS = NT * KS;
  constexpr int KPT = KS;
  int nb = NB - 1;  // next exchange buffer
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
    sort_wave_stage<32, NT>(k, kk, tid);
    sort_wave_stage<16, NT>(k, kk, tid);
    sort_wave_stage<8, NT>(k, kk, tid);
    sort_wave_stage<4, NT>(k, kk, tid);
    sort_wave_stage<2, NT>(k, kk, tid);
    sort_wave_stage<1, NT>(k, kk, tid);
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
  pool_keys<NT, KPT, NB>(conf, R, gamma, cum_conf, err, sm, k);
  pool_bitonic<NT, KPT, NB>(sm, k, (int)threadIdx.x);
}

// Step 3: exact fixed-point prefix in slot order.  Calls f(i, Tn, v) for every
// slot i < n of the thread, with Tn = T0 + (sum of the first i values) and
// v = floor(a_i * 2^36); returns the sum of all n values.  T0 = R * 2^36 for
// a whole pool.  Every thread must call it.
// key(m) gives the thread's slot tid + NT m.
template <int NT, int KPT, typename SM, typename Key, typename Fn>
__device__ __forceinline__ long long pool_scan(Key key, int n, long long T0, SM& sm, Fn f) {
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
    if (i < n) f(i, T0 + carry + before + (incl - vm), vm);
    carry += total;
    __syncthreads();  // wsum is rewritten for the next m
  }
  return carry;
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
  else pool_scan<NT, KPT>(key, n, (long long)R << FIX_SHIFT, sm, walk);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) drop = min(drop, __shfl_xor(drop, o));
  if (lane == 0 && drop < n) atomicMin(&sm.s_n, drop);
  __syncthreads();
  const int nstar = sm.s_n;
  pool_admit<NT, KPT, NB>(key, nstar, R, gamma, sm, verify_len);
  if (tid == 0) *n_admitted = nstar;
}

// The (rank + 1)-th smallest of the 32-bit values hv(m) over the slots with
// cand(m) (rank below their count): four 8-bit digit passes, most significant
// first, each an LDS histogram of the candidates whose higher digits match the
// ones chosen so far.  Returns w with #{h < w} <= rank < #{h <= w}, and in
// *rank_in_group the rank among the candidates equal to w.  Every thread must
// call it.
template <int NT, int KPT, typename Cand, typename HV>
__device__ __forceinline__ uint32_t select_rank(Cand cand, HV hv, int rank, uint32_t* hist, int* sel,
                                                int* rank_in_group = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0u, pmask = 0u;
  int r = rank;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += NT) hist[b] = 0u;
    __syncthreads();
#pragma unroll 1
    for (int m = 0; m < KPT; m++) {
      const uint32_t h = hv(m);
      if (cand(m) && (h & pmask) == prefix) atomicAdd(&hist[(h >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l .. 4l + 3; exactly one lane holds rank r
      const int c0 = (int)hist[4 * lane], c1 = (int)hist[4 * lane + 1];
      const int c2 = (int)hist[4 * lane + 2], c3 = (int)hist[4 * lane + 3];
      const int tot = c0 + c1 + c2 + c3;
      double incl;
      const int q = r - (int)wave_excl_scan_d((double)tot, &incl);
      if (q >= 0 && q < tot) {
        int bin = 4 * lane, rr = q;
        if (rr >= c0) {
          rr -= c0;
          bin++;
          if (rr >= c1) {
            rr -= c1;
            bin++;
            if (rr >= c2) {
              rr -= c2;
              bin++;
            }
          }
        }
        sel[0] = bin;
        sel[1] = rr;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel[0] << shift;
    pmask |= 255u << shift;
    r = sel[1];
    __syncthreads();  // hist and sel are rewritten by the next pass
  }
  if (rank_in_group) *rank_in_group = r;  // #{h < w} = rank - r
  return prefix;
}

// The early-stop walk needs the sorted pool only up to its first drop, so
// pools of more than 2048 candidates are sorted a chunk at a time.  The next
// chunk is every remaining candidate whose key lies below the (2048 + 1)-th
// smallest remaining key, found on the high word (the survival probability)
// by select_rank and, when a group of equal high words larger than a chunk
// leaves that empty, refined on the low word (the flat index) within the
// group: at most 2048 candidates, all of them below every candidate still
// left.  It is gathered into LDS, sorted, and walked with the prefix carried
// over from the chunks before; the walk ends at the first drop.  A chunk thus
// holds exactly the next slots of the whole sorted pool, and n*, T_n and the
// admitted set are those of the whole-pool sort.  The admitted candidates are
// the keys below the first one not admitted.
constexpr int SCHED_CHUNK = 2 * SCHED_THREADS;

// Two exchange buffers of a chunk sort carved out of a larger LDS array.
struct ChunkBufs {
  uint64_t* bufs[2];
};

template <int KPT>
__device__ __forceinline__ void schedule_chunked_body(const float* __restrict__ conf,
                                                      const float* __restrict__ sps, int R, int gamma,
                                                      int n_table, int32_t* __restrict__ verify_len,
                                                      int32_t* __restrict__ n_admitted,
                                                      float* __restrict__ cum_conf, int32_t* err) {
  constexpr int NT = SCHED_THREADS, NB = 2, CK = SCHED_CHUNK / NT;
  __shared__ SchedSmem<NT, KPT, NB> sm;
  __shared__ uint32_t hist[256];
  __shared__ int sel[2];
  __shared__ int s_cnt, s_drop;
  __shared__ uint64_t s_cut;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = R * gamma;
  {
    uint64_t unused[KPT];
    pool_keys<NT, KPT, NB>(conf, R, gamma, cum_conf, err, sm, unused);
  }
  // the pool stays in LDS in flat index order (bufs[0]); bufs[1] holds the
  // chunk (its first 2048 slots, then the sort's second exchange buffer)
  const uint64_t* K = sm.bufs[0];
  uint64_t* C = sm.bufs[1];
  ChunkBufs cb;
  cb.bufs[0] = C;
  cb.bufs[1] = C + SCHED_CHUNK;

  int base = 0;                               // pool slots already walked
  long long Tb = (long long)R << FIX_SHIFT;   // T at slot base
  uint64_t klo = 0ull;                        // remaining candidates: keys >= klo
  uint64_t cut = ~0ull;                       // admitted: keys below cut
  int nstar = n;
  auto cand = [&](int m) { return tid + NT * m < n && K[tid + NT * m] >= klo; };
  // gathers the candidates below khi into C; returns their count
  auto gather = [&](uint64_t khi) {
    if (tid == 0) s_cnt = 0;
    __syncthreads();
#pragma unroll 1
    for (int m = 0; m < KPT; m++) {
      const uint64_t x = K[tid + NT * m];
      if (tid + NT * m < n && x >= klo && x < khi) C[atomicAdd(&s_cnt, 1)] = x;
    }
    __syncthreads();
    return s_cnt;
  };
#pragma unroll 1
  while (base < n) {
    uint64_t khi = ~0ull;  // every real key is below it
    if (n - base > SCHED_CHUNK) {
      const uint32_t w = select_rank<NT, KPT>(cand, [&](int m) { return (uint32_t)(K[tid + NT * m] >> 32); },
                                              SCHED_CHUNK, hist, sel);
      khi = (uint64_t)w << 32;
    }
    int cs = gather(khi);
    if (cs == 0) {  // uniform: more than a chunk of keys share the high word w
      const uint32_t w = (uint32_t)(khi >> 32);
      const uint32_t w2 = select_rank<NT, KPT>(
          [&](int m) { return cand(m) && (uint32_t)(K[tid + NT * m] >> 32) == w; },
          [&](int m) { return (uint32_t)K[tid + NT * m]; }, SCHED_CHUNK, hist, sel);
      khi |= w2;
      __syncthreads();  // every thread has read s_cnt
      cs = gather(khi);
      // exactly a chunk by construction; the guard keeps the loop finite
      if (cs == 0) {
        nstar = base;
        cut = klo;
        break;
      }
    }
    for (int i = cs + tid; i < SCHED_CHUNK; i += NT) C[i] = ~0ull;
    __syncthreads();
    uint64_t c[CK];
#pragma unroll
    for (int m = 0; m < CK; m++) c[m] = C[tid + NT * m];
    // the first exchange stage writes cb.bufs[1], beyond the chunk's slots;
    // an opaque thread id keeps the stages' partner indices inside the loop
    int otid = tid;
    asm volatile("" : "+v"(otid));
    pool_bitonic<NT, CK, NB>(cb, c, otid);
    if (tid == 0) s_drop = cs;
    int drop = cs;
    auto walk = [&](int i, long long Tn, long long v) {
      const double th0 = (double)Tn * sps_at(sps, n_table, R + base + i);
      const double th1 = (double)(Tn + v) * sps_at(sps, n_table, R + base + i + 1);
      if (th1 < th0) drop = min(drop, i);
    };
    const long long tot = pool_scan<NT, CK>([&](int m) { return c[m]; }, cs, Tb, sm, walk);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) drop = min(drop, __shfl_xor(drop, o));
    if (lane == 0 && drop < cs) atomicMin(&s_drop, drop);
    __syncthreads();
    const int d = s_drop;
    if (d < cs) {  // uniform: the first drop is in this chunk, at sorted slot d
#pragma unroll
      for (int m = 0; m < CK; m++)
        if (tid + NT * m == d) s_cut = c[m];
      __syncthreads();
      cut = s_cut;
      nstar = base + d;
      break;
    }
    base += cs;
    Tb += tot;
    klo = khi;
    __syncthreads();  // the chunk buffer and the exchange buffers are reused
  }

  // Step 5 on the pool in index order: the admitted keys are those below cut
  int* cnt = reinterpret_cast<int*>(C);
  __syncthreads();
  for (int r = tid; r < R; r += NT) cnt[r] = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const uint64_t x = K[tid + NT * m];
    if (tid + NT * m < n && x < cut) atomicAdd(&cnt[(uint32_t)x / gamma], 1);
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) verify_len[r] = cnt[r];
  if (tid == 0) *n_admitted = nstar;
}

template <int KPT>
__global__ __launch_bounds__(SCHED_THREADS) void k_schedule_chunked(const float* __restrict__ conf,
                                                                   const float* __restrict__ sps, int R,
                                                                   int gamma, int n_table,
                                                                   int32_t* __restrict__ verify_len,
                                                                   int32_t* __restrict__ n_admitted,
                                                                   float* __restrict__ cum_conf, int32_t* err) {
  schedule_chunked_body<KPT>(conf, sps, R, gamma, n_table, verify_len, n_admitted, cum_conf, err);
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
    else pool_scan<NT, KPT>(key, n, (long long)R << FIX_SHIFT, sm, f);
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

  // the current pool's first K candidates are its K smallest keys: no second
  // sort, only the (K + 1)-th smallest key, selected on the high word and,
  // inside a group of equal high words, on the low word (the flat index)
  pool_keys<NT, KPT, NB>(conf, R, gamma, cum_conf, err, sm, k);
  // the keys in flat index order: LDS with one buffer, registers with two
  auto ckey = [&](int m) { return NB == 1 ? sm.bufs[0][tid + NT * m] : k[m]; };
  auto live = [&](int m) { return tid + NT * m < n; };
  uint32_t* hist = NB == 1 ? reinterpret_cast<uint32_t*>(sm.cstage) : reinterpret_cast<uint32_t*>(&sm.bufs[1][0]);
  uint64_t cut = ~0ull;  // admitted: keys below cut
  if (K < n) {
    int r;
    const uint32_t w = select_rank<NT, KPT>(live, [&](int m) { return (uint32_t)(ckey(m) >> 32); }, K, hist,
                                            sm.wmin, &r);
    cut = (uint64_t)w << 32;
    if (r > 0)  // uniform: the cut falls inside the group of keys equal to w
      cut |= select_rank<NT, KPT>([&](int m) { return live(m) && (uint32_t)(ckey(m) >> 32) == w; },
                                  [&](int m) { return (uint32_t)ckey(m); }, r, hist, sm.wmin);
  }
  int* cnt = NB == 1 ? reinterpret_cast<int*>(sm.cstage) : reinterpret_cast<int*>(&sm.bufs[0][0]);
  __syncthreads();
  for (int r = tid; r < R; r += NT) cnt[r] = 0;
  __syncthreads();
#pragma unroll
  for (int m = 0; m < KPT; m++) {
    const uint64_t x = ckey(m);
    if (live(m) && x < cut) atomicAdd(&cnt[(uint32_t)x / gamma], 1);
  }
  __syncthreads();
  for (int r = tid; r < R; r += NT) verify_len[r] = cnt[r];
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
      hipLaunchKernelGGL(k_schedule_chunked<4>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma,
                         n_table, verify_len, n_admitted, cum_conf, err);
    else
      hipLaunchKernelGGL(k_schedule_chunked<8>, dim3(1), dim3(SCHED_THREADS), 0, stream, conf, sps, R, gamma,
                         n_table, verify_len, n_admitted, cum_conf, err);
  }
  prof_after(DSPARK_KID_SCHEDULE, stream);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

}  // namespace dspark
