// Wave-level inverse-CDF selection over tile records (one wave per request).
//
// A tile record describes TILE = 256 consecutive columns of one logit (or
// residual) row as 8 floats: (m, s, s0, s1, s2, s3, 0, 0), where m is a shift
// (the tile maximum, or 0 for residual mass), s = (s0 + s1) + (s2 + s3) and
// s0..s3 are the masses of the four 64-column chunks relative to exp(m/T).
// Selection draws the tile holding u * Z (Z = total mass, fp64) and then the
// chunk inside it; the caller recomputes that chunk's 64 values and finishes
// with wave_pick64.
#pragma once

#include "common.h"

namespace dspark {

// Largest tile count per lane held in registers: nt <= 64 * MAX_TPL, i.e.
// V <= 64 * 16 * 256 = 262144.
constexpr int MAX_TPL = 16;
constexpr int MAX_V = 64 * MAX_TPL * TILE;

struct TilePick {
  int t;         // chosen tile
  int w;         // chosen 64-column chunk in the tile
  double rem;    // remaining mass inside the chunk (INFINITY: take the last positive column)
  double scale;  // exp((m_t - M) / T): converts chunk values to the row's scale
  double Z;      // total mass of the row (relative to exp(M / T))
  float M;       // row shift
  float mt;      // shift of the chosen tile
};

__device__ __forceinline__ double wave_excl_scan_d(double v, double* incl_out) {
  // inclusive scan within 16-lane rows (lanes past a row's start add 0.0),
  // then rows 1 and 3 add the last lane of rows 0 and 2, rows 2 and 3 add
  // lane 31; the exclusive value is the inclusive one of the lane before
  double incl = v;
  incl += dpp_f64<DPP_ROW_SHR + 1>(incl);
  incl += dpp_f64<DPP_ROW_SHR + 2>(incl);
  incl += dpp_f64<DPP_ROW_SHR + 4>(incl);
  incl += dpp_f64<DPP_ROW_SHR + 8>(incl);
  incl += dpp_f64<DPP_ROW_BCAST15, 0xA>(incl);
  incl += dpp_f64<DPP_ROW_BCAST31, 0xC>(incl);
  *incl_out = incl;
  return dpp_f64<DPP_WAVE_SHR1>(incl);
}

__device__ __forceinline__ int wave_min_i(int v) {
  return wave_reduce_i(v, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_max_i(int v) {
  return wave_reduce_i(v, [](int a, int b) { return max(a, b); });
}

// recs: the row's records (2 float4 per tile).  use_shift: weights are
// s * exp((m - M) / T) (softmax partials) or plain s (residual mass, m = 0).
__device__ __forceinline__ TilePick wave_select_tile(const float4* __restrict__ recs, int nt, bool use_shift,
                                            double invTd, double u) {
  const int lane = threadIdx.x & 63;
  const int per = ceil_div(nt, 64);
  const int t0 = min(nt, lane * per), t1 = min(nt, t0 + per);
  float m[MAX_TPL], s[MAX_TPL];
  float4 sw[MAX_TPL];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < MAX_TPL; i++) {
    const int t = t0 + i;
    const bool ok = (i < per) && (t < t1);
    const int tc = ok ? t : 0;  // branch-free: clamped address, masked value
    const float4 r0 = recs[2 * tc], r1 = recs[2 * tc + 1];
    m[i] = ok ? r0.x : -INFINITY;
    s[i] = ok ? r0.y : 0.f;
    sw[i] = ok ? make_float4(r0.z, r0.w, r1.x, r1.y) : make_float4(0.f, 0.f, 0.f, 0.f);
    mloc = fmaxf(mloc, m[i]);
  }
  const float M = use_shift ? wave_max(mloc) : 0.f;
  double w[MAX_TPL];
  double loc = 0.0;
#pragma unroll
  for (int i = 0; i < MAX_TPL; i++) {
    w[i] = 0.0;
    if (t0 + i < t1)
      w[i] = use_shift ? (double)s[i] * (double)exp_acc((m[i] - M) * (float)invTd) : (double)s[i];
    loc += w[i];
  }
  double incl_unused;
  const double ex = wave_excl_scan_d(loc, &incl_unused);
  const int owner_last = (nt - 1) / per;
  const double Z = __shfl(ex + loc, owner_last);
  const double target = u * Z;

  int found = 0x7fffffff, lastpos = -1;
  double before = 0.0, cum = 0.0;
  float fm = 0.f, lm = 0.f;
  float4 fsw = make_float4(0.f, 0.f, 0.f, 0.f), lsw = fsw;
#pragma unroll
  for (int i = 0; i < MAX_TPL; i++) {
    const int t = t0 + i;
    if (t < t1) {
      const double pp = cum;
      cum += w[i];
      if (found == 0x7fffffff && target < ex + cum) {
        found = t;
        before = ex + pp;
        fm = m[i];
        fsw = sw[i];
      }
      if (s[i] > 0.f) {
        lastpos = t;
        lm = m[i];
        lsw = sw[i];
      }
    }
  }
  TilePick P;
  P.Z = Z;
  P.M = M;
  const int tmin = wave_min_i(found);
  float4 csw;
  if (tmin != 0x7fffffff) {
    const int owner = tmin / per;
    P.t = tmin;
    P.rem = __shfl(target - before, owner);
    P.mt = __shfl(fm, owner);
    csw = make_float4(__shfl(fsw.x, owner), __shfl(fsw.y, owner), __shfl(fsw.z, owner),
                      __shfl(fsw.w, owner));
  } else {
    // rounding left u*Z past the last boundary: the last tile with mass
    const int tl = max(wave_max_i(lastpos), 0);
    const int owner = tl / per;
    P.t = tl;
    P.rem = INFINITY;
    P.mt = __shfl(lm, owner);
    csw = make_float4(__shfl(lsw.x, owner), __shfl(lsw.y, owner), __shfl(lsw.z, owner),
                      __shfl(lsw.w, owner));
  }
  P.scale = use_shift ? (double)exp_acc((P.mt - M) * (float)invTd) : 1.0;
  // chunk inside the tile (uniform across the wave)
  const float cs[4] = {csw.x, csw.y, csw.z, csw.w};
  double c = 0.0;
  int wstar = -1;
  double remw = P.rem;
  for (int k = 0; k < 4; k++) {
    const double nc = c + (double)cs[k] * P.scale;
    if (P.rem < nc) {
      wstar = k;
      remw = P.rem - c;
      break;
    }
    c = nc;
  }
  if (wstar < 0) {
    wstar = 0;
    for (int k = 0; k < 4; k++)
      if (cs[k] > 0.f) wstar = k;
    remw = INFINITY;
  }
  P.w = wstar;
  P.rem = remw;
  return P;
}

// Workgroup version (256 threads, tiles spread over all of them): the same
// choice as wave_select_tile with the row's records read by 4 waves, for a
// shorter latency chain when one workgroup serves one request.  Every thread
// returns the same pick.  nt <= 256 * BTPL.
constexpr int BTPL = 4;
struct BlockSelectSmem {
  float wmax[4];
  double wsum[4];
  double Z;
  int found[4], last[4];
  double rem;
  float mt;
  float4 csw;
};

// Tiles [t0, t1) of thread tid: tid * per, ... with per = ceil(nt / 256).
__device__ __forceinline__ void block_tile_range(int nt, int& t0, int& t1) {
  const int per = ceil_div(nt, 256);
  t0 = min(nt, (int)threadIdx.x * per);
  t1 = min(nt, t0 + per);
}

// Selection on records already held by the threads: m[i], s[i] and the four
// 64-column sums sw[i] of tile t0 + i (t0, t1 from block_tile_range, TPL at
// least the tiles per thread; entries at or past t1 hold m = -inf, s = 0,
// sw = 0).  All 256 threads call it.
template <int TPL>
__device__ __forceinline__ TilePick block_select_tile_vals(const float (&m)[TPL], const float (&s)[TPL],
                                                           const float4 (&sw)[TPL], int nt, bool use_shift,
                                                           double invTd, double u, BlockSelectSmem& sm) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int t0, t1;
  block_tile_range(nt, t0, t1);
  if (tid == 0) {  // defaults when no tile carries mass (Z = 0, reported by the caller)
    sm.rem = INFINITY;
    sm.mt = 0.f;
    sm.csw = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < TPL; i++) mloc = fmaxf(mloc, m[i]);
  float M = 0.f;
  const float wm = wave_max(mloc);
  if (lane == 0) sm.wmax[wave] = wm;
  lds_barrier();
  if (use_shift) M = fmaxf(fmaxf(sm.wmax[0], sm.wmax[1]), fmaxf(sm.wmax[2], sm.wmax[3]));
  double w[TPL];
  double loc = 0.0;
#pragma unroll
  for (int i = 0; i < TPL; i++) {
    w[i] = 0.0;
    if (t0 + i < t1)
      w[i] = use_shift ? (double)s[i] * (double)exp_acc((m[i] - M) * (float)invTd) : (double)s[i];
    loc += w[i];
  }
  double incl;
  const double ex = wave_excl_scan_d(loc, &incl);
  if (lane == 63) sm.wsum[wave] = incl;
  lds_barrier();
  double base = 0.0;
  for (int q = 0; q < wave; q++) base += sm.wsum[q];
  base += ex;
  // Z is the inclusive prefix at the last tile, so a draw below Z always
  // lands on a tile
  const int owner_last = (nt - 1) / ceil_div(nt, 256);
  if (tid == owner_last) sm.Z = base + loc;
  lds_barrier();
  const double Z = sm.Z;
  const double target = u * Z;

  int found = 0x7fffffff, lastpos = -1;
  double before = 0.0, cum = 0.0;
  float fm = 0.f, lm = 0.f;
  float4 fsw = make_float4(0.f, 0.f, 0.f, 0.f), lsw = fsw;
#pragma unroll
  for (int i = 0; i < TPL; i++) {
    const int t = t0 + i;
    if (t < t1) {
      const double pp = cum;
      cum += w[i];
      if (found == 0x7fffffff && target < base + cum) {
        found = t;
        before = base + pp;
        fm = m[i];
        fsw = sw[i];
      }
      if (s[i] > 0.f) {
        lastpos = t;
        lm = m[i];
        lsw = sw[i];
      }
    }
  }
  const int fw = wave_min_i(found), lw = wave_max_i(lastpos);
  if (lane == 0) {
    sm.found[wave] = fw;
    sm.last[wave] = lw;
  }
  lds_barrier();
  const int tmin = min(min(sm.found[0], sm.found[1]), min(sm.found[2], sm.found[3]));
  const int tl = max(max(max(sm.last[0], sm.last[1]), max(sm.last[2], sm.last[3])), 0);
  TilePick P;
  P.Z = Z;
  P.M = M;
  if (tmin != 0x7fffffff) {
    P.t = tmin;
    if (found == tmin && t0 <= tmin && tmin < t1) {
      sm.rem = target - before;
      sm.mt = fm;
      sm.csw = fsw;
    }
  } else {
    P.t = tl;
    if (t0 <= tl && tl < t1 && lastpos == tl) {
      sm.rem = INFINITY;
      sm.mt = lm;
      sm.csw = lsw;
    }
  }
  lds_barrier();
  P.rem = sm.rem;
  P.mt = sm.mt;
  const float4 csw = sm.csw;
  P.scale = use_shift ? (double)exp_acc((P.mt - M) * (float)invTd) : 1.0;
  const float cs[4] = {csw.x, csw.y, csw.z, csw.w};
  double c = 0.0;
  int wstar = -1;
  double remw = P.rem;
  for (int k = 0; k < 4; k++) {
    const double nc = c + (double)cs[k] * P.scale;
    if (P.rem < nc) {
      wstar = k;
      remw = P.rem - c;
      break;
    }
    c = nc;
  }
  if (wstar < 0) {
    wstar = 0;
    for (int k = 0; k < 4; k++)
      if (cs[k] > 0.f) wstar = k;
    remw = INFINITY;
  }
  P.w = wstar;
  P.rem = remw;
  return P;
}

// ld(i) returns float4 i of the row's records (2 per tile); the overload
// below reads them with plain loads.
template <typename Ld>
__device__ __forceinline__ TilePick block_select_tile_ld(Ld ld, int nt, bool use_shift, double invTd,
                                                         double u, BlockSelectSmem& sm) {
  int t0, t1;
  block_tile_range(nt, t0, t1);
  float m[BTPL], s[BTPL];
  float4 sw[BTPL];
#pragma unroll
  for (int i = 0; i < BTPL; i++) {
    const int t = t0 + i;
    const bool ok = t < t1;
    const int tc = ok ? t : 0;
    const float4 r0 = ld(2 * tc), r1 = ld(2 * tc + 1);
    m[i] = ok ? r0.x : -INFINITY;
    s[i] = ok ? r0.y : 0.f;
    sw[i] = ok ? make_float4(r0.z, r0.w, r1.x, r1.y) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  return block_select_tile_vals<BTPL>(m, s, sw, nt, use_shift, invTd, u, sm);
}

__device__ __forceinline__ TilePick block_select_tile(const float4* __restrict__ recs, int nt,
                                                      bool use_shift, double invTd, double u,
                                                      BlockSelectSmem& sm) {
  return block_select_tile_ld([&](int i) { return recs[i]; }, nt, use_shift, invTd, u, sm);
}

// Bias of one 64-column chunk for one request: bias[c] = sum_k w1[k] *
// W2[k][cb + c] (w1 in LDS as fp32; exact bf16 products, fp32 sums).  Thread
// (cg, q) of the 256 covers CPT = 8 / sizeof(WT) consecutive columns and
// k = q, q + NG, ... with 8-byte loads (64 consecutive columns per k row); the
// NG partial sums of a column are added in a fixed order.  Call from all 256
// threads (it has a barrier); lane c of wave 0 gets column cb + c, the other
// waves 0.  part must hold NG = 32 / sizeof(WT) rows of 64 floats.
template <typename WT, int KS>
__device__ __forceinline__ float chunk_bias(const WT* __restrict__ W2, int V, int r, int cb,
                                            const float* w1s, float (*part)[WCOLS]) {
  constexpr int CPT = 8 / sizeof(WT);
  constexpr int TPG = WCOLS / CPT;
  constexpr int NG = 256 / TPG;
  constexpr int KI = (16 * KS + NG - 1) / NG;
  static_assert(NG == 32 / sizeof(WT), "k groups must match the partial-sum array");
  const int tid = threadIdx.x;
  const int cg = tid % TPG, q = tid / TPG;
  const int c0 = cb + CPT * cg;
  const int c0c = (c0 < V) ? c0 : 0;  // columns past V: any valid column (masked by the caller)
  uint2 raw[KI];
#pragma unroll
  for (int i = 0; i < KI; i++) {
    const int k = min(q + NG * i, r - 1);
    raw[i] = *reinterpret_cast<const uint2*>(W2 + (size_t)k * V + c0c);
  }
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; c++) acc[c] = 0.f;
#pragma unroll
  for (int i = 0; i < KI; i++) {
    const int k = q + NG * i;
    if (k < r) {
      const float a = w1s[k];
#pragma unroll
      for (int c = 0; c < CPT; c++) acc[c] = fmaf(a, elem_of<WT>(raw[i], c), acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; c++) part[q][CPT * cg + c] = acc[c];
  lds_barrier();
  if ((tid >> 6) != 0) return 0.f;
  const int lane = tid & 63;
  float bias = part[0][lane];
#pragma unroll
  for (int g = 1; g < NG; g++) bias += part[g][lane];
  return bias;
}

// Gather the 64 chunk values held by lanes 0 and 32 (bias-block layout,
// element (p, t) of lane 32h is column 16(t/4) + 8h + 2(t%4) + p) so that
// lane c receives column c.
__device__ __forceinline__ float chunk_to_lanes(const float (&v)[2][16]) {
  const int c = threadIdx.x & 63;
  const int src = ((c >> 3) & 1) * 32;
  const int want_t = 4 * (c >> 4) + ((c >> 1) & 3), want_p = c & 1;
  float out = 0.f;
#pragma unroll
  for (int t = 0; t < 16; t++)
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const float x = __shfl(v[p][t], src);
      if (t == want_t && p == want_p) out = x;
    }
  return out;
}

// Inverse-CDF pick among 64 per-lane values (lane c = column c): smallest c
// with rem < scale * sum_{i <= c} v_i, else the last c with v_c > 0.
__device__ __forceinline__ int wave_pick64(float v, double scale, double rem) {
  const int lane = threadIdx.x & 63;
  double incl;
  wave_excl_scan_d((double)v * scale, &incl);
  const int hit = (rem < incl) ? lane : 0x7fffffff;
  const int c = wave_min_i(hit);
  if (c != 0x7fffffff) return c;
  return max(wave_max_i(v > 0.f ? lane : -1), 0);
}

}  // namespace dspark
