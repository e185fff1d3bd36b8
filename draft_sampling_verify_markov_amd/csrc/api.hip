// C ABI entry points: host-side argument checks, workspace queries and
// dispatch to the draft / schedule / verify launchers.
#include <mutex>

#include "select.h"

namespace dspark {
int draft_impl(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
               const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r, float T,
               int32_t* tokens, float* probs, float* stats, const DraftWs& dw, hipStream_t stream,
               const RnnHead* rnn = nullptr);
int schedule_impl(const float* conf, const float* sps, int R, int gamma, int n_table,
                  int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                  hipStream_t stream);
int schedule_async_impl(const float* conf, const float* conf_lag, const float* sps, int R, int gamma,
                        int n_table, int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* ws,
                        hipStream_t stream);
int schedule_threshold_impl(const float* conf, float theta, int R, int gamma, int32_t* verify_len,
                            int32_t* n_admitted, float* cum_conf, void* ws, hipStream_t stream);
int accept_rates_impl(const float* target, const float* base, const void* W1, const void* W2,
                      dspark_wtype w_type, const int32_t* anchor, const int32_t* dtok, const float* dstats,
                      int R, int gamma, int V, int r, float T, float* out, void* ws, hipStream_t stream);
int verify_impl(const float* target, const float* base, const void* W1, const void* W2,
                dspark_wtype w_type, const int32_t* anchor, const int32_t* dtok, const float* dprob,
                const float* dstats, const int32_t* vlen, const float* u_acc, const float* u_fin,
                int R, int gamma, int V, int r, float T, int32_t* out_tokens, int32_t* accept_len,
                float* target_probs, void* ws, hipStream_t stream, bool dense_rows = false,
                int part = VERIFY_ALL);

size_t sts_workspace_size_impl(int N, int gamma, int G, int bins);
int sts_fit_impl(const float* conf, const float* labels, const float* grid, int N, int gamma, int G, int bins,
                 float* tau, int32_t* tau_index, double* ece, double* ece_table, void* ws, hipStream_t stream);
int sts_apply_impl(const float* conf, const float* tau, int R, int gamma, float* out, void* ws,
                   hipStream_t stream);

__global__ void k_fill_i32(int32_t* p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Largest element count any kernel indexes with 32-bit products.
constexpr long long MAX_ELEMS = (1LL << 31) - 1;

static bool sizes_ok(int R, int gamma, int V, int r) {
  if (R < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA) return false;
  if (V < 8 || (V % 8) != 0 || V > MAX_V) return false;
  if (r < 16 || r > DSPARK_MAX_RANK || (r % 16) != 0) return false;
  if ((long long)R * (gamma + 1) * ceil_div(V, VSEG) > MAX_ELEMS) return false;
  return true;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct ProfState {
  int kid = 0;
  hipEvent_t* starts = nullptr;
  hipEvent_t* stops = nullptr;
  int n = 0, used = 0, repeat = 1;
};
static thread_local ProfState prof;

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

void prof_before(int kid, hipStream_t stream) {
  if (prof.kid == kid && prof.used < prof.n) (void)hipEventRecord(prof.starts[prof.used], stream);
}
void prof_after(int kid, hipStream_t stream) {
  if (prof.kid == kid && prof.used < prof.n) (void)hipEventRecord(prof.stops[prof.used++], stream);
}
int prof_repeat(int kid) { return (prof.kid == kid && prof.used < prof.n) ? prof.repeat : 1; }

static int check_ws(void* ws, size_t bytes, int R, int gamma, int V) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return DSPARK_EINVAL;
  if (bytes < ws_layout(R, gamma, V).total) return DSPARK_ENOSPC;
  return DSPARK_OK;
}

// ---------------------------------------------------------------------------
// dspark_draft_noalloc: the draft's sync words and tile records live in this
// file-scope device array instead of a caller workspace.  Layout: the sync
// words (SYNC_* offsets) at 0, the record region (shared by the one-launch and
// the per-step paths, one of which a call uses) at NOALLOC_REC.  Each device
// the library runs on holds its own copy until the process ends.
constexpr size_t NOALLOC_REC = (SYNC_BYTES + 255) & ~(size_t)255;
static_assert(NOALLOC_REC < DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES, "scratch holds the sync words");
static __device__ __align__(256) unsigned char scratch[DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device (the host-side name is only a
// stand-in for the symbol), found once per device with that device current.
constexpr int NOALLOC_MAX_DEVICES = 64;
struct NoallocDevice {
  std::once_flag once;
  unsigned char* ptr = nullptr;
  hipError_t status = hipSuccess;
};
static NoallocDevice noalloc_dev[NOALLOC_MAX_DEVICES];

// Scratch bytes a draft of these sizes uses (sync words and records).
static size_t noalloc_bytes(int R, int V) { return NOALLOC_REC + (size_t)R * ceil_div(V, TILE) * 32; }

// Set-up on the first call on the current device: the symbol's address, then
// the whole array cleared by a fill kernel on the caller's stream (ahead of
// that call's draft).  The clear makes every later tag unique (the one-launch
// draft's epoch restarts at zero with no sealed record left); a graph that
// captured the first call repeats the clear on every replay, which keeps
// that property.
static unsigned char* noalloc_scratch(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
  NoallocDevice& D = noalloc_dev[dev];
  std::call_once(D.once, [&] {
    void* p = nullptr;
    D.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (D.status != hipSuccess || p == nullptr) return;
    const size_t n = DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES / 4;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536)), dim3(256),
                       0, stream, static_cast<int32_t*>(p), n, 0);
    D.status = hipGetLastError();
    if (D.status == hipSuccess) D.ptr = static_cast<unsigned char*>(p);
  });
  return D.ptr;
}

}  // namespace dspark

using namespace dspark;

extern "C" {

size_t dspark_workspace_size(int R, int gamma, int V, int r) {
  if (!sizes_ok(R, gamma, V, r)) return 0;
  return ws_layout(R, gamma, V).total;
}

int dspark_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || workspace_bytes < 256) return DSPARK_EINVAL;
  // all of it: besides the error word, counters and sync words, the fused
  // draft's sealed records must not hold seals left by an earlier use of the
  // memory (a new workspace starts its epoch from zero again)
  const size_t n = workspace_bytes / 4;
  const size_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)(nb < 65536 ? nb : 65536)), dim3(256), 0, stream,
                     static_cast<int32_t*>(workspace), n, 0);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int dspark_device_error(void* workspace, size_t workspace_bytes, int32_t* host_bits,
                        hipStream_t stream) {
  if (!workspace || !host_bits || workspace_bytes < 256) return DSPARK_EINVAL;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return DSPARK_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return DSPARK_EHIP;
  *host_bits = v;
  hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(64), 0, stream, static_cast<int32_t*>(workspace), (size_t)1,
                     0);
  if (hipGetLastError() != hipSuccess) return DSPARK_EHIP;
  return hipStreamSynchronize(stream) == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

int dspark_profile_arm(int kid, hipEvent_t* starts, hipEvent_t* stops, int n, int repeat) {
  if (kid < DSPARK_KID_DRAFT_PARTIALS || kid > DSPARK_KID_DRAFT_ROWS || !starts || !stops ||
      n < 1 || repeat < 1 || repeat > 1000)
    return DSPARK_EINVAL;
  prof.kid = kid;
  prof.starts = starts;
  prof.stops = stops;
  prof.n = n;
  prof.used = 0;
  prof.repeat = repeat;
  return DSPARK_OK;
}

int dspark_profile_disarm(void) {
  const int used = prof.used;
  prof = ProfState();
  return used;
}

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_EINVAL: return "DSPARK_EINVAL: invalid argument";
    case DSPARK_ENOSPC: return "DSPARK_ENOSPC: workspace too small";
    case DSPARK_EHIP: return "DSPARK_EHIP: HIP runtime or launch failure";
    default: return "unknown dspark status";
  }
}

int dspark_draft(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
                 const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r,
                 float temperature, int32_t* draft_tokens, float* draft_probs, float* draft_stats,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!base || !W1 || !W2 || !anchor || !u_draft || !draft_tokens || !draft_probs || !draft_stats)
    return DSPARK_EINVAL;
  if (!aligned16(base) || !aligned16(W1) || !aligned16(W2)) return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  const int wsr = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (wsr != DSPARK_OK) return wsr;
  return draft_impl(base, W1, W2, w_type, anchor, u_draft, R, gamma, V, r, temperature,
                    draft_tokens, draft_probs, draft_stats, draft_ws(workspace, R, gamma, V), stream);
}

int dspark_draft_noalloc(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
                         const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r,
                         float temperature, int32_t* draft_tokens, float* draft_probs, float* draft_stats,
                         int32_t* device_error, hipStream_t stream) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!base || !W1 || !W2 || !anchor || !u_draft || !draft_tokens || !draft_probs || !draft_stats ||
      !device_error)
    return DSPARK_EINVAL;
  if (!aligned16(base) || !aligned16(W1) || !aligned16(W2)) return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  if (noalloc_bytes(R, V) > DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES) return DSPARK_ENOSPC;
  unsigned char* p = noalloc_scratch(stream);
  if (p == nullptr) return DSPARK_EHIP;
  const DraftWs dw{device_error, p, reinterpret_cast<uint32_t*>(p + NOALLOC_REC),
                   reinterpret_cast<float4*>(p + NOALLOC_REC)};
  return draft_impl(base, W1, W2, w_type, anchor, u_draft, R, gamma, V, r, temperature, draft_tokens,
                    draft_probs, draft_stats, dw, stream);
}

int dspark_schedule(const float* conf, const float* sps, int R, int gamma, int n_table,
                    int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (R < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || (long long)R * gamma > DSPARK_MAX_POOL)
    return DSPARK_EINVAL;
  if (n_table < 1) return DSPARK_EINVAL;
  if (!conf || !sps || !verify_len || !n_admitted) return DSPARK_EINVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSPARK_EINVAL;
  if (workspace_bytes < 256) return DSPARK_ENOSPC;
  return schedule_impl(conf, sps, R, gamma, n_table, verify_len, n_admitted, cum_conf, workspace,
                       stream);
}

int dspark_schedule_async(const float* conf, const float* conf_lag, const float* sps, int R, int gamma,
                          int n_table, int32_t* verify_len, int32_t* n_admitted, float* cum_conf,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (R < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || (long long)R * gamma > DSPARK_MAX_POOL)
    return DSPARK_EINVAL;
  if (n_table < 1) return DSPARK_EINVAL;
  if (!conf || !conf_lag || !sps || !verify_len || !n_admitted) return DSPARK_EINVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSPARK_EINVAL;
  if (workspace_bytes < 256) return DSPARK_ENOSPC;
  return schedule_async_impl(conf, conf_lag, sps, R, gamma, n_table, verify_len, n_admitted, cum_conf,
                             workspace, stream);
}

int dspark_schedule_threshold(const float* conf, float theta, int R, int gamma, int32_t* verify_len,
                              int32_t* n_admitted, float* cum_conf, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (R < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || (long long)R * gamma > DSPARK_MAX_POOL)
    return DSPARK_EINVAL;
  if (!(theta == theta)) return DSPARK_EINVAL;
  if (!conf || !verify_len || !n_admitted) return DSPARK_EINVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSPARK_EINVAL;
  if (workspace_bytes < 256) return DSPARK_ENOSPC;
  return schedule_threshold_impl(conf, theta, R, gamma, verify_len, n_admitted, cum_conf, workspace, stream);
}

int dspark_accept_rates(const float* target, const float* base, const void* W1, const void* W2,
                        dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                        const float* draft_stats, int R, int gamma, int V, int r, float temperature,
                        float* accept_rate, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return DSPARK_EINVAL;
  if (!target || !base || !W1 || !W2 || !anchor || !draft_tokens || !draft_stats || !accept_rate)
    return DSPARK_EINVAL;
  const int st = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (st != DSPARK_OK) return st;
  return accept_rates_impl(target, base, W1, W2, w_type, anchor, draft_tokens, draft_stats, R, gamma, V, r,
                           temperature, accept_rate, workspace, stream);
}

static int verify_checked(const float* target, const float* base, const void* W1, const void* W2,
                          dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                          const float* draft_probs, const float* draft_stats, const int32_t* verify_len,
                          const float* u_accept, const float* u_final, int R, int gamma, int V, int r,
                          float temperature, int32_t* out_tokens, int32_t* accept_len, float* target_probs,
                          void* workspace, size_t workspace_bytes, hipStream_t stream, int part) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!target || !base || !W1 || !W2 || !anchor || !draft_tokens || !draft_probs || !draft_stats ||
      !u_accept || !u_final || !out_tokens || !accept_len)
    return DSPARK_EINVAL;
  if (!aligned16(target) || !aligned16(base) || !aligned16(W1) || !aligned16(W2))
    return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  const int wsr = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (wsr != DSPARK_OK) return wsr;
  return verify_impl(target, base, W1, W2, w_type, anchor, draft_tokens, draft_probs, draft_stats,
                     verify_len, u_accept, u_final, R, gamma, V, r, temperature, out_tokens,
                     accept_len, target_probs, workspace, stream, false, part);
}

int dspark_verify(const float* target, const float* base, const void* W1, const void* W2,
                  dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                  const float* draft_probs, const float* draft_stats, const int32_t* verify_len,
                  const float* u_accept, const float* u_final, int R, int gamma, int V, int r,
                  float temperature, int32_t* out_tokens, int32_t* accept_len, float* target_probs,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return verify_checked(target, base, W1, W2, w_type, anchor, draft_tokens, draft_probs, draft_stats, verify_len,
                        u_accept, u_final, R, gamma, V, r, temperature, out_tokens, accept_len, target_probs,
                        workspace, workspace_bytes, stream, VERIFY_ALL);
}

int dspark_verify_finish(const float* target, const float* base, const void* W1, const void* W2,
                         dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                         const float* draft_probs, const float* draft_stats, const int32_t* verify_len,
                         const float* u_accept, const float* u_final, int R, int gamma, int V, int r,
                         float temperature, int32_t* out_tokens, int32_t* accept_len, float* target_probs,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return verify_checked(target, base, W1, W2, w_type, anchor, draft_tokens, draft_probs, draft_stats, verify_len,
                        u_accept, u_final, R, gamma, V, r, temperature, out_tokens, accept_len, target_probs,
                        workspace, workspace_bytes, stream, VERIFY_FINISH);
}

int dspark_verify_stream(const float* target, const int32_t* verify_len, int R, int gamma, int V,
                         float temperature, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sizes_ok(R, gamma, V, 16)) return DSPARK_EINVAL;
  if (!target || !aligned16(target)) return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  const int wsr = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (wsr != DSPARK_OK) return wsr;
  return verify_impl(target, nullptr, nullptr, nullptr, DSPARK_W_BF16, nullptr, nullptr, nullptr, nullptr,
                     verify_len, nullptr, nullptr, R, gamma, V, 16, temperature, nullptr, nullptr, nullptr,
                     workspace, stream, false, VERIFY_STREAM);
}

int dspark_draft_rnn(const float* base, const void* W1, const void* W2, const void* Wx, const void* Ws,
                     const float* rnn_bias, dspark_wtype w_type, const int32_t* anchor, const float* u_draft,
                     int R, int gamma, int V, int r, float temperature, int32_t* draft_tokens,
                     float* draft_probs, float* draft_stats, void* states, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!base || !W1 || !W2 || !Wx || !Ws || !rnn_bias || !anchor || !u_draft || !draft_tokens || !draft_probs ||
      !draft_stats || !states)
    return DSPARK_EINVAL;
  if (!aligned16(base) || !aligned16(W1) || !aligned16(W2) || !aligned16(Wx) || !aligned16(Ws) || !aligned16(states))
    return DSPARK_EINVAL;
  if ((unsigned long long)R * gamma * r * (w_type == DSPARK_W_BF16 ? 2 : 4) >= (1ull << 32)) return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  const int wsr = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (wsr != DSPARK_OK) return wsr;
  const RnnHead head{Wx, Ws, rnn_bias, states, ws_ptr<double>(workspace, ws_layout(R, gamma, V).rnn)};
  return draft_impl(base, W1, W2, w_type, anchor, u_draft, R, gamma, V, r, temperature, draft_tokens,
                    draft_probs, draft_stats, draft_ws(workspace, R, gamma, V), stream, &head);
}

static int verify_rnn_checked(const float* target, const float* base, const void* states, const void* W2,
                              dspark_wtype w_type, const int32_t* draft_tokens, const float* draft_probs,
                              const float* draft_stats, const int32_t* verify_len, const float* u_accept,
                              const float* u_final, int R, int gamma, int V, int r, float temperature,
                              int32_t* out_tokens, int32_t* accept_len, float* target_probs, void* workspace,
                              size_t workspace_bytes, hipStream_t stream, int part) {
  if (!sizes_ok(R, gamma, V, r)) return DSPARK_EINVAL;
  if (w_type != DSPARK_W_BF16 && w_type != DSPARK_W_F32) return DSPARK_EINVAL;
  if (!target || !base || !states || !W2 || !draft_tokens || !draft_probs || !draft_stats || !u_accept ||
      !u_final || !out_tokens || !accept_len)
    return DSPARK_EINVAL;
  if (!aligned16(target) || !aligned16(base) || !aligned16(states) || !aligned16(W2)) return DSPARK_EINVAL;
  if ((unsigned long long)R * gamma * r * (w_type == DSPARK_W_BF16 ? 2 : 4) >= (1ull << 32)) return DSPARK_EINVAL;
  if (!(temperature >= 0.f) || __builtin_isinf(temperature)) return DSPARK_EINVAL;
  const int wsr = check_ws(workspace, workspace_bytes, R, gamma, V);
  if (wsr != DSPARK_OK) return wsr;
  return verify_impl(target, base, states, W2, w_type, nullptr, draft_tokens, draft_probs, draft_stats,
                     verify_len, u_accept, u_final, R, gamma, V, r, temperature, out_tokens, accept_len,
                     target_probs, workspace, stream, true, part);
}

int dspark_verify_rnn(const float* target, const float* base, const void* states, const void* W2,
                      dspark_wtype w_type, const int32_t* draft_tokens, const float* draft_probs,
                      const float* draft_stats, const int32_t* verify_len, const float* u_accept,
                      const float* u_final, int R, int gamma, int V, int r, float temperature,
                      int32_t* out_tokens, int32_t* accept_len, float* target_probs, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return verify_rnn_checked(target, base, states, W2, w_type, draft_tokens, draft_probs, draft_stats, verify_len,
                            u_accept, u_final, R, gamma, V, r, temperature, out_tokens, accept_len, target_probs,
                            workspace, workspace_bytes, stream, VERIFY_ALL);
}

int dspark_verify_rnn_finish(const float* target, const float* base, const void* states, const void* W2,
                             dspark_wtype w_type, const int32_t* draft_tokens, const float* draft_probs,
                             const float* draft_stats, const int32_t* verify_len, const float* u_accept,
                             const float* u_final, int R, int gamma, int V, int r, float temperature,
                             int32_t* out_tokens, int32_t* accept_len, float* target_probs, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return verify_rnn_checked(target, base, states, W2, w_type, draft_tokens, draft_probs, draft_stats, verify_len,
                            u_accept, u_final, R, gamma, V, r, temperature, out_tokens, accept_len, target_probs,
                            workspace, workspace_bytes, stream, VERIFY_FINISH);
}

static bool sts_sizes_ok(int N, int gamma, int G, int bins) {
  return N >= 1 && N <= DSPARK_STS_MAX_N && gamma >= 1 && gamma <= DSPARK_MAX_GAMMA && G >= 1 &&
         G <= DSPARK_STS_MAX_GRID && bins >= 1 && bins <= DSPARK_STS_MAX_BINS;
}

size_t dspark_sts_workspace_size(int N, int gamma, int G, int bins) {
  if (!sts_sizes_ok(N, gamma, G, bins)) return 0;
  return sts_workspace_size_impl(N, gamma, G, bins);
}

int dspark_sts_fit(const float* conf, const float* labels, const float* grid, int N, int gamma, int G,
                   int bins, float* tau, int32_t* tau_index, double* ece, double* ece_table,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!sts_sizes_ok(N, gamma, G, bins)) return DSPARK_EINVAL;
  if (!conf || !labels || !grid || !tau || !ece) return DSPARK_EINVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSPARK_EINVAL;
  if (workspace_bytes < sts_workspace_size_impl(N, gamma, G, bins)) return DSPARK_ENOSPC;
  return sts_fit_impl(conf, labels, grid, N, gamma, G, bins, tau, tau_index, ece, ece_table, workspace,
                      stream);
}

int dspark_sts_apply(const float* conf, const float* tau, int R, int gamma, float* conf_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (R < 1 || gamma < 1 || gamma > DSPARK_MAX_GAMMA || (long long)R * gamma > MAX_ELEMS) return DSPARK_EINVAL;
  if (!conf || !tau || !conf_out) return DSPARK_EINVAL;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DSPARK_EINVAL;
  if (workspace_bytes < 256) return DSPARK_ENOSPC;
  return sts_apply_impl(conf, tau, R, gamma, conf_out, workspace, stream);
}

}  // extern "C"
