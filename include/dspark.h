/*
 * dspark.h - C ABI of the DSpark speculative-decoding round on AMD MI355X (gfx950).
 *
 * One round is three calls, each stream-ordered on the caller's HIP stream:
 *
 *   dspark_draft     Markov-head sequential drafting of gamma tokens per request
 *   dspark_schedule  hardware-aware prefix scheduler: per-request verify lengths
 *                    (dspark_schedule_async: the production variant with a
 *                    lagged cut length)
 *   dspark_verify    lossless rejection-sampling verification and emission
 *
 * Sources (page title, section):
 *   "DSpark: Aceleração da inferência de LLM com speculative decoding"
 *   (pt.news.hada.io): "Arquitetura" - the decode cycle (anchor, draft,
 *   scheduler cut, target verify, corrected token), Semi-Autoregressive
 *   Generation (parallel stage gives base logits; sequential stage adds a
 *   prefix-dependent transition bias), the Markov head (first-order bias from
 *   the previous token, low-rank B = W1 W2, default rank 256), the confidence
 *   head (c_k in (0,1)) and the Hardware-Aware Prefix Scheduler (survival
 *   probabilities a_{r,j}, cost table SPS(B), objective tau * SPS(B), global
 *   sort, greedy admission with early stop, non-anticipation);
 *   "Definição do problema" - speculative decoding verifies a drafted block in
 *   one target pass and keeps the longest prefix consistent with the target
 *   distribution by rejection sampling.
 *   "DeepSpec ... DSpark" (jdon.com), scheduler sections - one global pool of
 *   candidates sorted high to low, each admitted token grows the batch by 1.
 *
 * Conventions (all calls)
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     where a parameter says "host".  The library allocates no device memory
 *     (dspark_draft_noalloc's static array aside) and never modifies an input.
 *     Process-wide state: per device, whether the one-launch draft fits (an
 *     occupancy query, cached on first use) and dspark_draft_noalloc's array;
 *     per host thread, the optional launch-timing hook (dspark_profile_arm).
 *     Two environment variables are read on every dspark_draft call:
 *     DSPARK_DRAFT_KERNEL=stepwise selects the per-step kernels, and
 *     DSPARK_FUSED_SPIN_TICKS overrides the one-launch draft's wait limit
 *     (in 100 MHz ticks; 0 makes every wait that does not succeed at once
 *     give up, which the tests of that path use).  Every verify call reads
 *     DSPARK_VERIFY_KERNEL: "split" keeps the residual and finalize kernels
 *     apart for small problems (at most 16 column tiles), where one kernel
 *     per request otherwise does both; the outputs are the same.
 *   - Arrays are dense, row-major, with the last index contiguous.
 *   - W1/W2 are bf16 (bit patterns in uint16) or fp32 according to w_type.
 *   - No random numbers are drawn inside the library: every random choice is
 *     an inverse-CDF or threshold test on a caller-supplied uniform in [0, 1).
 *   - Host-side argument checks run before any launch; a failing check returns
 *     a negative status and launches nothing.  A failed launch returns
 *     DSPARK_EHIP.  Calls are asynchronous: results are ready when the stream
 *     reaches them.
 *   - Bad values in device memory (NaN logits, uniforms outside [0,1), tokens
 *     outside [0,V), confidences outside (0,1], draft probabilities <= 0) cannot
 *     be checked from the host (nor verify lengths outside [0, gamma]); kernels
 *     OR a DSPARK_DERR_* bit into an error
 *     word inside the workspace, substitute a safe value (token 0, uniform 0,
 *     confidence clamped) and carry on.  Read it with dspark_device_error.
 *   - The workspace is caller-allocated device memory of at least
 *     dspark_workspace_size(R, gamma, V, r) bytes, 256-byte aligned, cleared
 *     once with dspark_workspace_init.  Calls on one workspace must be ordered
 *     on one stream; concurrent calls need distinct workspaces.  One exception:
 *     dspark_verify_stream may run concurrently with dspark_draft or
 *     dspark_draft_rnn on the same workspace (they touch disjoint parts of it).
 *
 * Limits (the sizes the kernels are built for): 1 <= gamma <= 16,
 * 16 <= r <= 256 with r % 16 == 0, 8 <= V <= 262144 with V % 8 == 0
 * (16-byte aligned rows), R >= 1, R * gamma <= 8192 for dspark_schedule.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSPARK_OK = 0,
  DSPARK_EINVAL = -1, /* an argument is NULL, out of range, or not aligned   */
  DSPARK_ENOSPC = -2, /* workspace_bytes < dspark_workspace_size(...)         */
  DSPARK_EHIP = -3    /* a HIP runtime call or kernel launch failed           */
} dspark_status;

typedef enum {
  DSPARK_W_BF16 = 0,  /* W1, W2 hold bfloat16 bit patterns (uint16)           */
  DSPARK_W_F32 = 1    /* W1, W2 hold float32                                  */
} dspark_wtype;

/* Device-side data error bits, OR-ed into the workspace error word. */
#define DSPARK_DERR_NONFINITE 1 /* NaN/inf in a logit row (base + bias or target) */
#define DSPARK_DERR_UNIFORM 2   /* a uniform outside [0, 1); 0 was used instead    */
#define DSPARK_DERR_CONF 4      /* a confidence outside (0, 1]; clamped            */
#define DSPARK_DERR_TOKEN 8     /* a token id outside [0, V); 0 was used instead   */
#define DSPARK_DERR_PROB 16     /* a draft probability <= 0 or NaN; rejected       */
#define DSPARK_DERR_LENGTH 32   /* a verify length outside [0, gamma]; clamped     */
#define DSPARK_DERR_CALIB 64    /* calibration input out of range: a confidence or
                                   label outside [0, 1] (clamped, NaN -> 0) or a
                                   temperature that is not finite and > 0 (never
                                   chosen; dspark_sts_apply leaves c unchanged)  */
#define DSPARK_DERR_SYNC 128    /* the one-launch draft waited past its time limit
                                   for another workgroup (not all resident, or
                                   the GPU shared); its outputs are invalid     */

#define DSPARK_MAX_GAMMA 16
#define DSPARK_MAX_RANK 256
#define DSPARK_MAX_POOL 8192
#define DSPARK_STS_MAX_N (1 << 21)   /* held-out blocks per calibration fit */
#define DSPARK_STS_MAX_GRID 1024     /* candidate temperatures               */
#define DSPARK_STS_MAX_BINS 64       /* ECE bins                             */

/* Bytes of workspace the three calls need for these sizes (host-only query).
 * Returns 0 for sizes outside the limits above. */
size_t dspark_workspace_size(int R, int gamma, int V, int r);

/* Clear the whole workspace (error word, counters, the one-launch draft's sync
 * words and sealed records; asynchronous on stream).  Required once before
 * first use: the one-launch draft's tags are unique only from that clear on. */
int dspark_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Copy the workspace error word to *host_bits (host pointer), then clear it.
 * Synchronizes `stream`. */
int dspark_device_error(void* workspace, size_t workspace_bytes, int32_t* host_bits,
                        hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char* dspark_status_string(int status);

/*
 * dspark_draft - Markov-head sequential drafting.
 *
 * For k = 1..gamma and every request r, with x_0 = anchor[r]:
 *   z_k[v] = base[r, k-1, v] + sum_i W1[x_{k-1}, i] * W2[i, v]
 * (row of W1 = previous token, column of W2 = next token; bf16 products are
 * accumulated in fp32), then x_k is drawn from softmax(z_k / T) by inverse CDF
 * over ascending token id: x_k = min{v : u_draft[r,k-1] < F(v)}.  T == 0 is
 * greedy: x_k = argmax z_k, lowest id on ties.
 *
 *   base          [R, gamma, V] fp32   base logits of the parallel stage
 *   W1            [V, r]               previous-token factor
 *   W2            [r, V]               next-token factor
 *   anchor        [R] int32            token preceding position 1
 *   u_draft       [R, gamma] fp32      one uniform per draft event
 *   temperature   >= 0 (host scalar), 0 = greedy
 *   draft_tokens  out [R, gamma] int32 x_k
 *   draft_probs   out [R, gamma] fp32  q_k(x_k) (1 for greedy)
 *   draft_stats   out [R, gamma, 2] fp32 (m, Z): m = max_v z_k[v],
 *                 Z = sum_v exp((z_k[v] - m) / T); greedy writes (m, 1)
 *
 * Kernels: with bf16 factors, r in {16, 32, 64, 128, 256}, R <= 1024 and
 * ceil(V / 256) <= min(512, 2 x the compute units), all gamma steps run in one
 * persistent launch of one workgroup per compute unit; its workgroups wait
 * for each other's results through the workspace, so every one of them must
 * be resident at once.  The host checks that one workgroup fits on a compute
 * unit (472 registers per lane, about 148 KiB of LDS), not that the compute
 * units are free: kernels of other streams or processes that occupy them can
 * keep part of the grid waiting.  Every wait is bounded (0.5 s); one that
 * runs out sets DSPARK_DERR_SYNC, every workgroup still finishes, and the
 * call's outputs are then INVALID: a caller that shares the GPU must read the
 * error word (dspark_device_error) before using them.  Otherwise, small
 * problems (at most 16 column tiles, V <= 4096, and with fp32 factors
 * r * V <= 16384, with bf16 factors R * gamma * r * V * 2 bytes <= 32 MiB)
 * run all steps in one launch of one workgroup per request, which waits on
 * no other workgroup; the rest run two kernels per step, as does every call
 * with the environment variable DSPARK_DRAFT_KERNEL=stepwise.  All paths
 * give identical outputs.
 */
int dspark_draft(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
                 const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r,
                 float temperature, int32_t* draft_tokens, float* draft_probs, float* draft_stats,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_draft_noalloc - dspark_draft for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, outputs, kernels and results as
 * dspark_draft, without a workspace: the draft's sync words and tile records
 * live in a static device array of DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends.  The call makes
 * no hipMalloc / hipFree and no allocating library call.
 *
 *   device_error  in/out [1] int32 (device): DSPARK_DERR_* bits are OR-ed into
 *                 it (including DSPARK_DERR_SYNC); the caller clears it.
 *
 * Limit: 8448 + 32 * R * ceil(V / 256) <= DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES
 * (R <= 1024 at V = 131072); larger sizes return DSPARK_ENOSPC and launch
 * nothing.  The first call on a device clears the array with a kernel on
 * `stream` ahead of its draft (if that call is captured into a graph, every
 * replay repeats the clear, which is correct and a few microseconds slower).
 * Every call on one GPU shares that GPU's array and leaves its contents for
 * the next: calls that overlap on one GPU (other streams, other threads) race
 * and must not be issued.
 */
#define DSPARK_DRAFT_NOALLOC_SCRATCH_BYTES ((16u << 20) + 8448u)
int dspark_draft_noalloc(const float* base, const void* W1, const void* W2, dspark_wtype w_type,
                         const int32_t* anchor, const float* u_draft, int R, int gamma, int V, int r,
                         float temperature, int32_t* draft_tokens, float* draft_probs, float* draft_stats,
                         int32_t* device_error, hipStream_t stream);

/*
 * dspark_schedule - hardware-aware prefix scheduler.  Reads only confidences
 * and the cost table, never a drafted token (non-anticipation).
 *
 *   a[r,0] = c[r,0],  a[r,j] = fp32(a[r,j-1] * c[r,j])      (survival probability)
 *   pool of R*gamma candidates sorted by (a descending, r*gamma + j ascending)
 *   T_n   = R * 2^36 + sum of floor(a * 2^36) over the first n in the pool
 *           (expected emitted tokens, exact fixed point)
 *   Theta_n = double(T_n) * double(SPS(R + n)),  SPS(B) = sps[B-1] for
 *           B <= n_table, else 0
 *   n* = first n < R*gamma with Theta_{n+1} < Theta_n, else R*gamma
 *   verify_len[r] = number of row-r candidates among the first n*
 *
 *   conf         [R, gamma] fp32  conditional confidences c in (0, 1]
 *   sps          [n_table] fp32   throughput at verify batch B = i + 1
 *   verify_len   out [R] int32    L_r in [0, gamma]
 *   n_admitted   out [1] int32    n*
 *   cum_conf     out [R, gamma] fp32 a, or NULL
 *
 * A pool of at most 1024 candidates is handled by one 256-thread workgroup
 * (at most 40 registers per lane, about 12 KiB of LDS), small enough to run on
 * another stream beside a resident one-launch dspark_draft; larger pools by
 * one 1024-thread workgroup.
 */
int dspark_schedule(const float* conf, const float* sps, int R, int gamma, int n_table,
                    int32_t* verify_len, int32_t* n_admitted, float* cum_conf, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule_async - asynchronous production variant of the scheduler
 * ("DSpark: Aceleração da inferência de LLM com speculative decoding",
 * pt.news.hada.io, section "Implantação em produção", practical application
 * of the scheduler).  The serving engine needs the next verify batch size
 * before the current step finishes, so the cut length comes from the
 * confidences of two steps earlier and the early stop is removed:
 *
 *   K = the smallest n in [0, R*gamma] maximising Theta_n of the pool built
 *       from conf_lag (same a, T_n, Theta_n as dspark_schedule)
 *   verify_len[r] = number of row-r candidates among the first K of the pool
 *       built from conf (current cumulative confidences)
 *
 * K never depends on the current step's confidences or tokens.  The caller
 * keeps the two-step history (the library holds no state).
 *
 *   conf         [R, gamma] fp32  current conditional confidences in (0, 1]
 *   conf_lag     [R, gamma] fp32  confidences of two steps earlier, same shape
 *   sps, n_table                  as for dspark_schedule
 *   verify_len   out [R] int32    L_r
 *   n_admitted   out [1] int32    K
 *   cum_conf     out [R, gamma] fp32 a of conf, or NULL
 * Same checks and status codes as dspark_schedule (conf_lag must be non-NULL).
 * Like dspark_schedule, a pool of at most 1024 candidates is handled by one
 * 256-thread workgroup (at most 40 registers per lane, about 12 KiB of LDS)
 * that can run beside a resident one-launch dspark_draft.
 */
int dspark_schedule_async(const float* conf, const float* conf_lag, const float* sps, int R, int gamma,
                          int n_table, int32_t* verify_len, int32_t* n_admitted, float* cum_conf,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_schedule_threshold - static-threshold baseline ("DSpark: Aceleração da
 * inferência de LLM com speculative decoding", pt.news.hada.io, section
 * "Análise dos experimentos": the static threshold sweep, and why a fixed
 * threshold that ignores the system load is suboptimal in serving).
 *
 *   verify_len[r] = number of positions j with a[r,j] >= theta (a prefix,
 *                   since a is non-increasing); n_admitted = sum of them
 *
 *   conf, cum_conf  as for dspark_schedule; theta: host scalar (not NaN)
 *
 * One 256-thread workgroup of at most 16 registers per lane (any R): it can
 * run beside a resident one-launch dspark_draft.
 */
int dspark_schedule_threshold(const float* conf, float theta, int R, int gamma, int32_t* verify_len,
                              int32_t* n_admitted, float* cum_conf, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * dspark_verify - lossless rejection-sampling verification.
 *
 * Per request r, for k = 1..L_r in order: p = softmax(target[r,k-1] / T);
 * accept x_k iff u_accept[r,k-1] < p(x_k) / q_k(x_k); stop at the first
 * rejection k*.  Emitted: x_1..x_{A}, then y, with A = k*-1 on rejection or
 * L_r otherwise.  On rejection y is drawn by inverse CDF with u_final[r] from
 * max(0, p - pi_{k*}) normalised (pi_{k*} = the draft distribution at k*,
 * recomputed from base, W1, W2 and draft_stats; p itself if that mass is 0).
 * Without rejection y is drawn from softmax(target[r, L_r] / T) (bonus).
 * T == 0: accept iff x_k == argmax target[r,k-1]; y = argmax of row A.
 *
 *   target        [R, gamma+1, V] fp32 target logits; row k-1 scores draft
 *                 position k, row L_r scores the bonus position
 *   base, W1, W2, w_type, anchor   as given to dspark_draft
 *   draft_tokens, draft_probs, draft_stats  outputs of dspark_draft
 *   verify_len    [R] int32 from dspark_schedule, or NULL for L_r = gamma
 *   u_accept      [R, gamma] fp32, u_final [R] fp32
 *   out_tokens    out [R, gamma+1] int32: x_1..x_A, y, then -1
 *   accept_len    out [R] int32 A (emitted tokens = A + 1)
 *   target_probs  out [R, gamma] fp32 p_k(x_k) for k <= min(L_r, A + 1),
 *                 -1 elsewhere (greedy: 1 on a match, 0 on the mismatch); or NULL
 */
int dspark_verify(const float* target, const float* base, const void* W1, const void* W2,
                  dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                  const float* draft_probs, const float* draft_stats, const int32_t* verify_len,
                  const float* u_accept, const float* u_final, int R, int gamma, int V, int r,
                  float temperature, int32_t* out_tokens, int32_t* accept_len, float* target_probs,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_accept_rates - per-position acceptance labels ("DSpark: Aceleração da
 * inferência de LLM com speculative decoding", pt.news.hada.io, section
 * "Arquitetura", Confidence-Scheduled Verification: the confidence head is
 * trained on the analytic per-step acceptance rate; section "Treinamento":
 * that rate is 1 - |p_d - p_t|_1 / 2).
 *
 * For every request r and draft position k = 1..gamma:
 *   accept_rate[r, k-1] = 1 - (1/2) sum_v | q_k(v) - p_k(v) |
 * with q_k the draft distribution at k given the drafted prefix (base row
 * k-1 plus the Markov bias of x_{k-1}, x_0 = anchor, normalised with
 * draft_stats) and p_k = softmax(target[r, k-1] / T): the probability that
 * the rejection test accepts position k when the prefix is accepted.
 * Computed as 1 - sum_v max(0, p_k(v) - q_k(v)) (fp32 per 256-column tile,
 * fp64 across tiles).  Not part of the round; an offline label pass.
 *
 *   target, base, W1, W2, w_type, anchor  as for dspark_verify
 *   draft_tokens, draft_stats             outputs of dspark_draft
 *   temperature    > 0 (host scalar; T == 0 returns DSPARK_EINVAL)
 *   accept_rate    out [R, gamma] fp32
 * Uses the same workspace as dspark_verify (its verify scratch is overwritten).
 */
int dspark_accept_rates(const float* target, const float* base, const void* W1, const void* W2,
                        dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                        const float* draft_stats, int R, int gamma, int V, int r, float temperature,
                        float* accept_rate, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Optional launch-timing hook for benchmarks and profilers.
 *
 * While armed on the calling thread for kernel id `kid`, every launch of that
 * kernel made by this thread's dspark_* calls is bracketed by
 * hipEventRecord(starts[i], stream) before and hipEventRecord(stops[i], stream)
 * after, for i = 0, 1, ... up to n - 1; later launches are not timed.  With
 * repeat > 1 each timed launch is issued `repeat` times back to back inside its
 * event pair (every kernel of the library is idempotent for fixed inputs, so
 * results are unchanged); (stop - start) / repeat then approximates the kernel
 * duration without the event and dispatch latency of a single launch.  The
 * events are created (with timing enabled) and owned by the caller.  The state
 * is thread-local; other threads and unarmed calls are unaffected.
 * dspark_profile_arm returns DSPARK_EINVAL for a bad id, NULL arrays, n < 1 or
 * repeat outside [1, 1000].  dspark_profile_disarm returns the number of pairs
 * recorded.
 */
typedef enum {
  DSPARK_KID_DRAFT_PARTIALS = 1,  /* per-step bias GEMM + softmax partials */
  DSPARK_KID_DRAFT_SELECT = 2,    /* per-step inverse-CDF select            */
  DSPARK_KID_SCHEDULE = 3,        /* prefix scheduler                       */
  DSPARK_KID_VERIFY_STREAM = 4,   /* target-row stream (softmax partials)   */
  DSPARK_KID_VERIFY_DECIDE = 5,   /* row statistics + ordered accept tests  */
  DSPARK_KID_RESIDUAL = 6,        /* residual max(0, p - q) partials        */
  DSPARK_KID_VERIFY_FINALIZE = 7, /* residual / bonus sample and outputs    */
  DSPARK_KID_DRAFT_FUSED = 8,     /* all draft steps in one launch          */
  DSPARK_KID_DRAFT_ROWS = 9       /* small problems: one workgroup/request  */
} dspark_kernel_id;

int dspark_profile_arm(int kid, hipEvent_t* starts, hipEvent_t* stops, int n, int repeat);
int dspark_profile_disarm(void);

/*
 * dspark_verify in two parts, so that the target-row stream can overlap the
 * draft (it reads only target and the verify lengths).
 *
 * dspark_verify_stream: for every request, target rows 0..L_r (L_r from
 * verify_len, or gamma if NULL) are reduced to per-1024-column softmax (or,
 * at temperature 0, arg-max) partials kept in the workspace.
 * dspark_verify_finish: the rest of dspark_verify (row statistics, ordered
 * accept tests, residual or bonus emission), same arguments and outputs as
 * dspark_verify.  It must follow a dspark_verify_stream on the same workspace
 * with the same target, verify_len and temperature, with no other call on
 * that workspace in between except dspark_draft / dspark_draft_rnn.
 * dspark_verify = dspark_verify_stream + dspark_verify_finish.
 */
int dspark_verify_stream(const float* target, const int32_t* verify_len, int R, int gamma, int V,
                         float temperature, void* workspace, size_t workspace_bytes, hipStream_t stream);
int dspark_verify_finish(const float* target, const float* base, const void* W1, const void* W2,
                         dspark_wtype w_type, const int32_t* anchor, const int32_t* draft_tokens,
                         const float* draft_probs, const float* draft_stats, const int32_t* verify_len,
                         const float* u_accept, const float* u_final, int R, int gamma, int V, int r,
                         float temperature, int32_t* out_tokens, int32_t* accept_len, float* target_probs,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_draft_rnn - drafting with the RNN head instead of the Markov head
 * ("DSpark: Aceleração da inferência de LLM com speculative decoding",
 * pt.news.hada.io, section "Arquitetura", Semi-Autoregressive Generation, RNN
 * head: a recurrent state accumulates the whole in-block prefix with a gated
 * update; section "Experimentos": a small extra gain at long blocks).  The
 * pages give no equations; the update is the GRU form, with s_0 = 0 and
 * e = W1[x_{k-1}] (x_0 = anchor):
 *   u = sigmoid(e Wx[0] + s Ws[0] + b[0])       g = sigmoid(e Wx[1] + s Ws[1] + b[1])
 *   h = tanh(e Wx[2] + (g * s) Ws[2] + b[2])   s_k = (1 - u) * s + u * h
 * evaluated in fp64 and stored in the weights' type (fp32, then bf16
 * round-to-nearest-even for bf16 weights).  The transition bias at position k
 * is s_k . W2; everything else is dspark_draft.
 *
 *   base, W1, W2, w_type, anchor, u_draft, temperature, outputs: as dspark_draft
 *   Wx, Ws     [3, r, r] gate weights (update, reset, candidate), storage w_type,
 *              16-byte aligned;
 *              row = input unit, column = state unit
 *   rnn_bias   [3, r] fp32
 *   states     out [R, gamma, r] (w_type, 16-byte aligned): s_1..s_gamma, the
 *              rows dspark_verify_rnn recomputes the draft from
 * Same checks and status codes as dspark_draft; additionally R*gamma*r
 * elements of states must stay below 4 GiB.
 */
int dspark_draft_rnn(const float* base, const void* W1, const void* W2, const void* Wx, const void* Ws,
                     const float* rnn_bias, dspark_wtype w_type, const int32_t* anchor, const float* u_draft,
                     int R, int gamma, int V, int r, float temperature, int32_t* draft_tokens,
                     float* draft_probs, float* draft_stats, void* states, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_verify_rnn - dspark_verify for blocks drafted by dspark_draft_rnn:
 * identical tests and emission, except that the draft distribution at the
 * rejected position k* is recomputed as softmax((base[r, k*-1] + s_{k*} . W2) / T)
 * from the states dspark_draft_rnn wrote (W1 and the anchor are not needed).
 */
int dspark_verify_rnn(const float* target, const float* base, const void* states, const void* W2,
                      dspark_wtype w_type, const int32_t* draft_tokens, const float* draft_probs,
                      const float* draft_stats, const int32_t* verify_len, const float* u_accept,
                      const float* u_final, int R, int gamma, int V, int r, float temperature,
                      int32_t* out_tokens, int32_t* accept_len, float* target_probs, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);
/* The second part of dspark_verify_rnn, after dspark_verify_stream (as for
 * dspark_verify_finish). */
int dspark_verify_rnn_finish(const float* target, const float* base, const void* states, const void* W2,
                             dspark_wtype w_type, const int32_t* draft_tokens, const float* draft_probs,
                             const float* draft_stats, const int32_t* verify_len, const float* u_accept,
                             const float* u_final, int R, int gamma, int V, int r, float temperature,
                             int32_t* out_tokens, int32_t* accept_len, float* target_probs, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_sts_fit - sequential temperature scaling of the confidence head
 * ("DSpark: Aceleração da inferência de LLM com speculative decoding",
 * pt.news.hada.io, section "Arquitetura", Confidence-Scheduled Verification,
 * post-hoc calibration: each c_k is a conditional probability, the survival
 * estimate is the cumulative product over the prefix, and a 1-D grid search
 * runs left to right over the positions on a held-out set minimising ECE;
 * section "Análise dos experimentos": an over-confident head, ECE down to
 * about 1 % after calibration).
 *
 * Calibration map c' = sigmoid(logit(c) / tau_k), logit(c) = log(c / (1 - c)).
 * For k = 1..gamma in order, with tau_1..tau_{k-1} fixed, each candidate
 * grid[g] is scored by
 *   ECE = sum_b | sum_{i in bin b} (prod_{j<=k} c'_{i,j} - prod_{j<=k} labels[i,j]) | / N
 * with bins equal-width bins of [0, 1] (a prediction p falls in bin
 * min(floor(p * bins), bins - 1)); tau_k is the FIRST grid entry with the
 * smallest score.  Bin sums are exact 2^-40 fixed-point sums, so results are
 * bit-reproducible.
 *
 *   conf        [N, gamma] fp32  raw head outputs in [0, 1] (held-out blocks)
 *   labels      [N, gamma] fp32  conditional targets in [0, 1]: acceptance
 *                                rates from dspark_accept_rates, or 0/1 outcomes
 *   grid        [G] fp32         candidate temperatures (finite, > 0)
 *   bins        1..DSPARK_STS_MAX_BINS
 *   tau         out [gamma] fp32 chosen temperatures (copies of grid entries)
 *   tau_index   out [gamma] int32 chosen grid indices, or NULL
 *   ece         out [gamma] fp64 score of the chosen entry
 *   ece_table   out [gamma, G] fp64 every candidate's score, or NULL
 *   workspace   >= dspark_sts_workspace_size(N, gamma, G, bins) bytes,
 *               256-byte aligned; its first word is the device error word
 *               (read it with dspark_device_error)
 * Limits: 1 <= N <= DSPARK_STS_MAX_N, 1 <= gamma <= DSPARK_MAX_GAMMA,
 * 1 <= G <= DSPARK_STS_MAX_GRID.  Returns DSPARK_EINVAL / DSPARK_ENOSPC before
 * any launch on bad sizes, NULL required pointers or a short workspace.
 */
size_t dspark_sts_workspace_size(int N, int gamma, int G, int bins);
int dspark_sts_fit(const float* conf, const float* labels, const float* grid, int N, int gamma, int G,
                   int bins, float* tau, int32_t* tau_index, double* ece, double* ece_table,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dspark_sts_apply - calibrated confidences for the scheduler (same source):
 *   conf_out[r, k] = fp32( sigmoid(logit(conf[r, k]) / tau[k]) )
 * evaluated in fp64 with the same expression as dspark_sts_fit.  conf_out may
 * alias conf.  workspace: any workspace of >= 256 bytes (error word only).
 */
int dspark_sts_apply(const float* conf, const float* tau, int R, int gamma, float* conf_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
