"""Float64 NumPy oracle of one DSpark speculative-decoding round.

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of bench.py, never by the HIP library.

Sources (cited by page title and section; the pages quote the DSpark paper):
  [HADA]  "DSpark: Aceleração da inferência de LLM com speculative decoding"
          (pt.news.hada.io), sections "Definição do problema", "Arquitetura"
          (decode cycle, Semi-Autoregressive Generation, Markov head,
          Confidence-Scheduled Verification, Hardware-Aware Prefix Scheduler)
          and "Treinamento" (per-step acceptance 1 - TV/2).
  [AITALK] "DSpark: la apuesta de DeepSeek por la velocidad que no traiciona la
          calidad" (aitalk.it), sections "El cuello de botella de la
          inferencia" and "Verificar solo lo que importa".
  [JDON]  "DeepSpec发布：让大模型生成提速6倍，输出质量却一点没变差" (jdon.com),
          the scheduler sections (global candidate pool, early stop).

What the round computes, in the pages' order:
  1. Markov head (sequential stage): for k = 1..gamma, the prefix-dependent
     bias B_k = W1[x_{k-1}] . W2 is added to the parallel stage's base logits
     of position k, and x_k is sampled from the resulting distribution
     ([HADA] Arquitetura, Semi-Autoregressive Generation and Markov head;
     the anchor is the first prediction position, so x_0 is the anchor).
  2. Scheduler: survival probabilities a_{r,j} are cumulative products of
     the confidences c; all R*gamma candidates are pooled, sorted by a and
     admitted greedily while the expected throughput tau*SPS(B) rises; the
     walk stops at the first drop ([HADA] Hardware-Aware Prefix Scheduler;
     [JDON] global pool; [AITALK] Verificar solo lo que importa).
  3. Lossless verification: accept x_k with probability min(1, p/q), stop at
     the first rejection and emit one corrected token from the normalised
     residual max(0, p - q), or a bonus token from the next target row when
     the whole verified block is accepted ([HADA] Definição do problema and
     the decode cycle in Arquitetura; [AITALK] first section).

Readings where the pages are silent (each also listed in the design doc):
  * sampling is inverse-CDF over ascending token index with one uniform per
    event: x = min{v : u < F[v]}; if rounding leaves no such v, x is the last
    token with nonzero probability;
  * accept iff u < p/q (strict), so the acceptance probability is min(1, p/q);
  * draft and target share the temperature T; T = 0 means greedy: argmax with
    the lowest index on ties, accept iff the draft token equals the target
    argmax, emit the target argmax;
  * one final uniform per request serves the residual or the bonus sample;
    the bonus is drawn from target row L_r;
  * the residual falls back to p when its mass is zero;
  * the scheduler's a is an fp32 sequential product; the sort key is
    (a descending, flat index r*gamma + j ascending); sums of a are exact
    2^-36 fixed point; Theta_n = T_n * SPS(R + n) in fp64, SPS beyond the
    table is 0; the walk stops at the first strict drop;
  * the asynchronous production scheduler ([HADA] Implantação em produção)
    takes the cut length K as the first maximiser of Theta over the pool of
    the lagged confidences (same shape as the current ones, supplied by the
    caller) and admits the current pool's first K candidates; a table that
    ends before B = R gives Theta = 0 everywhere and K = 0;
  * sequential temperature scaling divides the head's logit by one
    temperature per position; ECE uses equal-width bins and the cumulative
    product of the conditional labels as the target of the cumulative
    product of calibrated confidences; ties in the grid search go to the
    first grid entry.

All floating point is float64 on the exact input values (bf16 and fp32
inputs widen exactly), except the scheduler's fp32 cumulative product.
"""

import numpy as np

FLAG_EPS = 1e-6          # events closer than this to a decision boundary flag the row
FIX_SHIFT = 36           # fixed-point scale 2^36 for survival-probability sums


# ---------------------------------------------------------------------------
# inputs


def widen_weights(w, w_dtype):
    """Return a float64 copy of a Markov factor stored as fp32 or as bf16 bits."""
    if w_dtype == "bf16":
        bits = np.ascontiguousarray(w, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(w, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# 1. Markov head and draft sampling  ([HADA] Arquitetura, Markov head)


def markov_bias(W1_64, W2_64, prev):
    """Transition bias rows W1[prev] @ W2 for an array of previous tokens.

    Row index of W1 is the previous token, column index of W2 the next token:
    after sampling "of" the bias raises "course" ([HADA] Markov head).
    """
    return W1_64[np.asarray(prev)] @ W2_64


def inverse_cdf(w, u):
    """Sample index from non-negative weights ``w`` (1-D) with uniform ``u``.

    Returns (index, margin, F) where F is the normalised cumulative sum,
    index = min{v : u < F[v]} (falls back to the last v with w[v] > 0), and
    margin = min(u - F[index-1], F[index] - u) is the distance of u to the
    nearest edge of the chosen interval.
    """
    total = w.sum()
    F = np.cumsum(w) / total
    idx = int(np.searchsorted(F, u, side="right"))
    if idx >= len(w):
        idx = int(np.flatnonzero(w > 0)[-1])
    lo = F[idx - 1] if idx > 0 else 0.0
    margin = min(u - lo, F[idx] - u)
    return idx, margin, F


def draft_distribution(z, T):
    """Softmax of logits z / T over the last axis (T > 0), in float64.

    Returns (pi, m, Z) with m = max z and Z = sum exp((z - m) / T), so that
    pi = exp((z - m) / T) / Z.
    """
    m = z.max(axis=-1, keepdims=True)
    e = np.exp((z - m) / T)
    Z = e.sum(axis=-1, keepdims=True)
    return e / Z, m[..., 0], Z[..., 0]


def _greedy(z):
    """Argmax (lowest index on ties) and top-1 minus top-2 gap, per row."""
    idx = np.argmax(z, axis=-1)
    top2 = np.partition(z, -2, axis=-1)[..., -2:] if z.shape[-1] > 1 else None
    top1 = z.max(axis=-1)
    gap = (top2[..., 1] - top2[..., 0]) if top2 is not None else np.full(top1.shape, np.inf)
    return idx, top1, gap


def draft(base, W1, W2, w_dtype, anchor, u_draft, T):
    """Sequential Markov-head drafting of gamma tokens for every request.

    base [R, gamma, V] fp32, W1 [V, r], W2 [r, V], anchor [R], u_draft [R, gamma].
    Returns dict(tokens int32 [R, gamma], probs [R, gamma] (q_k(x_k)),
    stats [R, gamma, 2] (max z, sum exp((z - max)/T)), margin [R, gamma]).
    For T = 0 (greedy) probs are 1, stats are (max z, 1) and margin is the
    top-1 minus top-2 logit gap.
    """
    W1_64, W2_64 = widen_weights(W1, w_dtype), widen_weights(W2, w_dtype)
    return _draft_loop(base, u_draft, T, anchor, lambda k, prev: markov_bias(W1_64, W2_64, prev))


def _draft_loop(base, u_draft, T, anchor, bias_of):
    """Left-to-right drafting: at step k the logits are base row k plus
    bias_of(k, previous tokens), and x_k is drawn from their softmax."""
    R, g, V = base.shape
    tokens = np.zeros((R, g), dtype=np.int32)
    probs = np.zeros((R, g))
    stats = np.zeros((R, g, 2))
    margin = np.zeros((R, g))
    prev = np.asarray(anchor, dtype=np.int64)
    for k in range(g):
        z = base[:, k, :].astype(np.float64) + bias_of(k, prev)
        if T == 0:
            idx, top1, gap = _greedy(z)
            tokens[:, k] = idx
            probs[:, k] = 1.0
            stats[:, k, 0], stats[:, k, 1] = top1, 1.0
            margin[:, k] = gap / np.maximum(1.0, np.abs(top1))
        else:
            pi, m, Z = draft_distribution(z, T)
            stats[:, k, 0], stats[:, k, 1] = m, Z
            for i in range(R):
                x, mg, _ = inverse_cdf(pi[i], float(u_draft[i, k]))
                tokens[i, k], probs[i, k], margin[i, k] = x, pi[i, x], mg
        prev = tokens[:, k].astype(np.int64)
    return dict(tokens=tokens, probs=probs, stats=stats, margin=margin)


# ---------------------------------------------------------------------------
# 2. Hardware-aware prefix scheduler  ([HADA] Hardware-Aware Prefix Scheduler)


def _pool(conf, sps):
    """Survival probabilities, sorted candidate pool and the throughput curve.

    a_{r,j} is the fp32 running product of the conditional confidences; the
    R*gamma candidates are sorted by a descending, flat index ascending on
    ties; T_n = R + (sum of the n best a) in exact 2^-36 fixed point (the
    expected emitted tokens of a verify batch of R anchors plus n drafts) and
    Theta_n = T_n * SPS(R + n) in float64, n = 0 .. R*gamma, with SPS = 0 past
    the end of the table ([HADA] Hardware-Aware Prefix Scheduler; [JDON]
    global pool).
    """
    c = np.asarray(conf, dtype=np.float32)
    R, g = c.shape
    a = np.empty_like(c)
    a[:, 0] = c[:, 0]
    for j in range(1, g):
        a[:, j] = a[:, j - 1] * c[:, j]          # float32 * float32 -> float32
    flat = np.arange(R * g, dtype=np.int64)
    af = a.reshape(-1)
    order = np.lexsort((flat, -af.astype(np.float64)))
    a_fx = np.floor(af[order].astype(np.float64) * float(1 << FIX_SHIFT)).astype(np.int64)
    T_n = np.concatenate([[0], np.cumsum(a_fx)]) + np.int64(R) * (np.int64(1) << FIX_SHIFT)
    n = np.arange(R * g + 1)
    B = R + n
    S = np.zeros(R * g + 1)
    ok = B <= len(sps)
    S[ok] = np.asarray(sps, dtype=np.float32)[B[ok] - 1].astype(np.float64)
    theta = T_n.astype(np.float64) * S
    return a, order, theta


def schedule(conf, sps):
    """Confidence scheduler: per-request verify lengths from confidences only.

    conf [R, gamma] fp32 conditional confidences c_{r,j} in (0, 1];
    sps [N] fp32 cost table, sps[i] = throughput at verify batch B = i + 1.
    Never reads a drafted token (the non-anticipation requirement).  The walk
    over the sorted pool admits candidates while Theta rises and stops at the
    first strict drop.
    Returns dict(verify_len int32 [R], n_admitted, cum_conf fp32 [R, gamma],
    theta float64 [R*gamma + 1], order int64 [R*gamma]).
    """
    R, g = np.shape(conf)
    a, order, theta = _pool(conf, sps)
    drops = np.flatnonzero(theta[1:] < theta[:-1])
    n_star = int(drops[0]) if len(drops) else R * g
    L = np.bincount(order[:n_star] // g, minlength=R).astype(np.int32)
    return dict(verify_len=L, n_admitted=n_star, cum_conf=a, theta=theta, order=order)


def schedule_async(conf, conf_lag, sps):
    """Asynchronous production variant of the scheduler.

    The cut length K is the global maximiser of Theta over the pool built from
    the confidences of two steps earlier (conf_lag), with no early stop; the
    current step's candidates, sorted by their own cumulative confidence, are
    admitted top-K ([HADA] Implantação em produção, practical application of
    the scheduler: lagged confidences only set K, the current ones order the
    candidates, early stopping is removed).  Ties of Theta take the smallest n.
    conf_lag has the shape of conf.
    Returns dict(verify_len int32 [R], n_admitted = K, cum_conf fp32 [R, gamma],
    theta_lag float64 [R*gamma + 1], order int64 [R*gamma]).
    """
    R, g = np.shape(conf)
    _, _, theta_lag = _pool(conf_lag, sps)
    K = int(np.argmax(theta_lag))                 # first maximum
    a, order, _ = _pool(conf, sps)
    L = np.bincount(order[:K] // g, minlength=R).astype(np.int32)
    return dict(verify_len=L, n_admitted=K, cum_conf=a, theta_lag=theta_lag, order=order)


def schedule_threshold(conf, theta):
    """Static-threshold baseline: verify while the survival probability holds.

    L_r = number of positions j with a_{r,j} >= theta (a is non-increasing in
    j, so these form a prefix).  The fixed rule ignores the system load that
    the prefix scheduler weighs ([HADA] Análise dos experimentos: the static
    threshold sweep and why static thresholds are suboptimal).
    Returns dict(verify_len int32 [R], n_admitted, cum_conf fp32 [R, gamma]).
    """
    c = np.asarray(conf, dtype=np.float32)
    a = np.empty_like(c)
    a[:, 0] = c[:, 0]
    for j in range(1, c.shape[1]):
        a[:, j] = a[:, j - 1] * c[:, j]
    L = (a >= np.float32(theta)).sum(axis=1).astype(np.int32)
    return dict(verify_len=L, n_admitted=int(L.sum()), cum_conf=a)


# ---------------------------------------------------------------------------
# 3. Lossless verification  ([HADA] Definição do problema; decode cycle)


def verify(target, base, W1, W2, w_dtype, anchor, draft_tokens, draft_probs,
           verify_len, u_accept, u_final, T, states=None):
    """Rejection-sampling verification of the drafted blocks.

    target [R, gamma+1, V]: row k-1 scores draft position k, row L_r scores the
    bonus.  draft_probs are the q_k(x_k) the draft reported.  verify_len [R]
    (None means gamma for every request).
    Returns dict(out_tokens int32 [R, gamma+1] (-1 padded), accept_len int32 [R],
    target_probs [R, gamma] (p_k(x_k) for every evaluated position, -1 for the
    rest), accept_margin [R, gamma] (inf where not evaluated), final_margin [R],
    residual_mass [R] (NaN for bonus rows)).
    states: the RNN head's per-position rows [R, gamma, r] (see draft_rnn);
    when given, the draft row at the rejection is base + states[k*] @ W2 and
    W1 / anchor are not used.
    """
    R, g1, V = target.shape
    g = g1 - 1
    L = np.full(R, g, dtype=np.int64) if verify_len is None else np.asarray(verify_len, np.int64)
    W2_64 = widen_weights(W2, w_dtype)
    W1_64 = None if states is not None else widen_weights(W1, w_dtype)
    x = np.asarray(draft_tokens, dtype=np.int64)
    q = np.asarray(draft_probs, dtype=np.float64)
    out = np.full((R, g + 1), -1, dtype=np.int32)
    A = np.zeros(R, dtype=np.int32)
    tp = np.full((R, g), -1.0)
    acc_m = np.full((R, g), np.inf)
    fin_m = np.full(R, np.inf)
    res_mass = np.full(R, np.nan)
    for i in range(R):
        kstar = None
        for k in range(1, L[i] + 1):
            t = target[i, k - 1].astype(np.float64)
            if T == 0:
                idx, top1, gap = _greedy(t)
                ok = int(idx) == x[i, k - 1]
                tp[i, k - 1] = 1.0 if ok else 0.0
                acc_m[i, k - 1] = gap / max(1.0, abs(top1))
            else:
                p, _, _ = draft_distribution(t, T)
                rho = p[x[i, k - 1]] / q[i, k - 1]
                ok = float(u_accept[i, k - 1]) < rho
                tp[i, k - 1] = p[x[i, k - 1]]
                acc_m[i, k - 1] = abs(float(u_accept[i, k - 1]) - rho)
            if not ok:
                kstar = k
                break
        A[i] = L[i] if kstar is None else kstar - 1
        out[i, :A[i]] = x[i, :A[i]]
        row = target[i, A[i]].astype(np.float64)       # rejected row k*-1, or bonus row L_r
        if T == 0:
            idx, top1, gap = _greedy(row)
            y = int(idx)
            fin_m[i] = gap / max(1.0, abs(top1))
        else:
            p, _, _ = draft_distribution(row, T)
            w = p
            if kstar is not None:
                if states is not None:
                    bias = np.asarray(states[i, kstar - 1], dtype=np.float64) @ W2_64
                else:
                    prev = anchor[i] if kstar == 1 else x[i, kstar - 2]
                    bias = markov_bias(W1_64, W2_64, [prev])[0]
                z = base[i, kstar - 1].astype(np.float64) + bias
                pi, _, _ = draft_distribution(z, T)
                d = np.maximum(0.0, p - pi)
                res_mass[i] = d.sum()
                if res_mass[i] > 0:
                    w = d
            y, fin_m[i], _ = inverse_cdf(w, float(u_final[i]))
        out[i, A[i]] = y
    return dict(out_tokens=out, accept_len=A, target_probs=tp, accept_margin=acc_m,
                final_margin=fin_m, residual_mass=res_mass)


# ---------------------------------------------------------------------------
# whole round and boundary flags


def run_round(inp, T=1.0, use_scheduler=None, scheduler="early", theta=None, head="markov"):
    """Draft -> schedule -> verify on one input dict from ``gen.make_inputs``.

    scheduler: "early" (the early-stop walk), "async" (the production
    variant, with the lagged confidences ``conf_lag``) or "threshold" (the
    static baseline with ``theta``).  head: "markov", or "rnn" (draft_rnn with
    the gate weights ``Wx``, ``Ws``, ``rnn_bias`` of the input dict; verify
    recomputes from the states).
    """
    sched = None
    if use_scheduler is None:
        use_scheduler = inp.get("conf") is not None
    if head == "rnn":
        d = draft_rnn(inp["base"], inp["W1"], inp["W2"], inp["Wx"], inp["Ws"], inp["rnn_bias"], inp["w_dtype"],
                      inp["anchor"], inp["u_draft"], T)
    else:
        d = draft(inp["base"], inp["W1"], inp["W2"], inp["w_dtype"], inp["anchor"], inp["u_draft"], T)
    L = None
    if use_scheduler:
        if scheduler == "async":
            sched = schedule_async(inp["conf"], inp["conf_lag"], inp["sps"])
        elif scheduler == "threshold":
            sched = schedule_threshold(inp["conf"], theta)
        else:
            sched = schedule(inp["conf"], inp["sps"])
        L = sched["verify_len"][inp["rows"]] if "rows" in inp else sched["verify_len"]
    v = verify(inp["target"], inp["base"], inp["W1"], inp["W2"], inp["w_dtype"], inp["anchor"],
               d["tokens"], d["probs"], L, inp["u_accept"], inp["u_final"], T, states=d.get("states"))
    flags = row_flags(d, v)
    return dict(draft=d, schedule=sched, verify=v, flags=flags,
                verify_len=(np.full(len(inp["anchor"]), inp["base"].shape[1], np.int32)
                            if L is None else np.asarray(L, np.int32)))


def row_flags(d, v, eps=FLAG_EPS):
    """Rows whose outcome lies within ``eps`` of a decision boundary.

    Covers every draft event, the accept tests that were evaluated, and the
    final sample.  Such rows are excluded from bit-exact comparison and counted.
    """
    return ((d["margin"] < eps).any(axis=1) | (v["accept_margin"] < eps).any(axis=1)
            | (v["final_margin"] < eps))


# ---------------------------------------------------------------------------
# Per-position acceptance labels ([HADA] Arquitetura, confidence head)


def accept_rates(target, base, W1, W2, w_dtype, anchor, draft_tokens, T):
    """c*_k = 1 - (1/2) || q_k - p_k ||_1 for every request and draft position.

    q_k is the draft distribution at position k given the drafted prefix
    (base row k-1 plus the Markov bias of x_{k-1}, x_0 = anchor), p_k the
    target distribution softmax(target[r, k-1] / T); c*_k is the probability
    that the rejection test accepts position k given the prefix, the analytic
    signal the confidence head is trained on ([HADA] Arquitetura,
    Confidence-Scheduled Verification, confidence head; Treinamento, L_tv).
    T > 0.
    Returns float64 [R, gamma].
    """
    R, g, V = base.shape
    W1_64, W2_64 = widen_weights(W1, w_dtype), widen_weights(W2, w_dtype)
    x = np.asarray(draft_tokens, dtype=np.int64)
    out = np.zeros((R, g))
    for k in range(g):
        prev = np.asarray(anchor, np.int64) if k == 0 else x[:, k - 1]
        z = base[:, k, :].astype(np.float64) + markov_bias(W1_64, W2_64, prev)
        q, _, _ = draft_distribution(z, T)
        p, _, _ = draft_distribution(target[:, k, :].astype(np.float64), T)
        out[:, k] = 1.0 - 0.5 * np.abs(q - p).sum(axis=1)
    return out


# ---------------------------------------------------------------------------
# 4. Sequential temperature scaling  ([HADA] Arquitetura, Confidence-Scheduled
#    Verification, post-hoc calibration; Análise dos experimentos, ECE before
#    and after calibration)


def sts_calibrate(conf, tau):
    """Temperature-scaled confidences c'_{i,k} = sigmoid(logit(c_{i,k}) / tau_k).

    The confidence head ends in a sigmoid, so dividing its logit
    log(c) - log(1 - c) by a per-position temperature is the calibration map
    ([HADA] confidence head: linear projection + sigmoid; STS).  c = 0 and
    c = 1 are fixed points.  conf [N, gamma] in [0, 1], tau [gamma] > 0.
    Returns float64 [N, gamma].
    """
    c = np.asarray(conf, dtype=np.float64)
    with np.errstate(divide="ignore"):
        ell = np.log(c) - np.log1p(-c)
    x = ell / np.asarray(tau, dtype=np.float64)[None, :]
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def ece(pred, target, bins):
    """Expected calibration error over `bins` equal-width bins of [0, 1].

    ECE = sum_b |sum_{i in bin b} (pred_i - target_i)| / N, i.e. the bin
    weight n_b / N times |mean prediction - mean target| in the bin; the bin
    of p is min(floor(p * bins), bins - 1).  Targets may be soft (in [0, 1]).
    """
    p = np.asarray(pred, dtype=np.float64)
    t = np.asarray(target, dtype=np.float64)
    b = np.minimum(np.floor(p * bins).astype(np.int64), bins - 1)
    s = np.bincount(b, weights=p - t, minlength=bins)
    return float(np.abs(s).sum() / len(p))


def sts_fit(conf, labels, grid, bins, follow=None):
    """Left-to-right 1-D grid search of one temperature per draft position.

    Each c_k is a conditional probability, so the survival estimate of a
    prefix is the cumulative product of the calibrated c'_j.  For k = 1..gamma
    in order, with tau_1..tau_{k-1} already fixed, every candidate grid[g] is
    scored by ECE(prod_{j<=k} c'_j, prod_{j<=k} l_j) on the held-out set and
    tau_k is the first minimiser ([HADA] STS: held-out grid search left to
    right minimising ECE, token order preserved).  labels are the conditional
    per-position targets: acceptance rates c*_k from accept_rates, or 0/1
    outcomes (1 while the prefix is accepted).

    conf, labels [N, gamma]; grid [G] candidate temperatures; bins >= 1.
    follow: optional [gamma] grid indices; position k then continues with
    grid[follow[k]] instead of its own minimiser (scores later positions
    after a near-tie).
    Returns dict(tau [gamma], index [gamma], ece [gamma] = score of the index
    used, table [gamma, G] = every candidate's score).
    """
    c = np.asarray(conf, dtype=np.float64)
    lab = np.asarray(labels, dtype=np.float64)
    grid = np.asarray(grid, dtype=np.float64)
    N, g = c.shape
    A = np.ones(N)
    Y = np.ones(N)
    table = np.zeros((g, len(grid)))
    idx = np.zeros(g, dtype=np.int64)
    for k in range(g):
        Y = Y * lab[:, k]
        ck = c[:, k:k + 1]
        for j in range(len(grid)):
            table[k, j] = ece(A * sts_calibrate(ck, grid[j:j + 1])[:, 0], Y, bins)
        idx[k] = int(np.argmin(table[k])) if follow is None else int(follow[k])
        A = A * sts_calibrate(ck, grid[idx[k]:idx[k] + 1])[:, 0]
    return dict(tau=grid[idx], index=idx, ece=table[np.arange(g), idx], table=table)


# ---------------------------------------------------------------------------
# 5. RNN head  ([HADA] Arquitetura, Semi-Autoregressive Generation, RNN head;
#    Experimentos, proposal length: small extra gain at long blocks)


def to_storage(x, w_dtype):
    """Round float64 values once to the storage type (nearest, ties to even)
    and return them as float64: fp32, or bf16 (8 significant bits over the
    exponent range of fp32; below 2^-126 the spacing stays 2^-133)."""
    x = np.asarray(x, dtype=np.float64)
    if w_dtype != "bf16":
        return x.astype(np.float32).astype(np.float64)
    _, e = np.frexp(x)                        # x = m 2^e with 1/2 <= |m| < 1
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def rnn_state_update(e, s, Wx_64, Ws_64, b_64, w_dtype):
    """One gated update of the recurrent state (GRU form, Cho et al. 2014):

      u = sigmoid(e Wx[0] + s Ws[0] + b[0])        update gate
      g = sigmoid(e Wx[1] + s Ws[1] + b[1])        reset gate
      h = tanh(e Wx[2] + (g * s) Ws[2] + b[2])     candidate
      s' = storage((1 - u) * s + u * h)

    e [R, r] the previous token's input row, s [R, r] the state; the new state
    is carried in the weights' storage type.  The pages describe the head as a
    recurrent state over the whole in-block prefix with a gated update and give
    no equations; this is the plainest gated recurrence.
    """
    u = _sigmoid(e @ Wx_64[0] + s @ Ws_64[0] + b_64[0])
    g = _sigmoid(e @ Wx_64[1] + s @ Ws_64[1] + b_64[1])
    h = np.tanh(e @ Wx_64[2] + (g * s) @ Ws_64[2] + b_64[2])
    return to_storage((1.0 - u) * s + u * h, w_dtype)


def _rnn_params(W1, Wx, Ws, bias, w_dtype):
    r = np.asarray(Wx).shape[-1]
    return (widen_weights(W1, w_dtype), widen_weights(Wx, w_dtype).reshape(3, r, r),
            widen_weights(Ws, w_dtype).reshape(3, r, r),
            np.asarray(bias, dtype=np.float32).astype(np.float64).reshape(3, r))


def draft_rnn(base, W1, W2, Wx, Ws, bias, w_dtype, anchor, u_draft, T):
    """Sequential drafting with the RNN head.

    The state s_k accumulates the in-block prefix x_0..x_{k-1} (x_0 = anchor,
    s_0 = 0, input row e = W1[x_{k-1}], rnn_state_update), and the transition
    bias at position k is s_k @ W2, added to base row k; sampling as in draft.
    Wx, Ws [3, r, r] (input and recurrent weights of the update, reset and
    candidate gates, same storage as W1/W2), bias [3, r] fp32.
    Returns draft's dict plus states [R, gamma, r] (float64 values of s_1..s_gamma,
    exact in the storage type).
    """
    R, g, V = base.shape
    W1_64, Wx_64, Ws_64, b_64 = _rnn_params(W1, Wx, Ws, bias, w_dtype)
    W2_64 = widen_weights(W2, w_dtype)
    states = np.zeros((R, g, W1_64.shape[1]))
    cur = {"s": np.zeros((R, W1_64.shape[1]))}

    def bias_of(k, prev):
        cur["s"] = rnn_state_update(W1_64[prev], cur["s"], Wx_64, Ws_64, b_64, w_dtype)
        states[:, k] = cur["s"]
        return cur["s"] @ W2_64

    out = _draft_loop(base, u_draft, T, anchor, bias_of)
    out["states"] = states
    return out
