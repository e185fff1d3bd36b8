"""Helpers of the GPU parity tests: device transfer and oracle comparison."""

import sys

import numpy as np
import torch

import draft_sampling_verify_markov_amd as D
import oracle as O

ATOL, RTOL = 1e-4, 1e-5   # floating-point parity bar for probabilities and statistics


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def w_to_dev(w, w_dtype, device):
    if w_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(device)


def to_dev(inp, device=None):
    device = device or dev()
    t = lambda a, dt=None: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(device)
    return dict(base=t(inp["base"], np.float32), target=t(inp["target"], np.float32),
                W1=w_to_dev(inp["W1"], inp["w_dtype"], device),
                W2=w_to_dev(inp["W2"], inp["w_dtype"], device),
                anchor=t(inp["anchor"], np.int32), u_draft=t(inp["u_draft"], np.float32),
                u_accept=t(inp["u_accept"], np.float32), u_final=t(inp["u_final"], np.float32),
                conf=t(inp["conf"], np.float32), sps=t(inp["sps"], np.float32),
                **({} if "Wx" not in inp else dict(Wx=w_to_dev(inp["Wx"], inp["w_dtype"], device),
                                                   Ws=w_to_dev(inp["Ws"], inp["w_dtype"], device),
                                                   rnn_bias=t(inp["rnn_bias"], np.float32))))


def gpu_round(inp, T, use_scheduler=None, device=None, head="markov"):
    d = to_dev(inp, device)
    R, g, V = inp["base"].shape
    r = inp["W1"].shape[1]
    ws = D.new_workspace(R, g, V, r, d["base"].device)
    if use_scheduler is None:
        use_scheduler = inp.get("conf") is not None
    out = D.run_round(d, T, ws, use_scheduler=use_scheduler, head=head)
    torch.cuda.synchronize()
    err = D.device_error(ws)
    if out["ws_sched"] is not None:
        err |= D.device_error(out["ws_sched"])
    res = {k: ((v.float() if v.dtype == torch.bfloat16 else v).cpu().numpy() if isinstance(v, torch.Tensor) else v)
           for k, v in out.items() if k != "ws_sched"}
    res["device_error"] = err
    return res


class Parity(int):
    """Result of compare_rounds: behaves as the flagged-row count (an int) and
    carries the full tally in ``.counts``."""

    def __new__(cls, counts):
        obj = super().__new__(cls, counts["flagged"])
        obj.counts = counts
        return obj


def compare_rounds(orc, gpu, rows=None, label=""):
    """Compare an oracle round with the GPU round on (a subset of) rows.

    orc comes from oracle.run_round on the rows given (or all rows); gpu holds
    whole-workload arrays, restricted to ``rows``.  Integer outputs must match
    exactly on rows the oracle does not flag; probabilities and statistics
    within ATOL/RTOL.  On flagged rows the draft must agree up to the first
    event near a boundary, and the probabilities and statistics are compared
    over the prefix whose tokens agree (all of it when the row matches).
    Returns a Parity: the flagged-row count, with ``.counts`` = dict(rows,
    flagged, flagged_mismatch, unflagged_mismatch).
    """
    sel = slice(None) if rows is None else np.asarray(rows)
    g_tok = gpu["draft_tokens"][sel]
    g_prob = gpu["draft_probs"][sel]
    g_stats = gpu["draft_stats"][sel]
    g_out = gpu["out_tokens"][sel]
    g_acc = gpu["accept_len"][sel]
    g_tp = gpu["target_probs"][sel]
    flags = orc["flags"]
    ok = ~flags
    n_flag = int(flags.sum())
    d = orc["draft"]
    v = orc["verify"]
    same = ((g_out == v["out_tokens"]).all(axis=1) & (g_tok == d["tokens"]).all(axis=1)
            & (g_acc == v["accept_len"]))
    counts = dict(rows=int(len(flags)), flagged=n_flag, flagged_mismatch=int((~same & flags).sum()),
                  unflagged_mismatch=int((~same & ok).sum()))
    say(f"[{label}] rows compared {counts['rows']}, flagged {n_flag}, "
        f"flagged rows that differ {counts['flagged_mismatch']}")
    bad_tok = np.flatnonzero(ok & (g_tok != d["tokens"]).any(axis=1))
    assert len(bad_tok) == 0, f"{label}: draft tokens differ on unflagged rows {bad_tok[:10]}"
    if orc["schedule"] is not None and gpu.get("verify_len") is not None:
        gL = gpu["verify_len"][sel]
        assert (gL == orc["verify_len"]).all(), f"{label}: verify lengths differ"
    bad_acc = np.flatnonzero(ok & (g_acc != v["accept_len"]))
    assert len(bad_acc) == 0, f"{label}: accept_len differs on rows {bad_acc[:10]}"
    bad_out = np.flatnonzero(ok & (g_out != v["out_tokens"]).any(axis=1))
    assert len(bad_out) == 0, f"{label}: out_tokens differ on rows {bad_out[:10]}"
    assert counts["unflagged_mismatch"] == 0
    # flagged rows: the draft must still agree up to the first event near a boundary
    dflag = d["margin"] < O.FLAG_EPS
    g_len = dflag.shape[1]
    first = np.where(dflag.any(axis=1), dflag.argmax(axis=1), g_len)
    for i in np.flatnonzero(flags):
        assert (g_tok[i, :first[i]] == d["tokens"][i, :first[i]]).all(), f"{label}: row {i} prefix"
    # every flagged request that differs must depart from the oracle at an
    # event that is itself within FLAG_EPS of its boundary
    flips = []
    for i in np.flatnonzero(flags & ~same):
        if (g_tok[i] != d["tokens"][i]).any():
            j = int(np.argmax(g_tok[i] != d["tokens"][i]))
            ev, m = f"draft position {j + 1}", float(d["margin"][i, j])
        elif g_acc[i] != v["accept_len"][i]:
            j = int(min(g_acc[i], v["accept_len"][i]))
            ev, m = f"accept test {j + 1}", float(v["accept_margin"][i, j])
        else:
            ev, m = "final sample", float(v["final_margin"][i])
        flips.append(m)
        say(f"[{label}] request {i} departs at the {ev}, margin {m:.3e}")
        assert m < O.FLAG_EPS, f"{label}: request {i} departs at an unflagged event ({ev}, margin {m:.3e})"
    counts["max_flip_margin"] = max(flips) if flips else None
    # probabilities and statistics: every position of a matching row; on a
    # row whose draft differs, the statistics up to the first differing token
    # (they depend on the tokens before it) and q up to the token before it
    tok_eq = (g_tok == d["tokens"])
    n_eq = np.where(tok_eq.all(axis=1), g_len, tok_eq.argmin(axis=1))
    k = np.arange(g_len)[None, :]
    m_stats = k <= n_eq[:, None]
    m_q = k < n_eq[:, None]
    np.testing.assert_allclose(g_prob[m_q], d["probs"][m_q], atol=ATOL, rtol=RTOL, err_msg=label + " q")
    np.testing.assert_allclose(g_stats[m_stats], d["stats"][m_stats], atol=ATOL, rtol=RTOL,
                               err_msg=label + " stats")
    np.testing.assert_allclose(g_tp[same], v["target_probs"][same], atol=ATOL, rtol=RTOL, err_msg=label + " p")
    return Parity(counts)
