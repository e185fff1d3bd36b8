"""GPU parity of the one-launch drafts (all gamma steps in one kernel).

dspark_draft runs the persistent one-launch kernel where it applies (bf16
factors, rank 16/32/64/128/256, at most two 256-column tiles per compute unit,
R <= 1024), else, for small problems, one launch of one workgroup per request;
DSPARK_DRAFT_KERNEL=stepwise selects the per-step kernels instead.  All do the
same arithmetic in the same order, so their outputs must be bit-identical; all
must match the float64 oracle on every request whose draws are not within
1e-6 of a CDF boundary.  The launch hook tells which kernel ran.
"""

import ctypes

import numpy as np
import pytest
import torch

import draft_sampling_verify_markov_amd as D
import oracle as O
from gen import make_inputs, config

from gpu_util import ATOL, RTOL, dev, say, to_dev

pytestmark = pytest.mark.gpu

KID_DRAFT_FUSED = 8
KID_DRAFT_ROWS = 9


def _draft(inp, T, kernel, monkeypatch, ws=None, d=None, kid=KID_DRAFT_FUSED):
    if kernel == "stepwise":
        monkeypatch.setenv("DSPARK_DRAFT_KERNEL", "stepwise")
    else:
        monkeypatch.delenv("DSPARK_DRAFT_KERNEL", raising=False)
    d = d or to_dev(inp)
    R, g, V = inp["base"].shape
    r = inp["W1"].shape[1]
    ws = ws if ws is not None else D.new_workspace(R, g, V, r, dev())
    lib = D.load_library()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    arr_s = (ctypes.c_void_p * 1)(ev[0].cuda_event)
    arr_e = (ctypes.c_void_p * 1)(ev[1].cuda_event)
    assert lib.dspark_profile_arm(kid, arr_s, arr_e, 1, 1) == 0
    try:
        tok, prob, stats = D.draft(d["base"], d["W1"], d["W2"], d["anchor"], d["u_draft"], T, ws)
        torch.cuda.synchronize()
    finally:
        fused_launches = lib.dspark_profile_disarm()
    err = D.device_error(ws)
    return dict(tokens=tok.cpu().numpy(), probs=prob.cpu().numpy(), stats=stats.cpu().numpy(),
                err=err, fused=fused_launches == 1)


def _oracle_check(inp, T, got, label):
    ref = O.draft(inp["base"], inp["W1"], inp["W2"], inp["w_dtype"], inp["anchor"], inp["u_draft"], T)
    near = ref["margin"] < O.FLAG_EPS
    ok = ~near.any(axis=1)
    say(f"[{label}] requests {len(ok)}, flagged {int((~ok).sum())}")
    bad = np.flatnonzero(ok & (got["tokens"] != ref["tokens"]).any(axis=1))
    assert len(bad) == 0, f"{label}: tokens differ from the oracle on unflagged requests {bad[:10]}"
    # flagged requests agree up to their first near-boundary draw
    first = np.where(near.any(axis=1), near.argmax(axis=1), near.shape[1])
    for i in np.flatnonzero(~ok):
        assert (got["tokens"][i, :first[i]] == ref["tokens"][i, :first[i]]).all(), f"{label}: request {i}"
    np.testing.assert_allclose(got["probs"][ok], ref["probs"][ok], atol=ATOL, rtol=RTOL, err_msg=label + " q")
    np.testing.assert_allclose(got["stats"][ok], ref["stats"][ok], atol=ATOL, rtol=RTOL, err_msg=label + " stats")


SHAPES = [
    (1, 1, 256, 16),        # one request, one tile
    (5, 3, 1000, 16),       # ragged vocabulary tail
    (33, 2, 520, 32),       # a second 32-row block
    (130, 2, 776, 64),      # two 128-request chunks
    (3, 16, 2048, 256),     # longest block, full rank
    (300, 3, 4096, 128),    # more requests than compute units: two draws per workgroup
    (20, 3, 100000, 32),    # between one and two tiles per workgroup
    (64, 4, 131072, 256),   # two tiles on every workgroup
    (1024, 2, 4096, 32),    # the largest request count: eight chunks, four draws per workgroup
]


@pytest.mark.parametrize("T", [1.0, 0.0, 0.7])
@pytest.mark.parametrize("R,g,V,r", SHAPES)
def test_one_launch_draft_matches_stepwise_and_oracle(R, g, V, r, T, monkeypatch):
    cfg = config(1, R=R, gamma=g, V=V, r=r, w_dtype="bf16", table="linear")
    inp = make_inputs(cfg, seed=1000 + R + g, seed_u=R)
    label = f"draft {R},{g},{V},{r} T={T}"
    say(f"[{label}] one-launch draft")
    a = _draft(inp, T, "fused", monkeypatch)
    assert a["fused"], "the one-launch draft did not run"
    assert a["err"] == 0, f"device error bits {a['err']}"
    say(f"[{label}] per-step draft")
    b = _draft(inp, T, "stepwise", monkeypatch)
    assert not b["fused"]
    assert b["err"] == 0
    for key in ("tokens", "probs", "stats"):
        assert np.array_equal(a[key], b[key]), f"{label}: {key} differ between the two kernels"
    _oracle_check(inp, T, a, label)


@pytest.mark.parametrize("R,g,V,r", [
    (8, 2, 131328, 32),     # 513 tiles: more than the one-launch draft holds
    (1025, 1, 1024, 32),    # more requests than it holds
    (16, 3, 4096, 48),      # a rank it has no kernel for
])
def test_outside_the_one_launch_limits(R, g, V, r, monkeypatch):
    """Outside its limits dspark_draft takes another path by itself (the
    per-request kernel for small problems, else the per-step kernels)."""
    cfg = config(1, R=R, gamma=g, V=V, r=r, w_dtype="bf16", table="linear")
    inp = make_inputs(cfg, seed=500 + R, seed_u=g)
    label = f"draft {R},{g},{V},{r}"
    say(f"[{label}] default path")
    a = _draft(inp, 1.0, "fused", monkeypatch)
    assert not a["fused"], "the one-launch draft ran outside its limits"
    assert a["err"] == 0
    _oracle_check(inp, 1.0, a, label)


# Small problems the one-launch draft does not take (fp32 factors, ranks it
# has no kernel for) run in one launch of one workgroup per request: the same
# per-row arithmetic as the per-step kernels, so bit-identical outputs.
@pytest.mark.parametrize("T", [1.0, 0.0, 0.7])
@pytest.mark.parametrize("R,g,V,r,w", [
    (4, 4, 512, 16, "f32"),      # the tiny workload's shape
    (5, 3, 1000, 16, "f32"),     # ragged vocabulary tail
    (33, 5, 264, 48, "f32"),     # more requests than a 32-row block, rank 48
    (3, 16, 1024, 16, "f32"),    # four tiles, the longest block
    (16, 3, 4096, 48, "bf16"),   # sixteen tiles, a rank the one-launch draft has no kernel for
])
def test_per_request_draft_matches_stepwise_and_oracle(R, g, V, r, w, T, monkeypatch):
    cfg = config(1, R=R, gamma=g, V=V, r=r, w_dtype=w, table="linear")
    inp = make_inputs(cfg, seed=2000 + R + g, seed_u=R + 1)
    label = f"per-request draft {R},{g},{V},{r},{w} T={T}"
    say(f"[{label}] default path")
    a = _draft(inp, T, "default", monkeypatch, kid=KID_DRAFT_ROWS)
    assert a["fused"], "the per-request draft did not run"
    assert a["err"] == 0, f"device error bits {a['err']}"
    b = _draft(inp, T, "stepwise", monkeypatch, kid=KID_DRAFT_ROWS)
    assert not b["fused"]
    assert b["err"] == 0
    for key in ("tokens", "probs", "stats"):
        assert np.array_equal(a[key], b[key]), f"{label}: {key} differ from the per-step kernels"
    _oracle_check(inp, T, a, label)


def test_repeated_calls_on_one_workspace(monkeypatch):
    """The step tags advance with a per-workspace epoch: back-to-back calls
    with different uniforms (and a greedy call between them) must each give
    the per-step kernels' result."""
    cfg = config(1, R=48, gamma=5, V=8192, r=64, w_dtype="bf16", table="linear")
    ws = D.new_workspace(48, 5, 8192, 64, dev())
    for i, (seed_u, T) in enumerate([(0, 1.0), (1, 0.0), (2, 1.0), (3, 0.7), (4, 1.0)]):
        inp = make_inputs(cfg, seed=77, seed_u=seed_u)
        say(f"[repeat {i}] seed_u={seed_u} T={T}")
        a = _draft(inp, T, "fused", monkeypatch, ws=ws)
        assert a["fused"] and a["err"] == 0
        b = _draft(inp, T, "stepwise", monkeypatch)
        for key in ("tokens", "probs", "stats"):
            assert np.array_equal(a[key], b[key]), f"call {i}: {key}"


def test_new_workspace_over_a_used_one(monkeypatch):
    """A workspace allocated where an earlier one lived starts its epoch at
    zero again, so the earlier call's sealed records carry tags the new calls
    will look for: dspark_workspace_init must clear them.  Two workspaces at
    the same address, different inputs: each call gives the per-step result."""
    cfg = config(1, R=64, gamma=3, V=16384, r=128, w_dtype="bf16", table="linear")
    ptrs = []
    for i in range(3):
        ws = D.new_workspace(64, 3, 16384, 128, dev())
        ptrs.append(ws.data_ptr())
        inp = make_inputs(cfg, seed=300 + i, seed_u=i)
        say(f"[reuse {i}] workspace at {ws.data_ptr():#x}")
        a = _draft(inp, 1.0, "fused", monkeypatch, ws=ws)
        assert a["fused"] and a["err"] == 0
        b = _draft(inp, 1.0, "stepwise", monkeypatch)
        for key in ("tokens", "probs", "stats"):
            assert np.array_equal(a[key], b[key]), f"workspace {i}: {key}"
        del ws
        torch.cuda.synchronize()
    say(f"[reuse] distinct workspace addresses: {len(set(ptrs))} of {len(ptrs)}")


def test_wait_time_out_sets_sync_error(monkeypatch):
    """With a time limit of 0 ticks (DSPARK_FUSED_SPIN_TICKS=0) every wait of
    the one-launch draft that does not succeed at once gives up: the call must
    still end, report DSPARK_DERR_SYNC, and leave the workspace usable (the
    next call, with the normal limit, gives the per-step kernels' result)."""
    cfg = config(1, R=64, gamma=4, V=65536, r=128, w_dtype="bf16", table="linear")
    inp = make_inputs(cfg, seed=41)
    ws = D.new_workspace(64, 4, 65536, 128, dev())
    monkeypatch.setenv("DSPARK_FUSED_SPIN_TICKS", "0")
    say("[time-out] draft with a zero time limit")
    a = _draft(inp, 1.0, "fused", monkeypatch, ws=ws)
    assert a["fused"]
    assert a["err"] & 128, f"expected the SYNC error bit, got {a['err']}"
    monkeypatch.delenv("DSPARK_FUSED_SPIN_TICKS")
    say("[time-out] the same workspace with the normal limit")
    a = _draft(inp, 1.0, "fused", monkeypatch, ws=ws)
    assert a["fused"] and a["err"] == 0
    b = _draft(inp, 1.0, "stepwise", monkeypatch)
    for key in ("tokens", "probs", "stats"):
        assert np.array_equal(a[key], b[key]), key


def test_checked_round_raises_on_sync_error(monkeypatch):
    """run_round(check=True) reads both error words after the round: a round
    whose one-launch draft gave up waiting (time limit 0) raises DSparkError
    naming SYNC; the same round with the normal limit returns its outputs and
    leaves both error words clear."""
    monkeypatch.delenv("DSPARK_DRAFT_KERNEL", raising=False)
    cfg = config(1, R=64, gamma=4, V=65536, r=128, w_dtype="bf16", table="linear")
    inp = make_inputs(cfg, seed=43)
    d = to_dev(inp)
    ws = D.new_workspace(64, 4, 65536, 128, dev())
    monkeypatch.setenv("DSPARK_FUSED_SPIN_TICKS", "0")
    say("[checked] round with a zero time limit")
    with pytest.raises(D.DSparkDeviceError, match="SYNC"):
        D.run_round(d, 1.0, ws, check=True)
    monkeypatch.delenv("DSPARK_FUSED_SPIN_TICKS")
    say("[checked] round with the normal limit")
    out = D.run_round(d, 1.0, ws, check=True)
    assert D.device_error(ws) == 0 and D.device_error(out["ws_sched"]) == 0
    assert (out["accept_len"] >= 0).all().item()


def test_one_launch_draft_in_a_graph(monkeypatch):
    """Captured once, replayed several times with eager work in between: every
    replay gives the eager result."""
    monkeypatch.delenv("DSPARK_DRAFT_KERNEL", raising=False)
    cfg = config(1, R=32, gamma=4, V=16384, r=256, w_dtype="bf16", table="linear")
    inp = make_inputs(cfg, seed=5)
    d = to_dev(inp)
    ws = D.new_workspace(32, 4, 16384, 256, dev())
    eager = D.draft(d["base"], d["W1"], d["W2"], d["anchor"], d["u_draft"], 1.0, ws)
    eager = [t.clone() for t in eager]
    out = tuple(torch.empty_like(t) for t in eager)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        D.draft(d["base"], d["W1"], d["W2"], d["anchor"], d["u_draft"], 1.0, ws, out=out)
    for rep in range(4):
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(out, eager):
            assert torch.equal(x, y), f"replay {rep}"
        # eager call in between (advances the epoch outside the graph)
        D.draft(d["base"], d["W1"], d["W2"], d["anchor"], d["u_draft"], 1.0, ws)
        torch.cuda.synchronize()
    assert D.device_error(ws) == 0
