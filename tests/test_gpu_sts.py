"""GPU parity of sequential temperature scaling (dspark_sts_fit, dspark_sts_apply)
against the float64 oracle.

Bar: every candidate's score (ECE) within 1e-9 absolute of the oracle, scored
after the same earlier choices; the chosen grid index equal to the oracle's
first minimiser unless the oracle's scores of the two entries are within 1e-9
of each other (a near-tie, counted as flagged).  Calibrated confidences from
dspark_sts_apply within one fp32 ulp of the oracle's fp64 map.
"""

import json
import os

import numpy as np
import pytest
import torch

import draft_sampling_verify_markov_amd as D
import oracle as O
from gen.sts import make_sts_inputs

from gpu_util import dev, say

pytestmark = pytest.mark.gpu

ECE_TOL = 1e-9
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _t(a, dt=np.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev())


def _fit(conf, lab, grid, bins):
    N, g = conf.shape
    ws = D.new_sts_workspace(N, g, len(grid), bins, dev())
    tau, idx, ece, table = D.sts_fit(_t(conf), _t(lab), _t(grid), bins, ws, with_table=True)
    torch.cuda.synchronize()
    err = D.device_error(ws)
    return (tau.cpu().numpy(), idx.cpu().numpy().astype(np.int64), ece.cpu().numpy(), table.cpu().numpy(),
            err)


def _compare(conf, lab, grid, bins, bad_cols=()):
    """Fit on the GPU and check it against the oracle; returns (index, flagged)."""
    conf = np.asarray(conf, np.float32)
    lab = np.asarray(lab, np.float32)
    grid = np.asarray(grid, np.float32)
    N, g = conf.shape
    say(f"sts fit N={N} gamma={g} G={len(grid)} bins={bins}")
    tau, idx, ece, table, err = _fit(conf, lab, grid, bins)
    ok_cols = np.array([j for j in range(len(grid)) if j not in bad_cols], dtype=np.int64)
    assert err == (64 if bad_cols else 0)
    # score every position after the GPU's own earlier choices
    # (the library clamps out-of-range values into [0, 1], NaN to 0; the
    # columns of invalid temperatures are excluded, so any finite value
    # stands in for them on the oracle side)
    grid_o = grid.astype(np.float64)
    grid_o[list(bad_cols)] = 1.0
    ref = O.sts_fit(np.clip(np.nan_to_num(conf, nan=0.0), 0, 1), np.clip(np.nan_to_num(lab, nan=0.0), 0, 1),
                    grid_o, bins, follow=idx)
    for j in bad_cols:
        assert np.isinf(table[:, j]).all()
    np.testing.assert_allclose(table[:, ok_cols], ref["table"][:, ok_cols], rtol=0, atol=ECE_TOL)
    flagged = 0
    for k in range(g):
        row = ref["table"][k][ok_cols]
        first = int(ok_cols[np.argmin(row)])
        if idx[k] != first:
            assert ref["table"][k][idx[k]] - row.min() <= ECE_TOL, (k, idx[k], first)
            flagged += 1
    assert np.array_equal(tau, grid[idx])
    assert np.array_equal(ece, table[np.arange(g), idx])
    return idx, flagged


def test_sts_worked_example_gpu():
    gd = json.load(open(os.path.join(GOLD, "sts_worked_example.json")))
    idx, flagged = _compare(np.array(gd["conf"]), np.array(gd["labels"]), np.array(gd["grid"]), gd["bins"])
    assert list(idx) == gd["index"] and flagged == 0


def test_sts_planted_temperatures_gpu():
    grid = np.array([0.5, 0.75, 1.0, 1.5, 2.0, 3.0], np.float32)
    rng = np.random.default_rng(21)
    s_idx = rng.integers(0, len(grid), 6)
    t = rng.normal(1.0, 1.5, (6000, 6))
    lab = 1.0 / (1.0 + np.exp(-t))
    conf = 1.0 / (1.0 + np.exp(-(grid[s_idx].astype(np.float64)[None, :] * t)))
    idx, flagged = _compare(conf, lab, grid, 15)
    assert np.array_equal(idx, s_idx) and flagged == 0


@pytest.mark.parametrize("N,g,G,bins", [
    (3000, 7, 64, 15),
    (2049, 3, 17, 1),
    (4351, 16, 33, 64),
    (1, 1, 1, 1),
    (70000, 2, 40, 16),
    (5000, 4, 1024, 17),
    (257, 5, 3, 2),
])
def test_sts_synthetic_shapes(N, g, G, bins):
    d = make_sts_inputs(N, g, G, bins, seed=N + g)
    idx, flagged = _compare(d["conf"], d["labels"], d["grid"], bins)
    say(f"  chosen {[int(i) for i in idx]} flagged {flagged}")


def test_sts_held_out_65536_blocks():
    """The calibration workload timed by the benchmark: 65536 held-out blocks of
    gamma = 7, 256 candidate temperatures, 15 bins."""
    d = make_sts_inputs(65536, 7, 256, 15, seed=0)
    idx, flagged = _compare(d["conf"], d["labels"], d["grid"], 15)
    assert flagged == 0
    # calibration lowers the cumulative ECE at every position (tau = 1 is not
    # in the grid, so compare with the uncalibrated product directly)
    raw = np.cumprod(d["conf"].astype(np.float64), axis=1)
    y = np.cumprod(d["labels"].astype(np.float64), axis=1)
    tau, _, ece, _, _ = _fit(d["conf"], d["labels"], d["grid"], 15)
    for k in range(7):
        assert ece[k] < O.ece(raw[:, k], y[:, k], 15)


def test_sts_deterministic_and_repeatable():
    d = make_sts_inputs(9000, 5, 100, 12, seed=3)
    a = _fit(d["conf"], d["labels"], d["grid"], 12)
    b = _fit(d["conf"], d["labels"], d["grid"], 12)
    for x, y in zip(a[:4], b[:4]):
        assert np.array_equal(x, y)


def test_sts_out_of_range_inputs():
    d = make_sts_inputs(3000, 4, 20, 10, seed=5)
    conf, lab, grid = d["conf"].copy(), d["labels"].copy(), d["grid"].copy()
    lab[7, 1] = np.nan
    conf[11, 2] = -0.25
    conf[12, 0] = 1.5
    grid[4] = -1.0
    grid[9] = np.inf
    idx, _ = _compare(conf, lab, grid, 10, bad_cols=(4, 9))
    assert 4 not in idx and 9 not in idx


def test_sts_apply_matches_the_map():
    d = make_sts_inputs(4000, 7, 64, 15, seed=8)
    tau, _, _, _, _ = _fit(d["conf"], d["labels"], d["grid"], 15)
    conf = d["conf"][:1000].copy()
    conf[0, :] = 0.0
    conf[1, :] = 1.0
    ws = D.new_workspace(4, 4, 512, 16, dev())
    out = D.sts_apply(_t(conf), _t(tau), ws).cpu().numpy()
    assert D.device_error(ws) == 0
    want = O.sts_calibrate(conf, tau.astype(np.float64))
    ulp = np.spacing(want.astype(np.float32))
    assert (np.abs(out.astype(np.float64) - want) <= ulp).all()
    assert (out[0] == 0).all() and (out[1] == 1).all()
    # in place, and a bad temperature leaves its column unchanged and flags it
    c_t = _t(conf)
    bad = tau.copy()
    bad[3] = 0.0
    D.sts_apply(c_t, _t(bad), ws, out=c_t)
    got = c_t.cpu().numpy()
    assert D.device_error(ws) == 64
    assert np.array_equal(got[:, 3], conf[:, 3])
    keep = [k for k in range(7) if k != 3]
    assert np.array_equal(got[:, keep], out[:, keep])


def test_calibrated_confidences_drive_the_scheduler():
    """Calibrate a batch of confidences and schedule on them: the GPU scheduler
    on the GPU's calibrated values equals the oracle scheduler on the same values,
    and those values are the oracle's map to within one ulp."""
    from gen import make_inputs
    inp = make_inputs(3, rows=[0], with_target=False)   # confidences and table only
    R, g = inp["conf"].shape
    d = make_sts_inputs(8192, g, 64, 15, seed=11)
    tau, _, _, _, _ = _fit(d["conf"], d["labels"], d["grid"], 15)
    ws = D.new_workspace(R, g, 512, 16, dev())
    cal = D.sts_apply(_t(inp["conf"]), _t(tau), ws)
    L, n, a = D.schedule(cal, _t(inp["sps"]), torch.zeros(256, dtype=torch.uint8, device=dev()))
    torch.cuda.synchronize()
    cal_h = cal.cpu().numpy()
    want = O.sts_calibrate(inp["conf"], tau.astype(np.float64))
    assert (np.abs(cal_h.astype(np.float64) - want) <= np.spacing(want.astype(np.float32))).all()
    ref = O.schedule(cal_h, inp["sps"])
    assert np.array_equal(L.cpu().numpy(), ref["verify_len"]) and int(n.cpu()[0]) == ref["n_admitted"]
