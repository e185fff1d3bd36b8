"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole round runs on the GPU, and the oracle recomputes a
sample of request rows one by one (the scheduler is global, so the oracle runs
it on all confidences).  Whole-workload properties are checked on every row.
"""

import numpy as np
import pytest

import oracle as O
from gen import make_inputs, config

from gpu_util import compare_rounds, gpu_round, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _rows(R, n, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(R, size=min(n, R), replace=False).tolist()) | {0, R - 1}
    return sorted(pick)


def _whole_round_properties(gpu, d):
    R, g = d["R"], d["gamma"]
    L = gpu["verify_len"] if gpu["verify_len"] is not None else np.full(R, g)
    A = gpu["accept_len"]
    out = gpu["out_tokens"]
    assert ((0 <= A) & (A <= L)).all()
    for r in range(R):
        a = A[r]
        assert (out[r, :a] == gpu["draft_tokens"][r, :a]).all()
        assert 0 <= out[r, a] < d["V"]
        assert (out[r, a + 1:] == -1).all()
    if gpu.get("n_admitted") is not None:
        assert int(gpu["n_admitted"][0]) == int(L.sum())
    tp = gpu["target_probs"]
    lim = np.minimum(L, A + 1)
    k = np.arange(1, g + 1)[None, :]
    assert (tp[k > lim[:, None]] == -1).all()
    assert ((tp[k <= lim[:, None]] >= 0) & (tp[k <= lim[:, None]] <= 1)).all()


@pytest.mark.parametrize("cfg,T,nrows", [(3, 1.0, 40), (4, 1.0, 16), (4, 0.0, 16), (5, 1.0, 24)])
def test_fullsize_sampled_rows(cfg, T, nrows):
    d = config(cfg)
    say(f"[cfg {cfg} T={T}] generating R={d['R']} gamma={d['gamma']} V={d['V']}")
    inp = make_inputs(cfg)
    gpu = gpu_round(inp, T)
    assert gpu["device_error"] == 0
    _whole_round_properties(gpu, d)
    del inp
    rows = _rows(d["R"], nrows, cfg)
    sub = make_inputs(cfg, rows=rows)
    orc = O.run_round(sub, T=T)
    n_flag = compare_rounds(orc, gpu, rows=rows, label=f"cfg {cfg} T={T}")
    A = gpu["accept_len"]
    say(f"[cfg {cfg} T={T}] mean accepted {A.mean():.3f}, tokens/round {int((A + 1).sum())}, "
        f"flagged {n_flag}/{len(rows)}")
