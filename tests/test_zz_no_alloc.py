"""dspark_draft_noalloc (the draft without a workspace, on the library's static
device scratch) against dspark_draft through the C ABI: identical outputs on
two calls in a row, the second smaller than the first, on the one-launch path
(bf16 factors) and the per-step path (fp32 factors), sampling and greedy; the
error word it writes stays clear; unflagged rows also match the oracle."""

import numpy as np
import pytest
import torch

import draft_sampling_verify_markov_amd as D
import oracle as O
from gen import make_inputs, config

from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _both(d, seed, T):
    inp = make_inputs(d, seed=seed)
    dd = to_dev(inp)
    dev = dd["base"].device
    R, g, V = inp["base"].shape
    r = inp["W1"].shape[1]
    ws = D.new_workspace(R, g, V, r, dev)
    ref = D.draft(dd["base"], dd["W1"], dd["W2"], dd["anchor"], dd["u_draft"], T, ws)
    out = (torch.full((R, g), -7, dtype=torch.int32, device=dev),
           torch.full((R, g), -7.0, dtype=torch.float32, device=dev),
           torch.full((R, g, 2), -7.0, dtype=torch.float32, device=dev))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    D.draft_noalloc(dd["base"], dd["W1"], dd["W2"], dd["anchor"], dd["u_draft"], T, err, out)
    torch.cuda.synchronize()
    assert D.device_error(ws) == 0
    assert int(err.cpu()[0]) == 0, f"device error bits {int(err.cpu()[0])}"
    for a, b, name in zip(out, ref, ("tokens", "probs", "stats")):
        assert torch.equal(a, b), f"{name} differ from dspark_draft"
    orc = O.draft(inp["base"], inp["W1"], inp["W2"], inp["w_dtype"], inp["anchor"], inp["u_draft"], T)
    ok = ~(orc["margin"] < O.FLAG_EPS).any(axis=1)
    assert (out[0].cpu().numpy()[ok] == orc["tokens"][ok]).all()
    np.testing.assert_allclose(out[1].cpu().numpy()[ok], orc["probs"][ok], atol=1e-4, rtol=1e-5)
    say(f"  noalloc draft R={R} gamma={g} V={V} r={r} {inp['w_dtype']} T={T}: equal to dspark_draft, "
        f"{int(ok.sum())}/{R} unflagged rows equal to the oracle")


@pytest.mark.parametrize("T", [1.0, 0.0])
@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
def test_noalloc_draft_equals_workspace_draft_twice(w_dtype, T):
    big = config(1, w_dtype=w_dtype, R=96, gamma=6, V=32768, r=256)
    small = config(1, w_dtype=w_dtype, R=20, gamma=3, V=4104, r=64)
    _both(big, 5, T)
    _both(small, 6, T)
