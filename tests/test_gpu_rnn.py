"""GPU parity of the RNN head (dspark_draft_rnn, dspark_verify_rnn) against
the float64 oracle.

Bar: the stored states s_1..s_gamma equal the oracle's bit for bit on every
request whose drafted prefix matches (the gates are fp64 on both sides and the
state is stored in the weights' type, so rounding never lands differently in
practice); tokens, verify and accept lengths bit-exact on unflagged requests;
probabilities and statistics within atol 1e-4 / rtol 1e-5.
"""

import numpy as np
import pytest

import oracle as O
from gen import make_inputs, config
from gen.rnn import make_rnn_weights

from gpu_util import compare_rounds, gpu_round, say

pytestmark = pytest.mark.gpu


def _with_rnn(inp, seed):
    w = make_rnn_weights(inp["W1"].shape[1], inp["w_dtype"], seed=seed)
    inp.update(Wx=w["Wx"], Ws=w["Ws"], rnn_bias=w["bias"])
    return inp


def _check_states(orc, gpu, rows=None):
    sel = slice(None) if rows is None else np.asarray(rows)
    g_states = gpu["states"][sel].astype(np.float64)
    o_states = orc["draft"]["states"]
    same_tok = (gpu["draft_tokens"][sel] == orc["draft"]["tokens"])
    n = 0
    for i in range(len(o_states)):
        # s_k depends on x_0..x_{k-1}: compare up to the first differing token
        k_end = len(same_tok[i]) if same_tok[i].all() else int(np.argmin(same_tok[i])) + 1
        assert np.array_equal(g_states[i, :k_end], o_states[i, :k_end]), f"row {i} states"
        n += k_end
    say(f"  states compared: {n} (request, position) rows, bit-exact")


def _run(inp, T, label, rows=None, oracle_inp=None):
    say(f"[{label}] RNN round R={inp['base'].shape[0]} gamma={inp['base'].shape[1]} "
        f"V={inp['base'].shape[2]} r={inp['W1'].shape[1]} {inp['w_dtype']} T={T}")
    gpu = gpu_round(inp, T, head="rnn")
    assert gpu["device_error"] == 0, f"device error bits {gpu['device_error']}"
    orc = O.run_round(oracle_inp if oracle_inp is not None else inp, T=T, head="rnn")
    nflag = compare_rounds(orc, gpu, rows=rows, label=label)
    _check_states(orc, gpu, rows)
    return gpu, orc, nflag


@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1.0, 0.7, 0.0])
def test_rnn_tiny(w_dtype, T):
    d = config(1, w_dtype=w_dtype)
    _run(_with_rnn(make_inputs(d, seed=2), 5), T, f"tiny {w_dtype}")


@pytest.mark.parametrize("R,g,V,r,w_dtype", [
    (1, 1, 8, 16, "bf16"),
    (5, 3, 1000, 16, "bf16"),
    (33, 2, 520, 48, "f32"),
    (130, 3, 776, 32, "bf16"),
    (3, 16, 2048, 256, "bf16"),
    (4, 6, 1032, 256, "f32"),
])
def test_rnn_shapes(R, g, V, r, w_dtype):
    d = config(1, R=R, gamma=g, V=V, r=r, w_dtype=w_dtype, table="linear")
    _run(_with_rnn(make_inputs(d, seed=9), 6), 1.0, f"shape {R},{g},{V},{r},{w_dtype}")


def test_rnn_bias_differs_from_the_markov_head():
    """Same inputs, the two heads: the drafts differ (the state carries more
    than the previous token), so the RNN path is not the Markov path."""
    d = config(1, R=24, gamma=6, V=2048, r=64, w_dtype="bf16")
    inp = _with_rnn(make_inputs(d, seed=4), 7)
    a = gpu_round(inp, 1.0, head="rnn")
    b = gpu_round(inp, 1.0, head="markov")
    assert not np.array_equal(a["draft_stats"], b["draft_stats"])


def _near_tie_biases(n, seed=0):
    """fp32 values b whose float64 tanh lies just above a bf16 tie whose lower
    neighbour is even: one rounding to bf16 goes up, an fp32 rounding first
    would land on the tie and go down.  The distance above the tie is at least
    2^-12 fp32 units in the last place, far above any fp64 tanh error."""
    rng = np.random.default_rng(seed)
    out = []
    lo = np.float32(0.3).view(np.uint32)
    while len(out) < n:
        start = int(lo) + int(rng.integers(0, 1 << 22))
        b = np.arange(start, start + (1 << 20), dtype=np.uint32).view(np.float32)
        t = np.tanh(b.astype(np.float64))
        m, e = np.frexp(t)
        k = np.floor(m * 256.0)                     # bf16 lower neighbour, in units of 2^(e-8)
        frac = m * 256.0 - k - 0.5                  # distance above the tie, bf16 units
        ok = (frac > 2.0**-28) & (frac < 2.0**-18) & (k % 2 == 0)
        out.extend(b[ok][: n - len(out)].tolist())
    b = np.array(out, np.float32)
    t = np.tanh(b.astype(np.float64))
    assert (O.to_storage(t, "bf16") != O.to_storage(t.astype(np.float32), "bf16")).all()
    return b


def test_rnn_state_is_rounded_once_to_bf16():
    """Open update gate (u = 1) and zero weights: s_1 = tanh(b_candidate), so
    the stored state shows the kernel's rounding of a planted near-tie."""
    from gen.inputs import bf16_bits_from_f32
    r, V, R, g = 16, 512, 4, 2
    inp = make_inputs(config(1, w_dtype="bf16", r=r, R=R, gamma=g), seed=3)
    b = np.zeros((3, r), np.float32)
    b[0] = 60.0                                     # sigmoid(60) == 1 in float64
    sign = np.where(np.arange(r) % 2 == 0, 1.0, -1.0).astype(np.float32)
    b[2] = _near_tie_biases(r) * sign
    z = bf16_bits_from_f32(np.zeros((3, r, r), np.float32))
    inp.update(Wx=z, Ws=z, rnn_bias=b)
    gpu = gpu_round(inp, 1.0, head="rnn")
    assert gpu["device_error"] == 0
    want = O.to_storage(np.tanh(b[2].astype(np.float64)), "bf16")
    got = gpu["states"][:, 0, :].astype(np.float64)
    assert np.array_equal(got, np.broadcast_to(want, got.shape)), "state not rounded once from fp64"
    say(f"  {R * r} planted near-tie states rounded once")
