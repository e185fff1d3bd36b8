"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks a worked
example, a closed form, an invariant, a special case that reduces to a library
routine, or exact enumeration by bisection over the uniforms.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _softmax(x):
    return special.softmax(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------------------
# worked trace of the decode cycle


def _trace_inputs(T):
    g = json.load(open(os.path.join(GOLD, "worked_trace.json")))
    V, t, peak = g["V"], g["tokens"], g["peak"]
    base = np.zeros((1, 4, V), np.float32)
    for k, name in enumerate("EFGH"):
        base[0, k, t[name]] = peak
    target = np.zeros((1, 5, V), np.float32)
    target[0, 0], target[0, 1] = base[0, 0], base[0, 1]
    target[0, 2, t["K"]] = peak
    target[0, 3, t["H"]] = peak
    target[0, 4, 0] = peak
    W1 = np.zeros((V, 2), np.float32)
    W2 = np.zeros((2, V), np.float32)
    inp = dict(base=base, target=target, W1=W1, W2=W2, w_dtype="f32",
               anchor=np.array([t["D"]], np.int32), rows=np.array([0]),
               u_draft=np.full((1, 4), g["u"], np.float32),
               u_accept=np.full((1, 4), g["u"], np.float32),
               u_final=np.full(1, g["u"], np.float32),
               conf=np.array([g["conf"]], np.float32),
               sps=np.array(g["sps_B_1_to_5"], np.float32))
    return g, inp


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_worked_trace(T):
    g, inp = _trace_inputs(T)
    e = g["expected"]
    res = O.run_round(inp, T=T)
    assert res["draft"]["tokens"][0].tolist() == e["draft_tokens"]
    s = res["schedule"]
    np.testing.assert_allclose(s["cum_conf"][0], e["cum_conf"], rtol=1e-6)
    np.testing.assert_allclose(s["theta"] / 2.0 ** 36, e["theta_scaled"], rtol=1e-6)
    assert s["n_admitted"] == e["n_admitted"]
    assert res["verify_len"][0] == e["verify_len"]
    assert res["verify"]["accept_len"][0] == e["accept_len"]
    assert res["verify"]["out_tokens"][0].tolist() == e["out_tokens"]
    assert not res["flags"][0]


# ---------------------------------------------------------------------------
# draft: softmax normalisation, exact bias, Markov direction, special cases


def _rand_case(rng, R=3, g=3, V=24, r=4, wsig=0.5):
    base = (rng.standard_normal((R, g, V)) * 2).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * wsig).astype(np.float32)
    W2 = (rng.standard_normal((r, V)) * wsig).astype(np.float32)
    anchor = rng.integers(0, V, R).astype(np.int32)
    return base, W1, W2, anchor


def test_softmax_normalisation_and_logsumexp():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 300)) * 4
    for T in (1.0, 0.7, 2.5):
        pi, m, Z = O.draft_distribution(z, T)
        np.testing.assert_allclose(pi.sum(axis=1), 1.0, atol=1e-13)
        np.testing.assert_allclose(np.log(Z) + m / T, special.logsumexp(z / T, axis=1), rtol=1e-13)
        np.testing.assert_allclose(pi, special.softmax(z / T, axis=1), atol=1e-15)


def test_bias_is_exact_sum_of_bf16_products():
    from gen.inputs import bf16_bits_from_f32
    rng = np.random.default_rng(2)
    V, r = 40, 16
    w1 = bf16_bits_from_f32(rng.standard_normal((V, r)).astype(np.float32) * 0.05)
    w2 = bf16_bits_from_f32(rng.standard_normal((r, V)).astype(np.float32) * 0.05)
    W1 = O.widen_weights(w1, "bf16")
    W2 = O.widen_weights(w2, "bf16")
    prev = [3, 17, 39]
    bias = O.markov_bias(W1, W2, prev)

    def exact(bits):   # bf16 pattern -> exact rational
        sign = -1 if bits >> 15 else 1
        ex = (bits >> 7) & 0xFF
        man = bits & 0x7F
        return sign * Fraction(128 + man, 128) * Fraction(2) ** (ex - 127)

    for i, pv in enumerate(prev):
        for v in (0, 7, 21, 39):
            s = sum(exact(int(w1[pv, k])) * exact(int(w2[k, v])) for k in range(r))
            assert abs(float(s) - bias[i, v]) <= 1e-15 * max(1.0, abs(float(s)))


def test_markov_direction_of_course():
    # vocabulary: 0 "of", 1 "course", 2 "problem", 3 "no", 4.. filler
    V, r = 8, 2
    W1 = np.zeros((V, r), np.float32)
    W2 = np.zeros((r, V), np.float32)
    W1[0, 0] = 1.0            # previous token "of" -> latent 0
    W2[0, 1], W2[0, 2] = 3.0, -3.0   # latent 0 raises "course", lowers "problem"
    base = np.zeros((1, 1, V), np.float32)
    base[0, 0, [1, 2]] = 2.0   # parallel stage is bimodal between the two
    res = O.draft(base, W1, W2, "f32", np.array([0], np.int32), np.array([[0.5]], np.float32), 1.0)
    z = base[0, 0].astype(np.float64).copy()
    z[1] += 3.0
    z[2] -= 3.0
    # index direction: row of W1 = previous token, column of W2 = next token
    assert res["tokens"][0, 0] == 1
    np.testing.assert_allclose(res["probs"][0, 0], _softmax(z)[1], rtol=1e-14)
    # after any other previous token the bias vanishes
    res2 = O.draft(base, W1, W2, "f32", np.array([5], np.int32), np.array([[0.5]], np.float32), 1.0)
    np.testing.assert_allclose(res2["probs"][0, 0], _softmax(base[0, 0])[res2["tokens"][0, 0]],
                               rtol=1e-14)
    # transposing the factors (a plausible bug) would bias the wrong pair
    assert O.markov_bias(W1.astype(np.float64), W2.astype(np.float64), [0])[0, 1] == 3.0
    assert O.markov_bias(W1.astype(np.float64), W2.astype(np.float64), [1])[0, 0] == 0.0


def test_zero_factors_give_independent_parallel_drafter():
    rng = np.random.default_rng(3)
    base, W1, W2, anchor = _rand_case(rng, R=4, g=5, V=30)
    W1[:] = 0
    W2[:] = 0
    u = rng.random((4, 5)).astype(np.float32)
    res = O.draft(base, W1, W2, "f32", anchor, u, 1.0)
    for i in range(4):
        for k in range(5):
            p = _softmax(base[i, k])
            x = int(np.searchsorted(np.cumsum(p), u[i, k], side="right"))
            assert res["tokens"][i, k] == x
            np.testing.assert_allclose(res["probs"][i, k], p[x], rtol=1e-13)
            np.testing.assert_allclose(res["stats"][i, k, 0], base[i, k].max())


def test_rank_one_bias_is_outer_product():
    rng = np.random.default_rng(4)
    base, W1, W2, anchor = _rand_case(rng, R=2, g=3, V=20, r=1)
    u = rng.random((2, 3)).astype(np.float32)
    res = O.draft(base, W1, W2, "f32", anchor, u, 1.0)
    prev = anchor.copy()
    for k in range(3):
        for i in range(2):
            z = base[i, k].astype(np.float64) + float(W1[prev[i], 0]) * W2[0].astype(np.float64)
            p = _softmax(z)
            np.testing.assert_allclose(res["probs"][i, k], p[res["tokens"][i, k]], rtol=1e-13)
            np.testing.assert_allclose(res["stats"][i, k, 1], np.exp(z - z.max()).sum(), rtol=1e-13)
        prev = res["tokens"][:, k]


def test_greedy_draft_is_argmax():
    rng = np.random.default_rng(5)
    base, W1, W2, anchor = _rand_case(rng)
    res = O.draft(base, W1, W2, "f32", anchor, np.zeros((3, 3), np.float32), 0.0)
    prev = anchor
    for k in range(3):
        z = base[:, k].astype(np.float64) + W1[prev].astype(np.float64) @ W2.astype(np.float64)
        assert (res["tokens"][:, k] == z.argmax(axis=1)).all()
        prev = res["tokens"][:, k]
    assert (res["probs"] == 1).all()


# ---------------------------------------------------------------------------
# exact enumeration by bisection over the uniforms


def _bisect_first(pred, iters=64):
    """Smallest u in [0, 1) (to ~2^-64) where the monotone predicate turns True."""
    lo, hi = 0.0, 1.0
    if pred(lo):
        return 0.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            hi = mid
        else:
            lo = mid
    return hi


def _interval_masses(f, n):
    """Measures of {u : f(u) = v} for a monotone non-decreasing f: [0,1) -> {0..n-1}."""
    edges = [0.0] + [_bisect_first(lambda u, v=v: f(u) >= v) for v in range(1, n)] + [1.0]
    return np.diff(edges), edges


class _Tiny:
    """A V = 4, gamma = 2 single-request round with x1-dependent target rows."""

    def __init__(self, seed, T=1.0):
        rng = np.random.default_rng(seed)
        self.V, self.T = 4, T
        self.base = (rng.standard_normal((1, 2, 4)) * 1.5).astype(np.float32)
        self.W1 = (rng.standard_normal((4, 2)) * 0.8).astype(np.float32)
        self.W2 = (rng.standard_normal((2, 4)) * 0.8).astype(np.float32)
        self.anchor = np.array([1], np.int32)
        self.T1 = (rng.standard_normal(4) * 1.5).astype(np.float32)          # target row 0
        self.T2 = (rng.standard_normal((4, 4)) * 1.5).astype(np.float32)     # row 1 given x1
        self.T3 = (rng.standard_normal(4) * 1.5).astype(np.float32)          # bonus row 2

    def draft(self, u1, u2):
        r = O.draft(self.base, self.W1, self.W2, "f32", self.anchor,
                    np.array([[u1, u2]]), self.T)
        return r["tokens"][0], r["probs"][0]

    def verify(self, x, q, L, ua1, ua2, uf):
        tgt = np.stack([self.T1, self.T2[x[0]], self.T3])[None]
        return O.verify(tgt, self.base, self.W1, self.W2, "f32", self.anchor, x[None], q[None],
                        np.array([L]), np.array([[ua1, ua2]]), np.array([uf]), self.T)

    def mid_u1(self, a):
        m, e = _interval_masses(lambda u: self.draft(u, 0.5)[0][0], 4)
        return 0.5 * (e[a] + e[a + 1]), m

    def first_token_law(self, L_of_x1):
        """Exact law of the first emitted token; L may depend on x1 (a control)."""
        P = np.zeros(4)
        _, m1 = self.mid_u1(0)
        for a in range(4):
            if m1[a] == 0:
                continue
            u1, _ = self.mid_u1(a)
            x, q = self.draft(u1, 0.5)
            L = L_of_x1(a)
            if L == 0:
                law, _ = _interval_masses(lambda uf: self.verify(x, q, 0, .5, .5, uf)["out_tokens"][0, 0], 4)
                P += m1[a] * law
                continue
            p_acc = _bisect_first(lambda ua: self.verify(x, q, L, ua, 0.0, 0.5)["accept_len"][0] == 0)
            P[a] += m1[a] * p_acc
            if p_acc < 1:
                law, _ = _interval_masses(
                    lambda uf: self.verify(x, q, L, 1 - 1e-17, 0.0, uf)["out_tokens"][0, 0], 4)
                P += m1[a] * (1 - p_acc) * law
        return P

    def second_token_law(self, a, L):
        """Exact law of the second emitted token given x1 = a was accepted."""
        u1, _ = self.mid_u1(a)
        P = np.zeros(4)
        if L == 1:
            x, q = self.draft(u1, 0.5)
            law, _ = _interval_masses(lambda uf: self.verify(x, q, 1, 0.0, .5, uf)["out_tokens"][0, 1], 4)
            return law
        m2, _ = _interval_masses(lambda u: self.draft(u1, u)[0][1], 4)
        e2 = np.concatenate([[0.0], np.cumsum(m2)])
        for b in range(4):
            if m2[b] == 0:
                continue
            x, q = self.draft(u1, 0.5 * (e2[b] + e2[b + 1]))
            assert x[0] == a and x[1] == b
            p_acc = _bisect_first(lambda ua: self.verify(x, q, 2, 0.0, ua, 0.5)["accept_len"][0] == 1)
            P[b] += m2[b] * p_acc
            if p_acc < 1:
                law, _ = _interval_masses(
                    lambda uf: self.verify(x, q, 2, 0.0, 1 - 1e-17, uf)["out_tokens"][0, 1], 4)
                P += m2[b] * (1 - p_acc) * law
        return P


@pytest.mark.parametrize("seed", [11, 12])
@pytest.mark.parametrize("L", [0, 1, 2])
def test_lossless_first_token_exact(seed, L):
    t = _Tiny(seed)
    P = t.first_token_law(lambda a: L)
    np.testing.assert_allclose(P, _softmax(t.T1), atol=1e-12)


@pytest.mark.parametrize("seed", [11, 13])
@pytest.mark.parametrize("L", [1, 2])
def test_lossless_second_token_exact(seed, L):
    t = _Tiny(seed)
    for a in range(4):
        np.testing.assert_allclose(t.second_token_law(a, L), _softmax(t.T2[a]), atol=1e-12)


def test_lossless_with_scheduler_lengths():
    t = _Tiny(14)
    sched = O.schedule(np.array([[0.9, 0.6]], np.float32),
                       np.array([1.0, 0.8, 0.5], np.float32))
    L = int(sched["verify_len"][0])
    P = t.first_token_law(lambda a: L)
    np.testing.assert_allclose(P, _softmax(t.T1), atol=1e-12)


def test_negative_control_anticipating_scheduler_is_biased():
    """Verify length chosen from the drafted token breaks losslessness."""
    t = _Tiny(11)
    _, m1 = t.mid_u1(0)
    fav = int(np.argmax(m1))
    P = t.first_token_law(lambda a: 1 if a == fav else 0)
    assert np.abs(P - _softmax(t.T1)).max() > 1e-3


def test_accept_probability_closed_form():
    """P(accept at position 1) = sum min(p, q) = 1 - TV(p, q)."""
    t = _Tiny(15)
    p = _softmax(t.T1)
    q = _softmax(t.base[0, 0].astype(np.float64) + t.W1[1].astype(np.float64) @ t.W2.astype(np.float64))
    _, m1 = t.mid_u1(0)
    P = 0.0
    for a in range(4):
        if m1[a] == 0:
            continue
        u1, _ = t.mid_u1(a)
        x, qq = t.draft(u1, 0.5)
        P += m1[a] * _bisect_first(lambda ua: t.verify(x, qq, 1, ua, 0.0, 0.5)["accept_len"][0] == 0)
    np.testing.assert_allclose(P, np.minimum(p, q).sum(), atol=1e-12)
    np.testing.assert_allclose(P, 1 - 0.5 * np.abs(p - q).sum(), atol=1e-12)


def test_residual_mass_is_half_l1_distance():
    rng = np.random.default_rng(16)
    R, g, V = 6, 3, 50
    base, W1, W2, anchor = _rand_case(rng, R=R, g=g, V=V)
    target = (rng.standard_normal((R, g + 1, V)) * 2).astype(np.float32)
    u = rng.random((R, g)).astype(np.float32)
    d = O.draft(base, W1, W2, "f32", anchor, u, 1.0)
    v = O.verify(target, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], None,
                 np.full((R, g), 0.999999, np.float32), rng.random(R).astype(np.float32), 1.0)
    for i in range(R):
        A = v["accept_len"][i]
        if A == g:
            continue
        prev = anchor[i] if A == 0 else d["tokens"][i, A - 1]
        pi = _softmax(base[i, A].astype(np.float64) + W1[prev].astype(np.float64) @ W2.astype(np.float64))
        p = _softmax(target[i, A])
        np.testing.assert_allclose(v["residual_mass"][i], 0.5 * np.abs(p - pi).sum(), rtol=1e-12)


def test_chi_square_first_emitted_token():
    rng = np.random.default_rng(17)
    R, g, V = 100000, 2, 16
    base1 = (rng.standard_normal((g, V)) * 1.5).astype(np.float32)
    W1 = (rng.standard_normal((V, 2)) * 0.5).astype(np.float32)
    W2 = (rng.standard_normal((2, V)) * 0.5).astype(np.float32)
    tgt1 = (base1[0] + rng.standard_normal(V) * 0.8).astype(np.float32)
    base = np.broadcast_to(base1, (R, g, V))
    target = np.broadcast_to(np.stack([tgt1, base1[1], base1[0]]), (R, g + 1, V))
    anchor = np.full(R, 3, np.int32)
    ur = np.random.default_rng(18)
    d = O.draft(base, W1, W2, "f32", anchor, ur.random((R, g), np.float32), 1.0)
    v = O.verify(target, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], np.ones(R, np.int64),
                 ur.random((R, g), np.float32), ur.random(R, np.float32), 1.0)
    y = v["out_tokens"][:, 0]
    exp = _softmax(tgt1) * R
    obs = np.bincount(y, minlength=V).astype(np.float64)
    keep = exp >= 5
    o = np.concatenate([obs[keep], [obs[~keep].sum()]]) if (~keep).any() else obs
    e = np.concatenate([exp[keep], [exp[~keep].sum()]]) if (~keep).any() else exp
    assert stats.chisquare(o, e).pvalue >= 1e-3


def test_equal_draft_and_target_always_accepts():
    rng = np.random.default_rng(19)
    R, g, V = 5, 4, 40
    base, W1, W2, anchor = _rand_case(rng, R=R, g=g, V=V)
    W1[:] = 0
    target = np.concatenate([base, base[:, :1]], axis=1)
    u = rng.random((R, g)).astype(np.float32)
    d = O.draft(base, W1, W2, "f32", anchor, u, 1.0)
    L = np.array([0, 1, 2, 3, 4])
    v = O.verify(target, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], L,
                 np.full((R, g), 0.99999994, np.float32), u[:, 0], 1.0)
    assert (v["accept_len"] == L).all()


def test_greedy_verify():
    rng = np.random.default_rng(20)
    R, g, V = 6, 3, 30
    base, W1, W2, anchor = _rand_case(rng, R=R, g=g, V=V)
    target = (rng.standard_normal((R, g + 1, V))).astype(np.float32)
    d = O.draft(base, W1, W2, "f32", anchor, np.zeros((R, g)), 0.0)
    # make row 0 accept everything, row 1 reject at 2
    for k in range(g):
        target[0, k, d["tokens"][0, k]] = 50
    target[1, 0, d["tokens"][1, 0]] = 50
    target[1, 1, d["tokens"][1, 1]] = -50
    v = O.verify(target, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], None,
                 np.zeros((R, g)), np.zeros(R), 0.0)
    assert v["accept_len"][0] == g
    assert v["out_tokens"][0, g] == int(np.argmax(target[0, g]))
    assert v["accept_len"][1] == 1
    assert v["out_tokens"][1, 1] == int(np.argmax(target[1, 1]))
    for i in range(R):
        A = v["accept_len"][i]
        assert (v["out_tokens"][i, :A] == d["tokens"][i, :A]).all()
        assert v["out_tokens"][i, A] == int(np.argmax(target[i, A]))


def test_boundary_uniform_is_flagged():
    rng = np.random.default_rng(21)
    base, W1, W2, anchor = _rand_case(rng, R=1, g=1, V=10)
    z = base[0, 0].astype(np.float64) + W1[anchor[0]].astype(np.float64) @ W2.astype(np.float64)
    F = np.cumsum(_softmax(z))
    for u, flagged in ((F[3] - 3e-7, True), (F[3] + 3e-7, True), (0.5 * (F[3] + F[4]), False)):
        d = O.draft(base, W1, W2, "f32", anchor, np.array([[u]]), 1.0)
        assert (d["margin"][0, 0] < O.FLAG_EPS) == flagged


# ---------------------------------------------------------------------------
# boundary flags: every clause of row_flags, planted against boundaries
# computed here from scipy's softmax (zero Markov factors, so the draft
# distribution at position k is softmax(base row k-1) and the target
# distribution softmax(target row k-1))


class _FlagCase:
    """One request, gamma = 3, V = 12, zero factors; drafted tokens chosen by
    putting u_draft in the middle of the chosen token's CDF interval."""

    V, G = 12, 3

    def __init__(self, seed=31, xs=(3, 2, 3)):
        rng = np.random.default_rng(seed)
        V, g = self.V, self.G
        self.base = (rng.standard_normal((1, g, V)) * 0.6).astype(np.float32)
        self.target = (rng.standard_normal((1, g + 1, V)) * 0.6).astype(np.float32)
        self.W1 = np.zeros((V, 2), np.float32)
        self.W2 = np.zeros((2, V), np.float32)
        self.anchor = np.array([0], np.int32)
        self.q = [_softmax(self.base[0, k]) for k in range(g)]          # draft distributions
        self.p = [_softmax(self.target[0, k]) for k in range(g + 1)]    # target distributions
        self.x = list(xs)
        u = []
        for k, xk in enumerate(xs):
            F = np.cumsum(self.q[k])
            lo = F[xk - 1] if xk > 0 else 0.0
            u.append(0.5 * (lo + F[xk]))
            assert F[xk] - lo > 1e-2           # the draft events sit far from every edge
        self.u_draft = np.array([u], np.float64)
        self.rho = [self.p[k][xs[k]] / self.q[k][xs[k]] for k in range(g)]

    def run(self, L, u_accept, u_final, T=1.0, u_draft=None):
        inp = dict(base=self.base, target=self.target, W1=self.W1, W2=self.W2, w_dtype="f32",
                   anchor=self.anchor, u_draft=self.u_draft if u_draft is None else u_draft,
                   u_accept=np.array([u_accept], np.float64), u_final=np.array([u_final], np.float64))
        d = O.draft(inp["base"], self.W1, self.W2, "f32", self.anchor, inp["u_draft"], T)
        v = O.verify(self.target, self.base, self.W1, self.W2, "f32", self.anchor, d["tokens"], d["probs"],
                     np.array([L]), inp["u_accept"], inp["u_final"], T)
        return d, v, bool(O.row_flags(d, v)[0])

    def residual_cdf(self, k):
        d = np.maximum(0.0, self.p[k - 1] - self.q[k - 1])
        return np.cumsum(d) / d.sum(), d / d.sum()

    @staticmethod
    def mid_of_largest(w):
        """Midpoint of the widest CDF interval of the weights w (far from every edge)."""
        F = np.cumsum(w) / np.sum(w)
        j = int(np.argmax(w))
        return 0.5 * ((F[j - 1] if j > 0 else 0.0) + F[j])


def _flag_case_with_rho_below_one():
    c = _FlagCase()
    assert 0.1 < c.rho[0] < 0.9 and 0.05 < c.rho[1]       # a real accept test at position 1
    return c


@pytest.mark.parametrize("delta,flagged", [(-3e-7, True), (3e-7, True), (-3e-6, False), (3e-6, False)])
def test_accept_test_near_p_over_q_flags(delta, flagged):
    """Accept events: |u - p/q| < 1e-6 flags the request, 3e-6 away does not."""
    c = _flag_case_with_rho_below_one()
    u = c.rho[0] + delta
    accepted = delta < 0
    # the final uniform sits mid-interval of whichever law it samples: the bonus
    # row 1 after an accept (L = 1), the residual at position 1 after a reject
    uf = c.mid_of_largest(c.p[1]) if accepted else c.mid_of_largest(c.residual_cdf(1)[1])
    d, v, fl = c.run(1, [u, 0.5, 0.5], uf)
    assert v["accept_len"][0] == (1 if accepted else 0)
    assert (d["margin"][0] > 1e-3).all() and v["final_margin"][0] > 1e-3
    assert fl == flagged


def test_accept_tests_after_the_rejection_never_flag():
    """Only the accept tests up to the first rejection are events: positions
    after k*, and positions past the verify length, do not flag even with u
    planted on p/q."""
    c = _flag_case_with_rho_below_one()
    u1 = min(0.999, c.rho[0] + 0.05)                      # reject at k* = 1
    uf = c.mid_of_largest(c.residual_cdf(1)[1])
    ua = [u1, min(c.rho[1], 0.999) - 1e-9, min(c.rho[2], 0.999) + 1e-9]
    d, v, fl = c.run(3, ua, uf)
    assert v["accept_len"][0] == 0 and not fl
    # accepted at position 1 with L = 1: position 2 is not verified
    d, v, fl = c.run(1, [0.0, min(c.rho[1], 0.999) - 1e-9, 0.5], c.mid_of_largest(c.p[1]))
    assert v["accept_len"][0] == 1 and not fl


@pytest.mark.parametrize("delta,flagged", [(-3e-7, True), (3e-7, True), (-3e-6, False), (3e-6, False)])
def test_final_sample_near_a_residual_edge_flags(delta, flagged):
    c = _flag_case_with_rho_below_one()
    F, w = c.residual_cdf(1)
    # an inner edge between two tokens that both carry residual mass
    j = next(i for i in range(c.V - 1) if w[i] > 0.02 and w[i + 1] > 0.02)
    d, v, fl = c.run(1, [0.999, 0.5, 0.5], F[j] + delta)
    assert v["accept_len"][0] == 0
    assert v["out_tokens"][0, 0] == (j if delta < 0 else j + 1)
    assert (d["margin"][0] > 1e-3).all() and abs(0.999 - c.rho[0]) > 1e-3
    assert fl == flagged


@pytest.mark.parametrize("L", [0, 1])
@pytest.mark.parametrize("delta,flagged", [(-3e-7, True), (3e-7, True), (-3e-6, False), (3e-6, False)])
def test_final_sample_near_a_bonus_edge_flags(L, delta, flagged):
    """The bonus sample from target row L (L = 0: a plain target step)."""
    c = _flag_case_with_rho_below_one()
    F = np.cumsum(c.p[L])
    j = 4
    d, v, fl = c.run(L, [0.0, 0.5, 0.5], F[j] + delta)
    assert v["accept_len"][0] == L
    assert v["out_tokens"][0, L] == (j if delta < 0 else j + 1)
    assert fl == flagged


def test_every_draft_event_flags_even_after_the_rejection():
    """Draft events count at all gamma positions, verified or not."""
    c = _flag_case_with_rho_below_one()
    F = np.cumsum(c.q[2])
    u_draft = c.u_draft.copy()
    u_draft[0, 2] = F[c.x[2]] - 3e-7                       # position 3, near its upper edge
    uf = c.mid_of_largest(c.residual_cdf(1)[1])
    d, v, fl = c.run(1, [0.999, 0.5, 0.5], uf, u_draft=u_draft)
    assert v["accept_len"][0] == 0 and d["tokens"][0, 2] == c.x[2]
    assert fl
    u_draft[0, 2] = F[c.x[2]] - 3e-6
    assert not c.run(1, [0.999, 0.5, 0.5], uf, u_draft=u_draft)[2]


def _greedy_case(gap_accept, gap_final, top=0.5):
    """Greedy round, one request, gamma = 2, V = 8, zero factors.  Draft argmaxes
    are tokens 3 and 6 (wide gaps); target row 0 has its maximum at token 3 and
    a runner-up gap_accept below it; target row 1 (the bonus row at L = 1) has
    its two largest values gap_final apart."""
    V = 8
    base = np.zeros((1, 2, V), np.float32)
    base[0, 0, 3] = base[0, 1, 6] = 5.0
    target = np.full((1, 3, V), top - 10.0, np.float32)
    target[0, 0, 3] = top
    target[0, 0, 1] = np.float32(top - gap_accept)
    target[0, 1, 2] = top
    target[0, 1, 5] = np.float32(top - gap_final)
    W1 = np.zeros((V, 2), np.float32)
    W2 = np.zeros((2, V), np.float32)
    anchor = np.array([0], np.int32)
    d = O.draft(base, W1, W2, "f32", anchor, np.zeros((1, 2)), 0.0)
    v = O.verify(target, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], np.array([1]),
                 np.zeros((1, 2)), np.zeros(1), 0.0)
    return d, v, bool(O.row_flags(d, v)[0]), target


@pytest.mark.parametrize("top", [0.5, -3.0])
def test_greedy_top2_gap_flags(top):
    """Greedy events flag when the top-2 gap is below 1e-6 * max(1, |top1|):
    in the verified target row (the accept test) and in the bonus row."""
    scale = max(1.0, abs(top))
    for ga, gf, want in ((5e-7 * scale, 1e-3, True), (1e-3, 5e-7 * scale, True),
                         (5e-6 * scale, 1e-3, False), (1e-3, 5e-6 * scale, False)):
        d, v, fl, target = _greedy_case(ga, gf, top)
        # the stored fp32 gaps are what the rule sees
        real_a = float(target[0, 0, 3]) - float(target[0, 0, 1])
        real_f = float(target[0, 1, 2]) - float(target[0, 1, 5])
        assert (real_a < 1e-6 * scale or real_f < 1e-6 * scale) == want
        assert d["tokens"][0].tolist() == [3, 6] and v["accept_len"][0] == 1
        assert v["out_tokens"][0].tolist() == [3, 2, -1]
        assert fl == want


# ---------------------------------------------------------------------------
# scheduler


def _sched_case(seed, R=8, g=5, ties=False):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
    if ties:
        c[rng.random((R, g)) < 0.3] = 1.0
    return c


@pytest.mark.parametrize("ties", [False, True])
def test_schedule_invariants(ties):
    c = _sched_case(30, R=16, g=6, ties=ties)
    sps = (1.0 / (1.0 + 0.02 * np.arange(1, 200))).astype(np.float32)
    s = O.schedule(c, sps)
    a = s["cum_conf"]
    assert (a[:, 1:] <= a[:, :-1]).all()                       # survival is non-increasing
    L, n = s["verify_len"], s["n_admitted"]
    assert L.sum() == n
    admitted = set(int(f) for f in s["order"][:n])
    for r in range(16):
        assert admitted & set(range(r * 6, r * 6 + 6)) == set(range(r * 6, r * 6 + L[r]))
    assert 0 <= n <= 16 * 6


def test_constant_table_admits_everything():
    c = _sched_case(31)
    s = O.schedule(c, np.ones(100, np.float32))
    assert s["n_admitted"] == c.size and (s["verify_len"] == c.shape[1]).all()


def test_table_end_is_a_wall():
    c = np.ones((4, 5), np.float32)
    s = O.schedule(c, np.ones(10, np.float32))       # B = 4 + n must stay <= 10
    assert s["n_admitted"] == 6


def test_early_stop_is_global_optimum_on_unimodal_objective():
    import itertools
    for seed in range(40, 60):
        rng = np.random.default_rng(seed)
        R, g = 3, 3
        c = rng.uniform(0.2, 1.0, (R, g)).astype(np.float32)
        slope = rng.uniform(0.05, 0.6)
        sps = (1.0 / (1.0 + slope * np.arange(1, 30))).astype(np.float32)
        s = O.schedule(c, sps)
        th = s["theta"]
        k = int(np.argmax(th))
        if not ((np.diff(th[: k + 1]) >= 0).all() and (np.diff(th[k:]) <= 0).all()):
            continue                               # precondition: unimodal along the pool order
        a = s["cum_conf"].astype(np.float64)
        best, bestL = -1.0, None
        for Lv in itertools.product(range(g + 1), repeat=R):
            tau = R + sum(a[r, :Lv[r]].sum() for r in range(R))
            val = tau * float(sps[R + sum(Lv) - 1])
            if val > best:
                best, bestL = val, Lv
        assert tuple(s["verify_len"]) == bestL


def test_stair_table_cut_lands_on_a_stair_edge():
    from gen.inputs import cost_table
    rng = np.random.default_rng(32)
    R, g = 128, 7
    c = rng.beta(8, 2, (R, g)).astype(np.float32)
    s = O.schedule(c, cost_table("stairs64", R, g))
    n = s["n_admitted"]
    assert 0 < n < R * g
    assert (R + n) % 64 == 0


def test_verify_length_ignores_drafted_tokens():
    """Non-anticipation: L depends on confidences only, never on tokens or uniforms."""
    from gen import make_inputs
    a = make_inputs(1)
    b = make_inputs(1, seed_u=99)
    ra, rb = O.run_round(a), O.run_round(b)
    assert (ra["draft"]["tokens"] != rb["draft"]["tokens"]).any()
    assert (ra["verify_len"] == rb["verify_len"]).all()
    # relabelling the vocabulary leaves the schedule alone as well
    perm = np.random.default_rng(5).permutation(a["base"].shape[2])
    c = dict(a, base=a["base"][:, :, perm], target=a["target"][:, :, perm], W2=a["W2"][:, perm])
    assert (O.run_round(c)["verify_len"] == ra["verify_len"]).all()


# ---------------------------------------------------------------------------
# asynchronous production scheduler ([HADA] Implantação em produção)


def test_async_schedule_worked_example():
    g = json.load(open(os.path.join(GOLD, "async_schedule.json")))
    c = np.array([g["conf"]], np.float32)
    cl = np.array([g["conf_lag"]], np.float32)
    sps = np.array(g["sps_B_1_to_5"], np.float32)
    s = O.schedule_async(c, cl, sps)
    e = g["expected"]
    np.testing.assert_allclose(s["theta_lag"] / float(1 << 36), e["theta_lag_scaled"], rtol=1e-6)
    assert s["n_admitted"] == e["K"]
    assert int(s["verify_len"][0]) == e["verify_len"]
    assert int(O.schedule(c, sps)["verify_len"][0]) == e["early_stop_verify_len"]


def test_async_with_current_confidences_matches_early_stop_on_unimodal_objective():
    """Theta along the sorted pool is unimodal for SPS(B) = 1/(1 + beta B) (the
    increments a_{n+1}(1 + beta(R+n)) - beta T_n never increase), so the global
    maximiser equals the first drop when the lag is the current pool."""
    checked = 0
    for seed in range(70, 90):
        rng = np.random.default_rng(seed)
        R, g = int(rng.integers(2, 9)), int(rng.integers(1, 8))
        c = rng.uniform(0.2, 1.0, (R, g)).astype(np.float32)
        beta = rng.uniform(0.002, 0.3)
        sps = (1.0 / (1.0 + beta * np.arange(1, R * (g + 1) + 5))).astype(np.float32)
        s0, s1 = O.schedule(c, sps), O.schedule_async(c, c, sps)
        th = s0["theta"]
        if (np.diff(th) == 0).any():
            continue                                   # plateau: the two tie rules differ
        checked += 1
        assert s1["n_admitted"] == s0["n_admitted"]
        assert (s1["verify_len"] == s0["verify_len"]).all()
    assert checked >= 15


def test_async_cut_is_exact_argmax():
    """K against the maximiser of Theta recomputed in exact rationals."""
    from fractions import Fraction
    checked = differs = 0
    for seed in range(90, 130):
        rng = np.random.default_rng(seed)
        R, g = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        cl = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        c = rng.uniform(0.05, 1.0, (R, g)).astype(np.float32)
        sps = np.sort(rng.uniform(0.1, 1.0, R * g + 3))[::-1].astype(np.float32)
        sps[rng.integers(0, len(sps))] *= np.float32(1.5)   # a bump: objective not unimodal
        a = np.empty_like(cl)
        a[:, 0] = cl[:, 0]
        for j in range(1, g):
            a[:, j] = a[:, j - 1] * cl[:, j]
        vals = sorted((Fraction(float(v)) for v in a.reshape(-1)), reverse=True)
        thetas = []
        for n in range(R * g + 1):
            B = R + n
            S = Fraction(float(sps[B - 1])) if B <= len(sps) else Fraction(0)
            thetas.append((R + sum(vals[:n])) * S)
        best = max(thetas)
        K_exact = thetas.index(best)
        second = max((t for i, t in enumerate(thetas) if i != K_exact), default=Fraction(0))
        if best - second < best * Fraction(1, 10 ** 8):
            continue                                    # fixed-point rounding could decide
        assert O.schedule_async(c, cl, sps)["n_admitted"] == K_exact
        checked += 1
        differs += O.schedule(cl, sps)["n_admitted"] != K_exact   # early stop would cut elsewhere
    assert checked >= 30 and differs >= 3


def test_async_schedule_invariants():
    rng = np.random.default_rng(33)
    R, g = 16, 6
    c = _sched_case(34, R=R, g=g, ties=True)
    cl = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
    sps = (1.0 / (1.0 + 0.02 * np.arange(1, 200))).astype(np.float32)
    s = O.schedule_async(c, cl, sps)
    L, K = s["verify_len"], s["n_admitted"]
    assert L.sum() == K and 0 <= K <= R * g
    admitted = set(int(f) for f in s["order"][:K])
    for r in range(R):                                  # admitted sets are prefixes
        assert admitted & set(range(r * g, r * g + g)) == set(range(r * g, r * g + L[r]))
    # K comes from the lagged pool only: independent of the current confidences
    # and of which request each lagged row belongs to
    c2 = rng.uniform(0.3, 1.0, (R, g)).astype(np.float32)
    assert O.schedule_async(c2, cl, sps)["n_admitted"] == K
    assert O.schedule_async(c, cl[rng.permutation(R)], sps)["n_admitted"] == K


def test_lossless_with_async_scheduler_lengths():
    t = _Tiny(15)
    sched = O.schedule_async(np.array([[0.9, 0.6]], np.float32), np.array([[0.7, 0.9]], np.float32),
                             np.array([1.0, 0.8, 0.5], np.float32))
    L = int(sched["verify_len"][0])
    P = t.first_token_law(lambda a: L)
    np.testing.assert_allclose(P, _softmax(t.T1), atol=1e-12)


# ---------------------------------------------------------------------------
# per-position acceptance labels c*_k and the static-threshold baseline


def test_accept_rate_equals_enumerated_acceptance_probability():
    """c*_1 and c*_2 against the exact acceptance probabilities of the oracle's
    own rejection test, found by bisection over the uniforms."""
    t = _Tiny(17)
    _, m1 = t.mid_u1(0)
    P1 = 0.0
    for a in range(4):
        if m1[a] == 0:
            continue
        u1, _ = t.mid_u1(a)
        x, qq = t.draft(u1, 0.5)
        P1 += m1[a] * _bisect_first(lambda ua: t.verify(x, qq, 1, ua, 0.0, 0.5)["accept_len"][0] == 0)
        # position 2 given x1 = a accepted: average the test over x2 ~ q2(. | a)
        m2, _ = _interval_masses(lambda u: t.draft(u1, u)[0][1], 4)
        e2 = np.concatenate([[0.0], np.cumsum(m2)])
        P2 = 0.0
        for b in range(4):
            if m2[b] == 0:
                continue
            x2, q2 = t.draft(u1, 0.5 * (e2[b] + e2[b + 1]))
            P2 += m2[b] * _bisect_first(lambda ua: t.verify(x2, q2, 2, 0.0, ua, 0.5)["accept_len"][0] == 1)
        tgt = np.stack([t.T1, t.T2[a], t.T3])[None]
        c = O.accept_rates(tgt, t.base, t.W1, t.W2, "f32", t.anchor, x2[None], 1.0)
        np.testing.assert_allclose(c[0, 1], P2, atol=1e-12)
        c1 = c[0, 0]
    np.testing.assert_allclose(c1, P1, atol=1e-12)


def test_accept_rate_is_one_when_target_equals_draft():
    rng = np.random.default_rng(18)
    R, g, V, r = 3, 4, 32, 16
    base = rng.standard_normal((R, g, V)).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.3).astype(np.float32)
    W2 = (rng.standard_normal((r, V)) * 0.3).astype(np.float32)
    anchor = rng.integers(0, V, R).astype(np.int32)
    d = O.draft(base, W1, W2, "f32", anchor, rng.random((R, g)), 1.0)
    # target rows = the draft logits themselves
    prev = np.concatenate([anchor[:, None], d["tokens"][:, :-1]], axis=1)
    z = np.stack([base[:, k].astype(np.float64) + O.markov_bias(W1.astype(np.float64), W2.astype(np.float64),
                                                                   prev[:, k]) for k in range(g)], axis=1)
    tgt = np.concatenate([z, z[:, -1:]], axis=1)
    c = O.accept_rates(tgt, base, W1, W2, "f32", anchor, d["tokens"], 1.0)
    np.testing.assert_allclose(c, 1.0, atol=1e-12)


def test_accept_rate_is_one_minus_residual_mass_at_the_rejection():
    rng = np.random.default_rng(19)
    R, g, V, r = 64, 3, 40, 16
    base = (rng.standard_normal((R, g, V)) * 2).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.4).astype(np.float32)
    W2 = (rng.standard_normal((r, V)) * 0.4).astype(np.float32)
    anchor = rng.integers(0, V, R).astype(np.int32)
    tgt = np.concatenate([base, base[:, -1:]], axis=1) + rng.standard_normal((R, g + 1, V)).astype(np.float32)
    d = O.draft(base, W1, W2, "f32", anchor, rng.random((R, g)), 1.0)
    v = O.verify(tgt, base, W1, W2, "f32", anchor, d["tokens"], d["probs"], None,
                 rng.random((R, g)), rng.random(R), 1.0)
    c = O.accept_rates(tgt, base, W1, W2, "f32", anchor, d["tokens"], 1.0)
    rej = np.flatnonzero(v["accept_len"] < g)
    assert len(rej) > 10
    k = v["accept_len"][rej]                       # 0-based rejected position
    np.testing.assert_allclose(c[rej, k], 1.0 - v["residual_mass"][rej], atol=1e-12)


def test_accept_rate_of_disjoint_distributions_is_zero():
    V = 8
    base = np.full((1, 1, V), -40.0, np.float32)
    base[0, 0, 2] = 40.0
    tgt = np.full((1, 2, V), -40.0, np.float32)
    tgt[0, 0, 5] = 40.0
    z = np.zeros((V, 16), np.float32)
    c = O.accept_rates(tgt, base, z, z.T.copy(), "f32", np.array([0], np.int32), np.array([[2]]), 1.0)
    assert 0.0 <= c[0, 0] < 1e-30


def test_threshold_schedule_limits_and_prefixes():
    c = _sched_case(35, R=20, g=7, ties=True)
    s0 = O.schedule_threshold(c, 0.0)
    assert (s0["verify_len"] == 7).all()
    assert O.schedule_threshold(c, 1.5)["n_admitted"] == 0
    last = None
    for th in np.linspace(0.0, 1.0, 41):
        s = O.schedule_threshold(c, th)
        a, L = s["cum_conf"], s["verify_len"]
        for r in range(20):                          # admitted positions form a prefix
            assert (a[r, :L[r]] >= np.float32(th)).all() and (L[r] == 7 or a[r, L[r]] < np.float32(th))
        if last is not None:
            assert (L <= last).all()                 # raising the threshold never adds
        last = L


def test_threshold_at_the_cut_reproduces_the_prefix_scheduler():
    """The prefix scheduler's admitted set is {a >= a_(n*)} (distinct values),
    so a static threshold placed exactly at the cut selects the same set."""
    for seed in range(36, 46):
        rng = np.random.default_rng(seed)
        c = rng.uniform(0.3, 1.0, (24, 6)).astype(np.float32)
        sps = (1.0 / (1.0 + rng.uniform(0.005, 0.05) * np.arange(1, 200))).astype(np.float32)
        s = O.schedule(c, sps)
        n = s["n_admitted"]
        if n == 0 or n == c.size:
            continue
        a_sorted = s["cum_conf"].reshape(-1)[s["order"]]
        if a_sorted[n - 1] == a_sorted[n]:
            continue                                  # tie at the cut
        t = O.schedule_threshold(c, a_sorted[n - 1])
        assert t["n_admitted"] == n and (t["verify_len"] == s["verify_len"]).all()


# ---------------------------------------------------------------------------
# sequential temperature scaling (calibration map, ECE, left-to-right search)


def _sts_gold():
    return json.load(open(os.path.join(GOLD, "sts_worked_example.json")))


def _frac(s):
    """'a/b' or 'a/b - d' from the fixture, as a float."""
    if " - " in s:
        a, b = s.split(" - ")
        return abs(float(Fraction(a)) - float(b))
    return float(Fraction(s))


def test_sts_calibration_closed_forms():
    """c' = 1 / (1 + ((1 - c)/c)^(1/tau)): exact rationals when the odds ratio
    is a perfect power (worked example fixture)."""
    g = _sts_gold()
    for pos, key in ((0, "calibrated_pos1"), (1, "calibrated_pos2")):
        c = np.array([[g["conf"][0][pos]]])
        for tau, want in zip(g["grid"], g[key]):
            got = O.sts_calibrate(c, [tau])[0, 0]
            assert got == pytest.approx(float(Fraction(want)), rel=1e-14)
    # temperature 1 is the identity; 0 and 1 are fixed points; the map is
    # increasing in c for every temperature (token order preserved)
    rng = np.random.default_rng(3)
    c = np.sort(rng.uniform(0.001, 0.999, 200))[:, None]
    assert np.allclose(O.sts_calibrate(c, [1.0]), c, rtol=1e-13, atol=0)
    for tau in (0.3, 1.0, 2.5):
        ends = O.sts_calibrate(np.array([[0.0], [1.0]]), [tau])[:, 0]
        assert ends[0] == 0.0 and ends[1] == 1.0
        assert (np.diff(O.sts_calibrate(c, [tau])[:, 0]) > 0).all()
    # tau -> large flattens towards 1/2, tau -> small sharpens towards 0/1
    assert abs(O.sts_calibrate(np.array([[0.9]]), [1e6])[0, 0] - 0.5) < 1e-6
    assert O.sts_calibrate(np.array([[0.6]]), [0.01])[0, 0] > 1 - 1e-12


def test_ece_hand_example():
    e = _sts_gold()["ece_example"]
    assert O.ece(e["pred"], e["target"], 10) == pytest.approx(e["ece_bins10"], abs=1e-15)
    assert O.ece(e["pred"], e["target"], 2) == pytest.approx(e["ece_bins2"], abs=1e-15)
    # bin edges: p = k/bins opens bin k, p = 1 falls in the last bin
    assert O.ece([0.5, 1.0], [0.0, 0.0], 2) == pytest.approx(0.75)          # bins {0.5,1.0} -> |1.5|/2
    assert O.ece([0.5, 0.4999], [1.0, 0.0], 2) == pytest.approx((0.5 + 0.4999) / 2)
    # one bin: |mean prediction - mean target|; perfect predictions score 0
    rng = np.random.default_rng(4)
    p, t = rng.uniform(size=500), rng.uniform(size=500)
    assert O.ece(p, t, 1) == pytest.approx(abs(p.mean() - t.mean()), rel=1e-12)
    assert O.ece(p, p, 15) == 0.0


def test_sts_worked_example_is_cumulative():
    g = _sts_gold()
    r = O.sts_fit(np.array(g["conf"]), np.array(g["labels"]), g["grid"], g["bins"])
    want = np.array([[_frac(s) for s in row] for row in g["table"]])
    assert np.allclose(r["table"], want, rtol=1e-12, atol=1e-15)
    assert list(r["index"]) == g["index"] and list(r["tau"]) == g["tau"]
    assert list(r["index"]) != g["index_if_not_cumulative"]


def _planted_sts(seed, N, gamma, grid):
    """Labels l_k = sigmoid(t_k), confidences c_k = sigmoid(s_k t_k) with s_k a
    grid entry: temperature s_k undoes the distortion exactly."""
    rng = np.random.default_rng(seed)
    s = rng.choice(grid, size=gamma)
    t = rng.normal(1.0, 1.5, (N, gamma))
    lab = special.expit(t)
    conf = special.expit(s[None, :] * t)
    return conf, lab, s


def test_sts_recovers_planted_temperatures():
    grid = np.array([0.5, 0.75, 1.0, 1.5, 2.0, 3.0])
    for seed in range(3):
        conf, lab, s = _planted_sts(seed, 2000, 5, grid)
        r = O.sts_fit(conf, lab, grid, 15)
        assert np.array_equal(r["tau"], s)
        assert (r["ece"] < 1e-12).all()
        # every other candidate scores strictly worse
        for k in range(5):
            others = np.delete(r["table"][k], r["index"][k])
            assert (others > 1e-6).all()


def test_sts_left_to_right():
    """tau_k depends on positions 1..k only; follow= replays given choices."""
    grid = np.geomspace(0.25, 4.0, 17)
    rng = np.random.default_rng(9)
    conf = rng.uniform(0.05, 0.995, (800, 4))
    lab = np.clip(conf ** 1.7 + rng.normal(0, 0.05, conf.shape), 0, 1)
    r = O.sts_fit(conf, lab, grid, 10)
    conf2, lab2 = conf.copy(), lab.copy()
    conf2[:, 2:] = rng.uniform(0.05, 0.995, (800, 2))
    lab2[:, 2:] = rng.uniform(0, 1, (800, 2))
    r2 = O.sts_fit(conf2, lab2, grid, 10)
    assert np.array_equal(r["index"][:2], r2["index"][:2])
    assert np.array_equal(r["table"][:2], r2["table"][:2])
    # following a different choice at position 1 changes later tables only
    f = r["index"].copy()
    f[0] = (f[0] + 3) % len(grid)
    r3 = O.sts_fit(conf, lab, grid, 10, follow=f)
    assert np.array_equal(r3["table"][0], r["table"][0])
    assert not np.array_equal(r3["table"][1], r["table"][1])
    # a labels-all-one block with c = 1 everywhere scores 0 for every tau
    r4 = O.sts_fit(np.ones((10, 3)), np.ones((10, 3)), grid, 10)
    assert (r4["table"] == 0).all() and (r4["index"] == 0).all()


# ---------------------------------------------------------------------------
# RNN head (gated recurrent state over the in-block prefix)


def test_storage_rounding_ties_to_even():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is halfway between 1 and
    # 1 + 2^-7 (goes to the even 1), 1 + 3 * 2^-8 halfway between 1 + 2^-7 and
    # 1 + 2^-6 (goes to the even 1 + 2^-6); just above a tie rounds up
    v = O.to_storage([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -(1 + 2**-8), 0.0], "bf16")
    assert list(v) == [1.0, 1 + 2**-6, 1 + 2**-7, -1.0, 0.0]
    assert O.to_storage([1 + 2**-30, 1 + 2**-23], "f32").tolist() == [1.0, 1 + 2**-23]


def test_storage_rounds_once_from_float64():
    """The state is rounded once: just above a bf16 tie it goes up, although
    an fp32 rounding first would land on the tie and go to the even
    neighbour.  Subnormal bf16 values sit on the 2^-133 grid."""
    x = [1 + 2**-8 + 2**-30, 0.5 + 2**-9 + 2**-40, -(0.75 + 2**-9 + 2**-33)]
    assert O.to_storage(x, "bf16").tolist() == [1 + 2**-7, 0.5 + 2**-8, -(0.75 + 2**-8)]
    twice = O.to_storage(np.asarray(x, np.float32).astype(np.float64), "bf16")
    assert twice.tolist() == [1.0, 0.5, -0.75]
    sub = [2**-133 * 5.5, 2**-133 * 4.5, 2**-133 * 4.5 + 2**-160, 2**-127 * (1 + 2**-9)]
    assert O.to_storage(sub, "bf16").tolist() == [2**-133 * 6, 2**-133 * 4, 2**-133 * 5, 2**-127]


def _rnn_case(r=16, V=64, R=3, g=5, seed=0):
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((R, g, V)) * 2).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.7).astype(np.float32)
    W2 = (rng.standard_normal((r, V)) * 0.7).astype(np.float32)
    anchor = rng.integers(0, V, R).astype(np.int32)
    u = rng.uniform(size=(R, g)).astype(np.float32)
    return base, W1, W2, anchor, u


def test_rnn_constant_candidate_closed_form():
    """Wx = Ws = 0, update bias 0 (u = 1/2), candidate bias c: h = tanh(c) and
    s_k = (1 - 2^-k) tanh(c), up to the fp32 rounding of each stored state."""
    r, g = 16, 5
    base, W1, W2, anchor, u = _rnn_case(r=r, g=g)
    Wx = np.zeros((3, r, r), np.float32)
    Ws = np.zeros((3, r, r), np.float32)
    b = np.zeros((3, r), np.float32)
    b[1] = 0.7
    b[2] = np.linspace(-2, 2, r)
    out = O.draft_rnn(base, W1, W2, Wx, Ws, b, "f32", anchor, u, 1.0)
    want = (1 - 2.0 ** -np.arange(1, g + 1))[:, None] * np.tanh(b[2].astype(np.float64))[None, :]
    np.testing.assert_allclose(out["states"], np.broadcast_to(want, out["states"].shape), rtol=0, atol=5e-7)


@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
def test_rnn_with_open_update_gate_is_a_markov_head(w_dtype):
    """u = 1, candidate tanh(e) and no recurrence: s_k = tanh(W1[x_{k-1}]) in
    storage, so the RNN draft is the Markov draft with table tanh(W1)."""
    from gen.inputs import bf16_bits_from_f32
    r = 16
    base, W1, W2, anchor, u = _rnn_case(r=r, seed=1)
    Wx = np.zeros((3, r, r), np.float32)
    Wx[2] = np.eye(r, dtype=np.float32)
    Ws = np.zeros((3, r, r), np.float32)
    b = np.zeros((3, r), np.float32)
    b[0] = 60.0                                      # sigmoid(60) == 1.0 in float64
    conv = (lambda x: bf16_bits_from_f32(x)) if w_dtype == "bf16" else (lambda x: x)
    W1s, W2s, Wxs, Wss = conv(W1), conv(W2), conv(Wx), conv(Ws)
    W1t = O.to_storage(np.tanh(O.widen_weights(W1s, w_dtype)), w_dtype).astype(np.float32)
    for T in (1.0, 0.0):
        a = O.draft_rnn(base, W1s, W2s, Wxs, Wss, b, w_dtype, anchor, u, T)
        m = O.draft(base, conv(W1t), W2s, w_dtype, anchor, u, T)
        assert np.array_equal(a["tokens"], m["tokens"])
        np.testing.assert_allclose(a["probs"], m["probs"], rtol=1e-13, atol=0)
        np.testing.assert_allclose(a["stats"], m["stats"], rtol=1e-13, atol=0)


def test_rnn_state_remembers_beyond_the_previous_token():
    """With u = 1/2 and candidate tanh(e): s_2 = 1/4 tanh(W1[x_0]) + 1/2 tanh(W1[x_1]),
    so the anchor still moves the position-2 bias (the Markov bias does not)."""
    r, V = 16, 64
    _, W1, W2, _, _ = _rnn_case(r=r, V=V, seed=2)
    W1_64 = W1.astype(np.float64)
    Wx = np.zeros((3, r, r))
    Wx[2] = np.eye(r)
    Ws = np.zeros((3, r, r))
    b = np.zeros((3, r))
    s0 = np.zeros((1, r))
    x1 = 5
    s2 = {}
    for a in (3, 9):
        s1 = O.rnn_state_update(W1_64[[a]], s0, Wx, Ws, b, "f32")
        s2[a] = O.rnn_state_update(W1_64[[x1]], s1, Wx, Ws, b, "f32")[0]
        want = 0.25 * np.tanh(W1_64[a]) + 0.5 * np.tanh(W1_64[x1])
        np.testing.assert_allclose(s2[a], want, rtol=0, atol=3e-7)
    assert np.abs(s2[3] - s2[9]).max() > 1e-2


def test_rnn_reset_gate_closes_the_recurrence():
    """u = 1, candidate tanh(e + (g * s) M): a closed reset gate (g = 0) gives
    s_2 = tanh(e_1); an open one (g = 1) gives s_2 = tanh(e_1 + s_1 M)."""
    r, V = 8, 32
    rng = np.random.default_rng(3)
    W1_64 = rng.standard_normal((V, r)) * 0.8
    M = rng.standard_normal((r, r)) * 0.8
    Wx = np.zeros((3, r, r))
    Wx[2] = np.eye(r)
    Ws = np.zeros((3, r, r))
    Ws[2] = M
    for bg, open_gate in ((-60.0, False), (60.0, True)):
        b = np.zeros((3, r))
        b[0], b[1] = 60.0, bg
        s1 = O.rnn_state_update(W1_64[[2]], np.zeros((1, r)), Wx, Ws, b, "f32")
        s2 = O.rnn_state_update(W1_64[[7]], s1, Wx, Ws, b, "f32")
        want = np.tanh(W1_64[7] + (s1[0] @ M if open_gate else 0.0))
        np.testing.assert_allclose(s2[0], want, rtol=0, atol=3e-7)


class _TinyRNN(_Tiny):
    """The same single-request V = 4, gamma = 2 round drafted by an RNN head."""

    def __init__(self, seed, T=1.0):
        super().__init__(seed, T)
        rng = np.random.default_rng(seed + 1000)
        self.Wx = (rng.standard_normal((3, 2, 2)) * 1.2).astype(np.float32)
        self.Ws = (rng.standard_normal((3, 2, 2)) * 1.2).astype(np.float32)
        self.b = (rng.standard_normal((3, 2)) * 0.5).astype(np.float32)
        self.W2 = (self.W2 * 2.5).astype(np.float32)     # a stronger state bias

    def draft(self, u1, u2):
        r = O.draft_rnn(self.base, self.W1, self.W2, self.Wx, self.Ws, self.b, "f32", self.anchor,
                        np.array([[u1, u2]]), self.T)
        return r["tokens"][0], r["probs"][0]

    def verify(self, x, q, L, ua1, ua2, uf):
        # the states of this drafted prefix (they depend on the anchor and x_1 only)
        u = np.zeros((1, 2))
        st = O.draft_rnn(self.base, self.W1, self.W2, self.Wx, self.Ws, self.b, "f32", self.anchor,
                         u, 0.0)["states"]
        W1_64 = self.W1.astype(np.float64)
        Wx, Ws, b = (self.Wx.astype(np.float64), self.Ws.astype(np.float64), self.b.astype(np.float64))
        s1 = O.rnn_state_update(W1_64[self.anchor], np.zeros((1, 2)), Wx, Ws, b, "f32")
        s2 = O.rnn_state_update(W1_64[[x[0]]], s1, Wx, Ws, b, "f32")
        assert np.array_equal(st[0, 0], s1[0])          # s_1 does not depend on any drafted token
        states = np.stack([s1[0], s2[0]])[None]
        tgt = np.stack([self.T1, self.T2[x[0]], self.T3])[None]
        return O.verify(tgt, self.base, None, self.W2, "f32", None, x[None], q[None], np.array([L]),
                        np.array([[ua1, ua2]]), np.array([uf]), self.T, states=states)


@pytest.mark.parametrize("seed", [21, 22])
@pytest.mark.parametrize("L", [1, 2])
def test_rnn_lossless_exact(seed, L):
    """Exact laws of the first and second emitted tokens equal the target's
    when the RNN head drafts and verify recomputes its rows from the states."""
    t = _TinyRNN(seed)
    np.testing.assert_allclose(t.first_token_law(lambda a: L), _softmax(t.T1), atol=1e-12)
    for a in range(4):
        np.testing.assert_allclose(t.second_token_law(a, L), _softmax(t.T2[a]), atol=1e-12)
