"""Seeded synthetic held-out set for sequential temperature scaling.

A stand-in for a held-out set of drafted blocks: per block and position k a
conditional acceptance label in (0, 1) (what the acceptance-label pass
produces) and a raw confidence-head output that is over-confident, i.e. a
sharpened and noisy version of the label on the logit scale.  The pages report
an over-confident head (ECE of a few per cent before calibration); the
constants below are a choice that reproduces that range.  Nothing here is the
calibration arithmetic itself.
"""

import numpy as np

TID_STS_LABEL, TID_STS_NOISE = 101, 102


def _logistic(x):
    return 1.0 / (1.0 + np.exp(-x))


def make_sts_inputs(N, gamma, G, bins=15, seed=0, tau_lo=0.25, tau_hi=4.0):
    """Held-out set: conf, labels float32 [N, gamma]; grid float32 [G] (geometric
    from tau_lo to tau_hi); bins.

    label logit t_k ~ N(2.2 - 0.15 k, 1.2); label = logistic(t_k);
    confidence = logistic(s_k t_k + e), s_k = 1.25 + 0.05 k, e ~ N(0, 0.5).
    """
    conf = np.empty((N, gamma), dtype=np.float32)
    lab = np.empty((N, gamma), dtype=np.float32)
    for k in range(gamma):
        t = np.random.default_rng([seed, TID_STS_LABEL, k]).normal(2.2 - 0.15 * k, 1.2, N)
        e = np.random.default_rng([seed, TID_STS_NOISE, k]).normal(0.0, 0.5, N)
        lab[:, k] = _logistic(t)
        conf[:, k] = _logistic((1.25 + 0.05 * k) * t + e)
    grid = np.geomspace(tau_lo, tau_hi, G).astype(np.float32) if G > 1 else np.array([1.0], np.float32)
    return dict(conf=conf, labels=lab, grid=grid, bins=int(bins), N=N, gamma=gamma, G=G)
