"""Seeded input generation for one round of each workload.

Every tensor has its own PCG64 stream, ``numpy.random.default_rng([seed,
tensor_id, ...])``.  Base and target logits use one stream per request row, so
any subset of rows can be regenerated on its own with identical values (the
oracle checks sampled rows of the full-size workloads that way).  Uniforms are
drawn from ``default_rng(seed_u)`` (seed 0 unless overridden) in the order
u_draft [R, gamma], u_accept [R, gamma], u_final [R], as float32 values in [0, 1).

Nothing here computes any part of the method.
"""

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import config as _config

TID_BASE, TID_TARGET, TID_SIGMA, TID_W1, TID_W2, TID_ANCHOR, TID_CONF = 1, 2, 3, 4, 5, 6, 7
TID_CONF_LAG = 8   # confidences of two steps earlier (asynchronous scheduler input)


def bf16_bits_from_f32(x):
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite (no
    overflow of the 32-bit rounding add).
    """
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def cost_table(kind, R, gamma):
    """Synthetic verify-throughput table SPS: entry i is for verify batch B = i + 1."""
    if kind is None:
        return None
    if kind == "linear":
        n = R * (gamma + 1)
        B = np.arange(1, n + 1, dtype=np.float64)
        return (1.0 / (1.0 + 0.1 * B)).astype(np.float32)
    if kind == "stairs64":
        B = np.arange(1, 1025, dtype=np.float64)
        return (1.0 / (1.0 + 0.001 * np.ceil(B / 64.0))).astype(np.float32)
    if kind == "stairs256_cliff2048":
        B = np.arange(1, 4097, dtype=np.float64)
        return (1.0 / (1.0 + 0.0002 * np.ceil(B / 256.0) + 0.5 * (B > 2048))).astype(np.float32)
    raise ValueError(f"unknown cost table {kind!r}")


def _target_sigmas(d, seed):
    R = d["R"]
    kind = d["target"]
    if kind[0] == "const":
        return np.full(R, kind[1], dtype=np.float64)
    if kind[0] == "uniform":
        return np.random.default_rng([seed, TID_SIGMA]).uniform(kind[1], kind[2], R)
    if kind[0] == "split":
        s = np.full(R, kind[2], dtype=np.float64)
        s[: R // 2] = kind[1]
        return s
    raise ValueError(f"unknown target recipe {kind!r}")


def _fill_row(d, seed, r, sigma, base_out, target_out):
    """Draw base rows 0..gamma (gamma + 1 of them) and target rows of request r."""
    g, V = d["gamma"], d["V"]
    rb = np.random.default_rng([seed, TID_BASE, r])
    ext = rb.standard_normal((g + 1, V), dtype=np.float32)
    if d["base"] == "bimodal":
        ext *= np.float32(3.0)
        for j in range(g + 1):
            ext[j, rb.choice(V, size=min(2, V), replace=False)] += np.float32(6.0)
    elif d["base"] == "peaked":
        ext *= np.float32(2.0)
        for j in range(g + 1):
            cnt = int(rb.integers(1, 4))
            ext[j, rb.choice(V, size=min(cnt, V), replace=False)] += np.float32(8.0)
    else:
        raise ValueError(f"unknown base recipe {d['base']!r}")
    if base_out is not None:
        base_out[:] = ext[:g]
    if target_out is not None:
        rt = np.random.default_rng([seed, TID_TARGET, r])
        noise = rt.standard_normal((g + 1, V), dtype=np.float32)
        np.multiply(noise, np.float32(sigma), out=noise)
        np.add(ext, noise, out=target_out)


def make_inputs(cfg, seed=None, seed_u=0, rows=None, with_target=True, threads=None):
    """Generate one round's inputs for workload ``cfg``.

    cfg      an int key of ``gen.CONFIGS``, an alternate key, or a dict
    seed     stream seed for every tensor except the uniforms (default: the
             int config key, or 0 for dicts/alternates)
    seed_u   seed of the uniform stream
    rows     optional sorted list of request rows; base/target/uniform rows
             are then generated for those rows only (values identical to the
             same rows of the full workload), while W1, W2, anchors of those
             rows, confidences and the cost table stay whole-workload
    Returns a dict of numpy arrays plus ``cfg`` (the workload description).
    """
    d = _config(cfg)
    if seed is None:
        seed = cfg if isinstance(cfg, int) else 0
    R, g, V, r = d["R"], d["gamma"], d["V"], d["r"]
    row_ids = np.arange(R) if rows is None else np.asarray(sorted(rows), dtype=np.int64)
    n = len(row_ids)

    sig = _target_sigmas(d, seed)
    base = np.empty((n, g, V), dtype=np.float32)
    target = np.empty((n, g + 1, V), dtype=np.float32) if with_target else None
    workers = threads or min(8, os.cpu_count() or 1)

    def work(i):
        _fill_row(d, seed, int(row_ids[i]), sig[row_ids[i]], base[i],
                  None if target is None else target[i])

    if n * (g + 1) * V > (1 << 22) and workers > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(n)))
    else:
        for i in range(n):
            work(i)

    w1 = np.random.default_rng([seed, TID_W1]).standard_normal((V, r), dtype=np.float32)
    w1 *= np.float32(d["w_sigma"])
    w2 = np.random.default_rng([seed, TID_W2]).standard_normal((r, V), dtype=np.float32)
    w2 *= np.float32(d["w_sigma"])
    if d["w_dtype"] == "bf16":
        w1, w2 = bf16_bits_from_f32(w1), bf16_bits_from_f32(w2)
    anchor = np.random.default_rng([seed, TID_ANCHOR]).integers(0, V, R).astype(np.int32)

    def draw_conf(tid):
        rc = np.random.default_rng([seed, tid])
        if d["conf"][0] == "uniform":
            c = rc.uniform(d["conf"][1], d["conf"][2], (R, g))
        elif d["conf"][0] == "beta":
            c = rc.beta(d["conf"][1], d["conf"][2], (R, g))
        else:
            raise ValueError(f"unknown confidence recipe {d['conf']!r}")
        return c.astype(np.float32)

    conf = conf_lag = None
    if d["conf"] is not None:
        conf = draw_conf(TID_CONF)
        # stand-in for the confidences of two steps earlier: same recipe,
        # independent draws
        conf_lag = draw_conf(TID_CONF_LAG)

    ru = np.random.default_rng(seed_u)
    u_draft = ru.random((R, g), dtype=np.float32)
    u_accept = ru.random((R, g), dtype=np.float32)
    u_final = ru.random(R, dtype=np.float32)

    out = dict(cfg=d, rows=row_ids, base=base, target=target, W1=w1, W2=w2,
               w_dtype=d["w_dtype"], anchor=anchor[row_ids], anchor_all=anchor,
               u_draft=u_draft[row_ids], u_accept=u_accept[row_ids], u_final=u_final[row_ids],
               conf=conf, conf_lag=conf_lag, sps=cost_table(d["table"], R, g))
    return out


def algorithmic_bytes(cfg_dict, emitted_rows, scheduled_rows):
    """Bytes a round must move with each needed input read once.

    emitted_rows   sum over requests of (accepted + 1): target rows needed
    scheduled_rows sum over requests of (verify length + 1)
    Returns (minimum, as_scheduled) in bytes.
    """
    d = cfg_dict
    R, g, V, r = d["R"], d["gamma"], d["V"], d["r"]
    wb = 2 if d["w_dtype"] == "bf16" else 4
    fixed = 4 * R * g * V + wb * r * V + wb * R * g * r
    return fixed + 4 * V * emitted_rows, fixed + 4 * V * scheduled_rows


__all__ = ["make_inputs", "bf16_bits_from_f32", "bf16_bits_to_f32", "cost_table",
           "algorithmic_bytes"]
