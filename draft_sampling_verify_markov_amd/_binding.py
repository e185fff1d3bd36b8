"""ctypes marshalling for libdspark.so (see include/dspark.h for the contract)."""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
DSPARK_W_BF16, DSPARK_W_F32 = 0, 1
STATUS = {0: "DSPARK_OK", -1: "DSPARK_EINVAL", -2: "DSPARK_ENOSPC", -3: "DSPARK_EHIP"}
DERR_BITS = {1: "NONFINITE", 2: "UNIFORM", 4: "CONF", 8: "TOKEN", 16: "PROB", 32: "LENGTH", 64: "CALIB", 128: "SYNC"}

_lib = None


class DSparkError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


class DSparkDeviceError(DSparkError):
    """Device-side error bits (DSPARK_DERR_*) found after a round."""

    def __init__(self, bits):
        names = ", ".join(v for k, v in DERR_BITS.items() if bits & k)
        RuntimeError.__init__(self, f"device-side error bits {bits:#x} ({names}) set by the round")
        self.status = None
        self.bits = bits


def lib_path():
    return os.environ.get("DSPARK_LIB", os.path.join(HERE, "libdspark.so"))


def load_library():
    """Load libdspark.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m draft_sampling_verify_markov_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.dspark_workspace_size.argtypes = [I, I, I, I]
    lib.dspark_workspace_size.restype = Z
    lib.dspark_workspace_init.argtypes = [P, Z, P]
    lib.dspark_workspace_init.restype = I
    lib.dspark_device_error.argtypes = [P, Z, ctypes.POINTER(ctypes.c_int32), P]
    lib.dspark_device_error.restype = I
    lib.dspark_status_string.argtypes = [I]
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_draft.argtypes = [P, P, P, I, P, P, I, I, I, I, F, P, P, P, P, Z, P]
    lib.dspark_draft.restype = I
    lib.dspark_draft_noalloc.argtypes = [P, P, P, I, P, P, I, I, I, I, F, P, P, P, P, P]
    lib.dspark_draft_noalloc.restype = I
    lib.dspark_schedule.argtypes = [P, P, I, I, I, P, P, P, P, Z, P]
    lib.dspark_schedule.restype = I
    lib.dspark_schedule_async.argtypes = [P, P, P, I, I, I, P, P, P, P, Z, P]
    lib.dspark_schedule_async.restype = I
    lib.dspark_schedule_threshold.argtypes = [P, F, I, I, P, P, P, P, Z, P]
    lib.dspark_schedule_threshold.restype = I
    lib.dspark_accept_rates.argtypes = [P, P, P, P, I, P, P, P, I, I, I, I, F, P, P, Z, P]
    lib.dspark_accept_rates.restype = I
    lib.dspark_verify.argtypes = [P, P, P, P, I, P, P, P, P, P, P, P, I, I, I, I, F, P, P, P, P, Z, P]
    lib.dspark_verify.restype = I
    lib.dspark_verify_stream.argtypes = [P, P, I, I, I, F, P, Z, P]
    lib.dspark_verify_stream.restype = I
    lib.dspark_verify_finish.argtypes = lib.dspark_verify.argtypes
    lib.dspark_verify_finish.restype = I
    lib.dspark_verify_rnn_finish.argtypes = [P, P, P, P, I, P, P, P, P, P, P, I, I, I, I, F, P, P, P, P, Z, P]
    lib.dspark_verify_rnn_finish.restype = I
    lib.dspark_draft_rnn.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, F, P, P, P, P, P, Z, P]
    lib.dspark_draft_rnn.restype = I
    lib.dspark_verify_rnn.argtypes = [P, P, P, P, I, P, P, P, P, P, P, I, I, I, I, F, P, P, P, P, Z, P]
    lib.dspark_verify_rnn.restype = I
    lib.dspark_sts_workspace_size.argtypes = [I, I, I, I]
    lib.dspark_sts_workspace_size.restype = Z
    lib.dspark_sts_fit.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, Z, P]
    lib.dspark_sts_fit.restype = I
    lib.dspark_sts_apply.argtypes = [P, P, I, I, P, P, Z, P]
    lib.dspark_sts_apply.restype = I
    lib.dspark_profile_arm.argtypes = [I, P, P, I, I]
    lib.dspark_profile_arm.restype = I
    lib.dspark_profile_disarm.argtypes = []
    lib.dspark_profile_disarm.restype = I
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise DSparkError(fn, status)


def _ptr(t, dtype, shape, name, device):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _wtype(W):
    if W.dtype == torch.bfloat16 or W.dtype in (torch.int16, torch.uint16):
        return DSPARK_W_BF16
    if W.dtype == torch.float32:
        return DSPARK_W_F32
    raise TypeError(f"W1/W2 dtype {W.dtype}: expected bfloat16 (or its uint16 bits) or float32")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(R, gamma, V, r):
    n = load_library().dspark_workspace_size(R, gamma, V, r)
    if n == 0:
        raise ValueError(f"sizes outside the library limits: R={R} gamma={gamma} V={V} r={r}")
    return n


def new_workspace(R, gamma, V, r, device):
    """Allocate (torch) and clear a workspace for these sizes."""
    ws = torch.empty(workspace_size(R, gamma, V, r), dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def workspace_init(ws):
    _check("dspark_workspace_init",
           load_library().dspark_workspace_init(ws.data_ptr(), ws.numel(), _stream(ws.device)))


def device_error(ws):
    """Return (and clear) the device-side data error bits of a workspace."""
    v = ctypes.c_int32(0)
    _check("dspark_device_error", load_library().dspark_device_error(
        ws.data_ptr(), ws.numel(), ctypes.byref(v), _stream(ws.device)))
    return int(v.value)


def draft(base, W1, W2, anchor, u_draft, temperature, ws, out=None):
    """dspark_draft.  Returns (draft_tokens, draft_probs, draft_stats)."""
    R, g, V = base.shape
    r = W1.shape[1]
    dev = base.device
    wt = _wtype(W1)
    wdt = W1.dtype
    if out is None:
        out = (torch.empty((R, g), dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev),
               torch.empty((R, g, 2), dtype=torch.float32, device=dev))
    tok, prob, stats = out
    args = (_ptr(base, torch.float32, (R, g, V), "base", dev),
            _ptr(W1, wdt, (V, r), "W1", dev), _ptr(W2, wdt, (r, V), "W2", dev), wt,
            _ptr(anchor, torch.int32, (R,), "anchor", dev),
            _ptr(u_draft, torch.float32, (R, g), "u_draft", dev),
            R, g, V, r, float(temperature),
            _ptr(tok, torch.int32, (R, g), "draft_tokens", dev),
            _ptr(prob, torch.float32, (R, g), "draft_probs", dev),
            _ptr(stats, torch.float32, (R, g, 2), "draft_stats", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_draft", load_library().dspark_draft(*args))
    return tok, prob, stats


def draft_noalloc(base, W1, W2, anchor, u_draft, temperature, device_error, out):
    """dspark_draft_noalloc: dspark_draft without a workspace (static device
    scratch).  ``out`` = (draft_tokens, draft_probs, draft_stats) preallocated
    by the caller, ``device_error`` a 1-element int32 device tensor the error
    bits are OR-ed into.  Allocates nothing.  Returns ``out``."""
    R, g, V = base.shape
    r = W1.shape[1]
    dev = base.device
    wt = _wtype(W1)
    wdt = W1.dtype
    tok, prob, stats = out
    args = (_ptr(base, torch.float32, (R, g, V), "base", dev),
            _ptr(W1, wdt, (V, r), "W1", dev), _ptr(W2, wdt, (r, V), "W2", dev), wt,
            _ptr(anchor, torch.int32, (R,), "anchor", dev),
            _ptr(u_draft, torch.float32, (R, g), "u_draft", dev),
            R, g, V, r, float(temperature),
            _ptr(tok, torch.int32, (R, g), "draft_tokens", dev),
            _ptr(prob, torch.float32, (R, g), "draft_probs", dev),
            _ptr(stats, torch.float32, (R, g, 2), "draft_stats", dev),
            _ptr(device_error, torch.int32, (1,), "device_error", dev), _stream(dev))
    _check("dspark_draft_noalloc", load_library().dspark_draft_noalloc(*args))
    return out


def schedule(conf, sps, ws, out=None, with_cum=True):
    """dspark_schedule.  Returns (verify_len, n_admitted[1], cum_conf or None)."""
    R, g = conf.shape
    dev = conf.device
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev) if with_cum else None)
    L, n, a = out
    args = (_ptr(conf, torch.float32, (R, g), "conf", dev),
            _ptr(sps, torch.float32, (sps.numel(),), "sps", dev), R, g, sps.numel(),
            _ptr(L, torch.int32, (R,), "verify_len", dev), _ptr(n, torch.int32, (1,), "n_admitted", dev),
            _ptr(a, torch.float32, (R, g), "cum_conf", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_schedule", load_library().dspark_schedule(*args))
    return L, n, a


def schedule_async(conf, conf_lag, sps, ws, out=None, with_cum=True):
    """dspark_schedule_async.  Returns (verify_len, K[1], cum_conf or None)."""
    R, g = conf.shape
    dev = conf.device
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev) if with_cum else None)
    L, n, a = out
    args = (_ptr(conf, torch.float32, (R, g), "conf", dev),
            _ptr(conf_lag, torch.float32, (R, g), "conf_lag", dev),
            _ptr(sps, torch.float32, (sps.numel(),), "sps", dev), R, g, sps.numel(),
            _ptr(L, torch.int32, (R,), "verify_len", dev), _ptr(n, torch.int32, (1,), "n_admitted", dev),
            _ptr(a, torch.float32, (R, g), "cum_conf", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_schedule_async", load_library().dspark_schedule_async(*args))
    return L, n, a


def schedule_threshold(conf, theta, ws, out=None, with_cum=True):
    """dspark_schedule_threshold.  Returns (verify_len, n_admitted[1], cum_conf or None)."""
    R, g = conf.shape
    dev = conf.device
    if out is None:
        out = (torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev) if with_cum else None)
    L, n, a = out
    args = (_ptr(conf, torch.float32, (R, g), "conf", dev), float(theta), R, g,
            _ptr(L, torch.int32, (R,), "verify_len", dev), _ptr(n, torch.int32, (1,), "n_admitted", dev),
            _ptr(a, torch.float32, (R, g), "cum_conf", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_schedule_threshold", load_library().dspark_schedule_threshold(*args))
    return L, n, a


def accept_rates(target, base, W1, W2, anchor, draft_tokens, draft_stats, temperature, ws, out=None):
    """dspark_accept_rates.  Returns accept_rate [R, gamma] fp32."""
    R, g1, V = target.shape
    g = g1 - 1
    r = W1.shape[1]
    dev = target.device
    wt = _wtype(W1)
    wdt = W1.dtype
    if out is None:
        out = torch.empty((R, g), dtype=torch.float32, device=dev)
    args = (_ptr(target, torch.float32, (R, g + 1, V), "target", dev),
            _ptr(base, torch.float32, (R, g, V), "base", dev),
            _ptr(W1, wdt, (V, r), "W1", dev), _ptr(W2, wdt, (r, V), "W2", dev), wt,
            _ptr(anchor, torch.int32, (R,), "anchor", dev),
            _ptr(draft_tokens, torch.int32, (R, g), "draft_tokens", dev),
            _ptr(draft_stats, torch.float32, (R, g, 2), "draft_stats", dev),
            R, g, V, r, float(temperature), _ptr(out, torch.float32, (R, g), "accept_rate", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_accept_rates", load_library().dspark_accept_rates(*args))
    return out


def verify(target, base, W1, W2, anchor, draft_tokens, draft_probs, draft_stats, verify_len,
           u_accept, u_final, temperature, ws, out=None, with_probs=True, finish_only=False):
    """dspark_verify (dspark_verify_finish with finish_only, after verify_stream).
    Returns (out_tokens, accept_len, target_probs or None)."""
    R, g1, V = target.shape
    g = g1 - 1
    r = W1.shape[1]
    dev = target.device
    wt = _wtype(W1)
    wdt = W1.dtype
    if out is None:
        out = (torch.empty((R, g + 1), dtype=torch.int32, device=dev),
               torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev) if with_probs else None)
    ot, al, tp = out
    args = (_ptr(target, torch.float32, (R, g + 1, V), "target", dev),
            _ptr(base, torch.float32, (R, g, V), "base", dev),
            _ptr(W1, wdt, (V, r), "W1", dev), _ptr(W2, wdt, (r, V), "W2", dev), wt,
            _ptr(anchor, torch.int32, (R,), "anchor", dev),
            _ptr(draft_tokens, torch.int32, (R, g), "draft_tokens", dev),
            _ptr(draft_probs, torch.float32, (R, g), "draft_probs", dev),
            _ptr(draft_stats, torch.float32, (R, g, 2), "draft_stats", dev),
            _ptr(verify_len, torch.int32, (R,), "verify_len", dev),
            _ptr(u_accept, torch.float32, (R, g), "u_accept", dev),
            _ptr(u_final, torch.float32, (R,), "u_final", dev),
            R, g, V, r, float(temperature),
            _ptr(ot, torch.int32, (R, g + 1), "out_tokens", dev),
            _ptr(al, torch.int32, (R,), "accept_len", dev),
            _ptr(tp, torch.float32, (R, g), "target_probs", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    fn = "dspark_verify_finish" if finish_only else "dspark_verify"
    _check(fn, getattr(load_library(), fn)(*args))
    return ot, al, tp


def verify_stream(target, verify_len, temperature, ws):
    """dspark_verify_stream: the target-row partials (draft-independent part of verify)."""
    R, g1, V = target.shape
    dev = target.device
    args = (_ptr(target, torch.float32, (R, g1, V), "target", dev),
            _ptr(verify_len, torch.int32, (R,), "verify_len", dev), R, g1 - 1, V, float(temperature),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_verify_stream", load_library().dspark_verify_stream(*args))


def draft_rnn(base, W1, W2, Wx, Ws, rnn_bias, anchor, u_draft, temperature, ws, out=None):
    """dspark_draft_rnn.  Returns (draft_tokens, draft_probs, draft_stats, states)."""
    R, g, V = base.shape
    r = W1.shape[1]
    dev = base.device
    wt, wdt = _wtype(W1), W1.dtype
    if out is None:
        out = (torch.empty((R, g), dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev),
               torch.empty((R, g, 2), dtype=torch.float32, device=dev),
               torch.empty((R, g, r), dtype=wdt, device=dev))
    tok, prob, stats, states = out
    args = (_ptr(base, torch.float32, (R, g, V), "base", dev), _ptr(W1, wdt, (V, r), "W1", dev),
            _ptr(W2, wdt, (r, V), "W2", dev), _ptr(Wx, wdt, (3, r, r), "Wx", dev), _ptr(Ws, wdt, (3, r, r), "Ws", dev),
            _ptr(rnn_bias, torch.float32, (3, r), "rnn_bias", dev), wt,
            _ptr(anchor, torch.int32, (R,), "anchor", dev), _ptr(u_draft, torch.float32, (R, g), "u_draft", dev),
            R, g, V, r, float(temperature),
            _ptr(tok, torch.int32, (R, g), "draft_tokens", dev), _ptr(prob, torch.float32, (R, g), "draft_probs", dev),
            _ptr(stats, torch.float32, (R, g, 2), "draft_stats", dev), _ptr(states, wdt, (R, g, r), "states", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_draft_rnn", load_library().dspark_draft_rnn(*args))
    return tok, prob, stats, states


def verify_rnn(target, base, states, W2, draft_tokens, draft_probs, draft_stats, verify_len, u_accept, u_final,
               temperature, ws, out=None, with_probs=True, finish_only=False):
    """dspark_verify_rnn (dspark_verify_rnn_finish with finish_only, after verify_stream).
    Returns (out_tokens, accept_len, target_probs or None)."""
    R, g1, V = target.shape
    g = g1 - 1
    r = states.shape[2]
    dev = target.device
    wt, wdt = _wtype(W2), W2.dtype
    if out is None:
        out = (torch.empty((R, g + 1), dtype=torch.int32, device=dev),
               torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty((R, g), dtype=torch.float32, device=dev) if with_probs else None)
    ot, al, tp = out
    args = (_ptr(target, torch.float32, (R, g + 1, V), "target", dev),
            _ptr(base, torch.float32, (R, g, V), "base", dev),
            _ptr(states, wdt, (R, g, r), "states", dev), _ptr(W2, wdt, (r, V), "W2", dev), wt,
            _ptr(draft_tokens, torch.int32, (R, g), "draft_tokens", dev),
            _ptr(draft_probs, torch.float32, (R, g), "draft_probs", dev),
            _ptr(draft_stats, torch.float32, (R, g, 2), "draft_stats", dev),
            _ptr(verify_len, torch.int32, (R,), "verify_len", dev),
            _ptr(u_accept, torch.float32, (R, g), "u_accept", dev),
            _ptr(u_final, torch.float32, (R,), "u_final", dev),
            R, g, V, r, float(temperature),
            _ptr(ot, torch.int32, (R, g + 1), "out_tokens", dev),
            _ptr(al, torch.int32, (R,), "accept_len", dev),
            _ptr(tp, torch.float32, (R, g), "target_probs", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    fn = "dspark_verify_rnn_finish" if finish_only else "dspark_verify_rnn"
    _check(fn, getattr(load_library(), fn)(*args))
    return ot, al, tp


def sts_workspace_size(N, gamma, G, bins):
    n = load_library().dspark_sts_workspace_size(N, gamma, G, bins)
    if n == 0:
        raise ValueError(f"sizes outside the calibration limits: N={N} gamma={gamma} G={G} bins={bins}")
    return n


def new_sts_workspace(N, gamma, G, bins, device):
    """Allocate (torch) and clear a calibration workspace for these sizes."""
    ws = torch.empty(sts_workspace_size(N, gamma, G, bins), dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def sts_fit(conf, labels, grid, bins, ws, out=None, with_table=False):
    """dspark_sts_fit.  Returns (tau [gamma] fp32, tau_index [gamma] int32,
    ece [gamma] fp64, ece_table [gamma, G] fp64 or None)."""
    N, g = conf.shape
    G = grid.shape[0]
    dev = conf.device
    if out is None:
        out = (torch.empty(g, dtype=torch.float32, device=dev), torch.empty(g, dtype=torch.int32, device=dev),
               torch.empty(g, dtype=torch.float64, device=dev),
               torch.empty((g, G), dtype=torch.float64, device=dev) if with_table else None)
    tau, idx, ece, table = out
    args = (_ptr(conf, torch.float32, (N, g), "conf", dev), _ptr(labels, torch.float32, (N, g), "labels", dev),
            _ptr(grid, torch.float32, (G,), "grid", dev), N, g, G, int(bins),
            _ptr(tau, torch.float32, (g,), "tau", dev), _ptr(idx, torch.int32, (g,), "tau_index", dev),
            _ptr(ece, torch.float64, (g,), "ece", dev), _ptr(table, torch.float64, (g, G), "ece_table", dev),
            ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_sts_fit", load_library().dspark_sts_fit(*args))
    return tau, idx, ece, table


def sts_apply(conf, tau, ws, out=None):
    """dspark_sts_apply.  Returns the calibrated confidences [R, gamma] fp32."""
    R, g = conf.shape
    dev = conf.device
    if out is None:
        out = torch.empty((R, g), dtype=torch.float32, device=dev)
    args = (_ptr(conf, torch.float32, (R, g), "conf", dev), _ptr(tau, torch.float32, (g,), "tau", dev), R, g,
            _ptr(out, torch.float32, (R, g), "conf_out", dev), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("dspark_sts_apply", load_library().dspark_sts_apply(*args))
    return out


_side_streams = {}


def _side_stream(device):
    if device not in _side_streams:
        _side_streams[device] = torch.cuda.Stream(device=device)
    return _side_streams[device]


def run_round(dev_inputs, temperature, ws, use_scheduler=True, ws_sched=None, scheduler="early", theta=None,
              head="markov", check=False):
    """draft -> schedule -> verify on a dict of device tensors.

    The scheduler reads only confidences and the cost table, and verify's
    target-row stream reads only the target and the verify lengths: both run
    on a side stream (forked from and joined back to the current stream;
    capturable into a HIP graph) while the draft runs on the current stream;
    verify then finishes on the current stream.  The draft is enqueued first,
    on the stream that needs no event wait, so its workgroups are resident
    before the side stream's kernels take the free slots (with the draft
    behind the event wait instead, eager rounds lost up to 130 microseconds
    to target-row blocks that filled the compute units before the one-launch
    draft could start).  The early-stop and asynchronous schedulers on a pool
    of at most 1024 candidates, and the static-threshold scheduler, are
    workgroups small enough to share a compute unit with the one-launch draft
    and run beside it; larger pools are scheduled first, before the fork.
    The scheduler uses its own small workspace
    ``ws_sched`` (allocated here if not given).  ``scheduler`` is
    "early" (dspark_schedule), "async" (dspark_schedule_async with the
    lagged confidences ``conf_lag`` of the input dict) or "threshold"
    (dspark_schedule_threshold with ``theta``).  ``head`` "rnn" drafts with
    dspark_draft_rnn (gate weights ``Wx``, ``Ws``, ``rnn_bias`` of the input
    dict) and verifies with dspark_verify_rnn.  ``check``: synchronize, read
    (and clear) the error words of ``ws`` and ``ws_sched`` and raise
    DSparkError if any device-side error bit is set; a round with
    DSPARK_DERR_SYNC (a wait of the one-launch draft that ran out of time) has
    invalid outputs.  Not for graph capture, since it synchronizes.
    """
    if head not in ("markov", "rnn"):
        raise ValueError(f"head must be 'markov' or 'rnn', got {head!r}")
    if scheduler not in ("early", "async", "threshold"):
        raise ValueError(f"scheduler must be 'early', 'async' or 'threshold', got {scheduler!r}")
    if scheduler == "threshold" and theta is None:
        raise ValueError("scheduler='threshold' needs theta")
    d = dev_inputs
    dev = d["base"].device
    cur = torch.cuda.current_stream(dev)
    R, g, V = d["base"].shape
    L = n = None
    sched = use_scheduler and d.get("conf") is not None
    if sched and ws_sched is None:
        ws_sched = torch.zeros(256, dtype=torch.uint8, device=dev)
    beside = sched and (scheduler == "threshold" or d["conf"].numel() <= 1024)

    # every output is allocated on the current stream, which reads them after
    # the join (on the side stream the scheduler only writes into its own)
    sched_out = None
    if sched:
        sched_out = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
                     None)

    def run_scheduler():
        if scheduler == "async":
            return schedule_async(d["conf"], d["conf_lag"], d["sps"], ws_sched, out=sched_out)
        if scheduler == "threshold":
            return schedule_threshold(d["conf"], theta, ws_sched, out=sched_out)
        return schedule(d["conf"], d["sps"], ws_sched, out=sched_out)

    if sched and not beside:
        L, n, _ = run_scheduler()
    tok = torch.empty((R, g), dtype=torch.int32, device=dev)
    prob = torch.empty((R, g), dtype=torch.float32, device=dev)
    stats = torch.empty((R, g, 2), dtype=torch.float32, device=dev)
    states = None
    if head == "rnn":
        states = torch.empty((R, g, d["W1"].shape[1]), dtype=d["W1"].dtype, device=dev)
    side = _side_stream(dev)
    side.wait_stream(cur)
    if head == "rnn":
        draft_rnn(d["base"], d["W1"], d["W2"], d["Wx"], d["Ws"], d["rnn_bias"], d["anchor"], d["u_draft"],
                  temperature, ws, out=(tok, prob, stats, states))
    else:
        draft(d["base"], d["W1"], d["W2"], d["anchor"], d["u_draft"], temperature, ws, out=(tok, prob, stats))
    # side stream, beside the draft: the scheduler (when small) and the
    # target-row stream of verify (it needs only the verify lengths)
    with torch.cuda.stream(side):
        if beside:
            L, n, _ = run_scheduler()
        verify_stream(d["target"], L, temperature, ws)
    cur.wait_stream(side)
    if head == "rnn":
        ot, al, tp = verify_rnn(d["target"], d["base"], states, d["W2"], tok, prob, stats, L, d["u_accept"],
                                d["u_final"], temperature, ws, finish_only=True)
    else:
        ot, al, tp = verify(d["target"], d["base"], d["W1"], d["W2"], d["anchor"], tok, prob, stats, L,
                            d["u_accept"], d["u_final"], temperature, ws, finish_only=True)
    if check:
        bits = device_error(ws) | (device_error(ws_sched) if ws_sched is not None else 0)
        if bits:
            raise DSparkDeviceError(bits)
    return dict(draft_tokens=tok, draft_probs=prob, draft_stats=stats, verify_len=L, n_admitted=n,
                out_tokens=ot, accept_len=al, target_probs=tp, ws_sched=ws_sched, states=states)
