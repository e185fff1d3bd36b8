"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspace, and rejects bad arguments on the host
before launching anything."""

import ctypes
import os
import re

import pytest

import draft_sampling_verify_markov_amd as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dspark_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return D.load_library()


def test_header_declares_the_round(lib):
    names = _declared_functions()
    for n in ("dspark_draft", "dspark_schedule", "dspark_verify", "dspark_workspace_size",
              "dspark_workspace_init", "dspark_device_error", "dspark_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_workspace_size_limits(lib):
    assert D.workspace_size(128, 7, 131072, 256) > 0
    assert lib.dspark_workspace_size(4, 4, 500, 16) == 0      # V % 8 != 0
    assert lib.dspark_workspace_size(4, 17, 512, 16) == 0     # gamma > 16
    assert lib.dspark_workspace_size(4, 4, 512, 24) == 0      # r % 16 != 0
    assert lib.dspark_workspace_size(4, 4, 512, 272) == 0     # r > 256
    assert lib.dspark_workspace_size(0, 4, 512, 16) == 0      # R < 1
    # grows with every size
    a = D.workspace_size(4, 4, 512, 16)
    assert D.workspace_size(8, 4, 512, 16) > a
    assert D.workspace_size(4, 8, 512, 16) > a
    assert D.workspace_size(4, 4, 8192, 16) > a


EINVAL, ENOSPC = -1, -2


def _draft(lib, **kw):
    a = dict(base=16, W1=16, W2=16, wt=0, anchor=16, u=16, R=4, g=4, V=512, r=16, T=1.0,
             tok=16, prob=16, stats=16, ws=256, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.dspark_draft(a["base"], a["W1"], a["W2"], a["wt"], a["anchor"], a["u"], a["R"], a["g"],
                            a["V"], a["r"], a["T"], a["tok"], a["prob"], a["stats"], a["ws"], a["wsb"],
                            a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(base=None), EINVAL), (dict(W2=None), EINVAL), (dict(tok=None), EINVAL),
    (dict(V=500), EINVAL), (dict(g=0), EINVAL), (dict(g=17), EINVAL), (dict(r=8), EINVAL),
    (dict(R=0), EINVAL), (dict(T=-1.0), EINVAL), (dict(T=float("nan")), EINVAL),
    (dict(T=float("inf")), EINVAL), (dict(wt=7), EINVAL), (dict(base=18), EINVAL),
    (dict(ws=None), EINVAL), (dict(ws=128), EINVAL), (dict(wsb=100), ENOSPC),
])
def test_draft_rejects_bad_arguments(lib, kw, status):
    assert _draft(lib, **kw) == status


def test_schedule_rejects_bad_arguments(lib):
    f = lib.dspark_schedule
    assert f(None, 16, 4, 4, 10, 16, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 16, 1000, 9, 10, 16, 16, None, 256, 4096, None) == EINVAL   # pool > 8192
    assert f(16, 16, 4, 4, 0, 16, 16, None, 256, 4096, None) == EINVAL       # empty table
    assert f(16, 16, 4, 0, 10, 16, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 16, 4, 4, 10, None, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 16, 4, 4, 10, 16, 16, None, 256, 100, None) == ENOSPC


def test_schedule_async_rejects_bad_arguments(lib):
    f = lib.dspark_schedule_async
    assert f(None, 16, 16, 4, 4, 10, 16, 16, None, 256, 4096, None) == EINVAL
    assert f(16, None, 16, 4, 4, 10, 16, 16, None, 256, 4096, None) == EINVAL    # no lagged pool
    assert f(16, 16, 16, 1000, 9, 10, 16, 16, None, 256, 4096, None) == EINVAL   # pool > 8192
    assert f(16, 16, 16, 4, 4, 0, 16, 16, None, 256, 4096, None) == EINVAL       # empty table
    assert f(16, 16, 16, 4, 4, 10, None, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 16, 16, 4, 4, 10, 16, 16, None, 250, 4096, None) == EINVAL      # misaligned workspace
    assert f(16, 16, 16, 4, 4, 10, 16, 16, None, 256, 100, None) == ENOSPC


def test_schedule_threshold_rejects_bad_arguments(lib):
    f = lib.dspark_schedule_threshold
    assert f(None, 0.5, 4, 4, 16, 16, None, 256, 4096, None) == EINVAL
    assert f(16, float("nan"), 4, 4, 16, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 0.5, 1000, 9, 16, 16, None, 256, 4096, None) == EINVAL      # pool > 8192
    assert f(16, 0.5, 4, 4, None, 16, None, 256, 4096, None) == EINVAL
    assert f(16, 0.5, 4, 4, 16, 16, None, 256, 100, None) == ENOSPC


def test_accept_rates_rejects_bad_arguments(lib):
    good = [16, 16, 16, 16, 0, 16, 16, 16, 4, 4, 512, 16, 1.0, 16, 256, 1 << 24, None]
    bad = list(good); bad[12] = 0.0
    assert lib.dspark_accept_rates(*bad) == EINVAL                      # greedy has no label
    bad = list(good); bad[12] = float("inf")
    assert lib.dspark_accept_rates(*bad) == EINVAL
    bad = list(good); bad[4] = 7
    assert lib.dspark_accept_rates(*bad) == EINVAL                      # unknown weight type
    bad = list(good); bad[7] = None
    assert lib.dspark_accept_rates(*bad) == EINVAL                      # no draft statistics
    bad = list(good); bad[11] = 24
    assert lib.dspark_accept_rates(*bad) == EINVAL                      # r % 16 != 0
    bad = list(good); bad[15] = 1024
    assert lib.dspark_accept_rates(*bad) == ENOSPC


def test_rnn_entry_points_reject_bad_arguments(lib):
    need = lib.dspark_workspace_size(4, 4, 512, 16)
    # base W1 W2 Wx Ws bias wt anchor u R g V r T tok prob stats states ws wsb stream
    good = [16, 16, 16, 16, 16, 16, 0, 16, 16, 4, 4, 512, 16, 1.0, 16, 16, 16, 16, 256, need, None]
    f = lib.dspark_draft_rnn
    for i in (0, 1, 2, 3, 4, 5, 7, 8, 14, 15, 16, 17):
        bad = list(good); bad[i] = None
        assert f(*bad) == EINVAL, i
    for i, v in ((6, 7), (9, 0), (10, 17), (11, 500), (12, 24), (13, -1.0), (17, 18)):
        bad = list(good); bad[i] = v
        assert f(*bad) == EINVAL, i
    bad = list(good); bad[19] = need - 1
    assert f(*bad) == ENOSPC
    # target base states W2 wt tok prob stats L ua uf R g V r T out acc tp ws wsb stream
    vg = [16, 16, 16, 16, 0, 16, 16, 16, None, 16, 16, 4, 4, 512, 16, 1.0, 16, 16, None, 256, need, None]
    v = lib.dspark_verify_rnn
    for i in (0, 1, 2, 3, 5, 6, 7, 9, 10, 16, 17):
        bad = list(vg); bad[i] = None
        assert v(*bad) == EINVAL, i
    for i, val in ((4, 9), (12, 0), (13, 12), (15, float("nan")), (2, 20)):
        bad = list(vg); bad[i] = val
        assert v(*bad) == EINVAL, i
    bad = list(vg); bad[20] = 1000
    assert v(*bad) == ENOSPC


def test_split_verify_rejects_bad_arguments(lib):
    need = lib.dspark_workspace_size(4, 4, 512, 16)
    f = lib.dspark_verify_stream
    good = [16, None, 4, 4, 512, 1.0, 256, need, None]
    for i, v in ((0, None), (0, 18), (2, 0), (3, 17), (4, 500), (5, -1.0), (5, float("inf")), (6, None),
                 (6, 128)):
        bad = list(good); bad[i] = v
        assert f(*bad) == EINVAL, i
    bad = list(good); bad[7] = need - 1
    assert f(*bad) == ENOSPC
    assert lib.dspark_verify_finish(None, 16, 16, 16, 0, 16, 16, 16, 16, None, 16, 16, 4, 4, 512, 16, 1.0, 16, 16,
                                    None, 256, need, None) == EINVAL
    assert lib.dspark_verify_rnn_finish(16, 16, None, 16, 0, 16, 16, 16, None, 16, 16, 4, 4, 512, 16, 1.0, 16, 16,
                                        None, 256, need, None) == EINVAL


def test_sts_workspace_and_argument_checks(lib):
    sz = lib.dspark_sts_workspace_size
    assert sz(65536, 7, 256, 15) >= 256 + 2 * 8 * 65536 + 7 * 256 * 8 + 64 * 256 * 15 * 8
    assert sz(1, 1, 1, 1) > 0 and sz(1 << 21, 16, 1024, 64) > 0
    for bad in ((0, 7, 8, 15), ((1 << 21) + 1, 7, 8, 15), (10, 0, 8, 15), (10, 17, 8, 15), (10, 7, 0, 15),
                (10, 7, 1025, 15), (10, 7, 8, 0), (10, 7, 8, 65)):
        assert sz(*bad) == 0, bad
    f = lib.dspark_sts_fit
    need = sz(100, 4, 8, 10)
    good = [16, 16, 16, 100, 4, 8, 10, 16, None, 16, None, 256, need, None]
    for i in (0, 1, 2, 7, 9):                                           # required pointers
        bad = list(good); bad[i] = None
        assert f(*bad) == EINVAL, i
    for i, v in ((3, 0), (4, 17), (5, 0), (6, 65)):
        bad = list(good); bad[i] = v
        assert f(*bad) == EINVAL, i
    bad = list(good); bad[11] = 128                                     # unaligned workspace
    assert f(*bad) == EINVAL
    bad = list(good); bad[12] = need - 1
    assert f(*bad) == ENOSPC
    a = lib.dspark_sts_apply
    assert a(None, 16, 4, 4, 16, 256, 256, None) == EINVAL
    assert a(16, 16, 4, 0, 16, 256, 256, None) == EINVAL
    assert a(16, 16, 4, 4, None, 256, 256, None) == EINVAL
    assert a(16, 16, 4, 4, 16, 256, 255, None) == ENOSPC


def test_verify_rejects_bad_arguments(lib):
    base = [16, 16, 16, 16, 0, 16, 16, 16, 16, None, 16, 16, 4, 4, 512, 16, 1.0, 16, 16, None, 256,
            1 << 20, None]
    bad = list(base)
    bad[0] = None
    assert lib.dspark_verify(*bad) == EINVAL
    bad = list(base)
    bad[14] = 100
    assert lib.dspark_verify(*bad) == EINVAL
    bad = list(base)
    bad[21] = 64
    assert lib.dspark_verify(*bad) == ENOSPC


def test_profile_hook_arguments(lib):
    # arming only stores the caller's event arrays; nothing is recorded until a launch
    arr = (ctypes.c_void_p * 4)(1, 2, 3, 4)
    EINVAL = -1
    assert lib.dspark_profile_arm(0, arr, arr, 4, 1) == EINVAL          # unknown kernel id
    assert lib.dspark_profile_arm(10, arr, arr, 4, 1) == EINVAL
    assert lib.dspark_profile_arm(8, arr, arr, 4, 1) == 0              # one-launch draft
    assert lib.dspark_profile_disarm() == 0
    assert lib.dspark_profile_arm(9, arr, arr, 4, 1) == 0              # one workgroup per request
    assert lib.dspark_profile_disarm() == 0
    assert lib.dspark_profile_arm(1, None, arr, 4, 1) == EINVAL         # NULL arrays
    assert lib.dspark_profile_arm(1, arr, None, 4, 1) == EINVAL
    assert lib.dspark_profile_arm(1, arr, arr, 0, 1) == EINVAL          # no pairs
    assert lib.dspark_profile_arm(1, arr, arr, 4, 0) == EINVAL          # repeat out of range
    assert lib.dspark_profile_arm(1, arr, arr, 4, 1001) == EINVAL
    assert lib.dspark_profile_arm(1, arr, arr, 4, 8) == 0
    assert lib.dspark_profile_disarm() == 0


def test_status_strings(lib):
    assert b"ENOSPC" in lib.dspark_status_string(-2)
    assert b"EINVAL" in lib.dspark_status_string(-1)
    assert b"EHIP" in lib.dspark_status_string(-3)


def test_binding_checks_tensors():
    import torch
    with pytest.raises(TypeError):
        D.draft(torch.zeros(2, 2, 8), torch.zeros(8, 16, dtype=torch.float64),
                torch.zeros(16, 8, dtype=torch.float64), None, None, 1.0, None)


def _draft_noalloc(lib, **kw):
    a = dict(base=16, W1=16, W2=16, wt=0, anchor=16, u=16, R=4, g=4, V=512, r=16, T=1.0,
             tok=16, prob=16, stats=16, err=16, stream=None)
    a.update(kw)
    return lib.dspark_draft_noalloc(a["base"], a["W1"], a["W2"], a["wt"], a["anchor"], a["u"], a["R"], a["g"],
                                    a["V"], a["r"], a["T"], a["tok"], a["prob"], a["stats"], a["err"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(base=None), EINVAL), (dict(err=None), EINVAL), (dict(V=500), EINVAL), (dict(g=17), EINVAL),
    (dict(T=-1.0), EINVAL), (dict(wt=7), EINVAL), (dict(W1=18), EINVAL),
    # the static scratch holds 8448 + 32 R ceil(V / 256) bytes at most
    (dict(R=1025, V=131072), ENOSPC), (dict(R=4097, V=32768), ENOSPC),
])
def test_draft_noalloc_rejects_bad_arguments_and_oversized_calls(lib, kw, status):
    """Checked on the host before the scratch array is touched."""
    assert _draft_noalloc(lib, **kw) == status


def test_device_error_names_its_bits():
    e = D.DSparkDeviceError(128 | 8)
    assert isinstance(e, D.DSparkError) and e.bits == 136
    assert "SYNC" in str(e) and "TOKEN" in str(e) and "NONFINITE" not in str(e)
