"""Host-side checks of the C ABI (no GPU needed).

* libsemicrf.so loads and exports every function include/semicrf.h declares;
* semicrf_workspace_size and every entry point reject invalid arguments with
  the documented status BEFORE any launch (so these calls never touch a
  device: NULL pointers, bad sizes, unsupported C/K, bad flags or checkpoint
  interval, a workspace that is too small).
"""
import ctypes
import os
import re

import pytest

from semi_markov_crf_zero_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "semicrf.h")


@pytest.fixture(scope="module")
def lib():
    return bd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(semicrf_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd.EXPORTS)


def test_status_strings(lib):
    for code in range(7):
        assert len(bd.status_string(code)) >= 2
    assert bd.status_string(99) == "unknown status"


def test_default_checkpoint_interval(lib):
    assert bd.semicrf_default_checkpoint_interval(131072, 512) == 8192
    assert bd.semicrf_default_checkpoint_interval(1048576, 256) == 16384
    assert bd.semicrf_default_checkpoint_interval(4096, 64) == 512
    assert bd.semicrf_default_checkpoint_interval(256, 16) == 64
    assert bd.semicrf_default_checkpoint_interval(3, 100) == 3  # capped at T


def test_checkpoint_interval_fills_the_sweep(lib):
    # halved from ceil(sqrt(T*K)) while 2*B*ceil(T/interval) < 256, not below max(2K, 32)
    assert bd.semicrf_checkpoint_interval(4, 131072, 512) == 4096    # genome: 256 workgroups
    assert bd.semicrf_checkpoint_interval(1, 1048576, 256) == 8192   # extreme: 256
    assert bd.semicrf_checkpoint_interval(16, 4096, 64) == 512       # speech: 256 already
    assert bd.semicrf_checkpoint_interval(32, 512, 32) == 128        # nlp: 256 already
    assert bd.semicrf_checkpoint_interval(4, 256, 16) == 32          # tiny: floor 2K = 32
    assert bd.semicrf_checkpoint_interval(64, 100000, 8) == 895      # already >= 512 workgroups
    assert bd.semicrf_checkpoint_interval(1, 3, 100) == 3            # capped at T
    assert bd.semicrf_checkpoint_interval(0, 10, 4) == 0
    for B, T, K in ((4, 131072, 512), (1, 1048576, 256), (2, 777, 5), (3, 50, 80)):
        d = bd.semicrf_checkpoint_interval(B, T, K)
        assert 1 <= d <= bd.semicrf_default_checkpoint_interval(T, K)


@pytest.mark.parametrize("args,code", [
    ((bd.OP_FWD_BWD, 0, 10, 4, 4), 2),
    ((bd.OP_FWD_BWD, 1, 0, 4, 4), 2),
    ((bd.OP_FWD_BWD, 1, 10, 0, 4), 2),
    ((bd.OP_FWD_BWD, 1, 10, 4, 0), 2),
    ((bd.OP_FWD_BWD, 1, 10, 257, 4), 3),
    ((bd.OP_FWD_BWD, 1, 10, 64, 257), 3),   # K*C > 16384
    ((bd.OP_FWD_BWD, 1, 10, 256, 65), 3),   # K > 32*floor(512/C)
    ((bd.OP_VITERBI, 1, 10, 16, 1025), 3),
    ((7, 1, 10, 4, 4), 6),
    ((bd.OP_FWD_BWD, 40000, 40000, 2, 4), 2),  # B*(T+1)*C >= 2^31
])
def test_workspace_size_errors(lib, args, code):
    n = ctypes.c_size_t(0)
    assert lib.semicrf_workspace_size(*args, 0, 0, ctypes.byref(n)) == code


def test_workspace_size_flags_and_interval(lib):
    n = ctypes.c_size_t(0)
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 2, 0, ctypes.byref(n)) == 6
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 0, -1, ctypes.byref(n)) == 6
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 0, 0, None) == 1
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 1, 7, ctypes.byref(n)) == 0
    small = n.value
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 1, 50, ctypes.byref(n)) == 0
    assert n.value != small  # the checkpoint count and chunk scratch depend on the interval


def test_supported_workloads_have_a_configuration(lib):
    from semi_markov_crf_zero_amd.workloads import WORKLOADS
    for w in WORKLOADS.values():
        for op in (bd.OP_SCAN, bd.OP_LOGZ, bd.OP_FWD_BWD, bd.OP_VITERBI):
            assert bd.semicrf_workspace_size(op, w.B, w.T, w.C, w.K) > 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def test_null_pointers_rejected_before_launch(lib):
    P = FAKE
    # fwd_bwd: each required pointer NULL in turn
    base = [P, P, P, P, 2, 10, 4, 4, 0, 0, None, P, P, P, P, None, P, 1 << 30, None]
    for idx in (0, 1, 2, 3, 11, 12, 13, 14):
        args = list(base)
        args[idx] = None
        assert lib.semicrf_fwd_bwd(*args) == 1
    assert lib.semicrf_logz_fwd(None, P, P, P, 2, 10, 4, 4, 0, P, P, 1 << 30, None) == 1
    assert lib.semicrf_viterbi(P, P, P, P, 2, 10, 4, 4, 0, P, P, P, None, P, P, 1 << 30, None) == 1
    assert lib.semicrf_cumulative_scores(P, P, 2, 10, 4, 0, None, P, P, 1 << 30, None) == 1


def test_small_workspace_rejected_before_launch(lib):
    P = FAKE
    need = bd.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 10, 4, 4)
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 0, 0, None, P, P, P, P, None, P,
                               need - 1, None) == 4
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 0, 0, None, P, P, P, P, None, None,
                               need, None) == 4
    need = bd.semicrf_workspace_size(bd.OP_LOGZ, 2, 10, 4, 4)
    assert lib.semicrf_logz_fwd(P, P, P, P, 2, 10, 4, 4, 0, P, P, need - 1, None) == 4
    need = bd.semicrf_workspace_size(bd.OP_VITERBI, 2, 10, 4, 4)
    assert lib.semicrf_viterbi(P, P, P, P, 2, 10, 4, 4, 0, P, P, P, P, P, P, need - 1, None) == 4
    need = bd.semicrf_workspace_size(bd.OP_SCAN, 2, 10, 4, 1)
    assert lib.semicrf_cumulative_scores(P, P, 2, 10, 4, 0, P, P, P, need - 1, None) == 4


def test_bad_sizes_rejected_before_launch(lib):
    P = FAKE
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 300, 4, 0, 0, None, P, P, P, P, None, P,
                               1 << 30, None) == 3
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 4, 0, None, P, P, P, P, None, P,
                               1 << 30, None) == 6
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 0, -3, None, P, P, P, P, None, P,
                               1 << 30, None) == 6
    assert lib.semicrf_logz_fwd(P, P, P, P, -1, 10, 4, 4, 0, P, P, 1 << 30, None) == 2


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        bd.semicrf_logz_fwd(x, torch.ones(1, dtype=torch.int32), torch.zeros(2, 2), torch.zeros(3, 2))
