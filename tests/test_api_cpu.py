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
    for code in range(8):
        assert len(bd.status_string(code)) >= 2
    assert bd.status_string(99) == "unknown status"


def test_default_checkpoint_interval(lib):
    assert bd.semicrf_default_checkpoint_interval(131072, 512) == 8192
    assert bd.semicrf_default_checkpoint_interval(1048576, 256) == 16384
    assert bd.semicrf_default_checkpoint_interval(4096, 64) == 512
    assert bd.semicrf_default_checkpoint_interval(256, 16) == 64
    assert bd.semicrf_default_checkpoint_interval(3, 100) == 3  # capped at T


def test_checkpoint_interval_fills_the_sweep(lib):
    # halved from ceil(sqrt(T*K)) while 2*B*ceil(T/interval) is below the
    # workgroups the GPU runs at once (512 for the C <= 32 engine while two of
    # its workgroups fit a compute unit's LDS and registers, else 256), not
    # below max(2K, 32)
    ci = bd.semicrf_checkpoint_interval
    assert ci(4, 131072, 16, 512) == 2048     # genome: 512 windowed workgroups
    assert ci(4, 131072, 16, 1024) == 2897    # LDS-ring engine: 256 workgroups
    assert ci(1, 1048576, 64, 256) == 8192    # extreme: 256
    assert ci(16, 4096, 256, 64) == 512       # speech: 256 already
    assert ci(32, 512, 24, 32) == 128         # nlp: 256 already (C > 16: one per unit)
    assert ci(32, 512, 16, 32) == 64          # C <= 16: 512 windowed workgroups
    assert ci(4, 256, 8, 16) == 32            # tiny: floor 2K = 32
    assert ci(64, 100000, 8, 8) == 895        # already >= 512 workgroups
    assert ci(1, 3, 4, 100) == 3              # capped at T
    assert ci(0, 10, 4, 4) == 0
    assert ci(1, 10, 0, 4) == 0
    for B, T, C, K in ((4, 131072, 16, 512), (1, 1048576, 64, 256), (2, 777, 3, 5),
                       (3, 50, 40, 80)):
        d = ci(B, T, C, K)
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
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 8, 0, ctypes.byref(n)) == 6
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 0, -1, ctypes.byref(n)) == 6
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 0, 0, None) == 1
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 1, 7, ctypes.byref(n)) == 0
    small = n.value
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 1, 50, ctypes.byref(n)) == 0
    assert n.value != small  # the checkpoint count and chunk scratch depend on the interval


def test_float64_flag_selects_the_float64_sweep(lib):
    # 64 < C <= 256, K <= 64 runs the float32-ring sweep by default; the flag
    # moves it to the float64 LDS-ring sweep, whose 1024-thread instance
    # streams a float32 exp(trans) table from the workspace (larger workspace)
    n32, n64, m = ctypes.c_size_t(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    for op in (bd.OP_LOGZ, bd.OP_FWD_BWD):
        assert lib.semicrf_workspace_size(op, 2, 300, 256, 64, 0, 0, ctypes.byref(n32)) == 0
        assert lib.semicrf_workspace_size(op, 2, 300, 256, 64, bd.FLOAT64, 0,
                                          ctypes.byref(n64)) == 0
        assert n64.value > n32.value
        # shapes outside the float32 sweep: the flag changes nothing
        assert lib.semicrf_workspace_size(op, 2, 300, 64, 64, 0, 0, ctypes.byref(n32)) == 0
        assert lib.semicrf_workspace_size(op, 2, 300, 64, 64, bd.FLOAT64, 0, ctypes.byref(m)) == 0
        assert m.value == n32.value


def test_low_memory_viterbi_workspace(lib):
    # the whole decoder keeps decisions and predecessor words for every
    # position (8 bytes per position and label); the low-memory decoder keeps
    # one window of chunks.  extreme: B=1, T=2^20, C=64, K=256
    full, low = ctypes.c_size_t(0), ctypes.c_size_t(0)
    args = (bd.OP_VITERBI, 1, 1 << 20, 64, 256)
    assert lib.semicrf_workspace_size(*args, 0, 0, ctypes.byref(full)) == 0
    assert lib.semicrf_workspace_size(*args, bd.LOW_MEMORY, 0, ctypes.byref(low)) == 0
    S = 8 * ((1 << 20) + 1) * 64
    assert full.value - S > 8 * (1 << 20) * 64  # beyond the scores: decisions of every position
    # a window of ceil(sqrt(64)) + 1 = 9 of the 64 chunks, plus the window's
    # segment lists
    assert low.value - S < 0.2 * (full.value - S)


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
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 8, 0, None, P, P, P, P, None, P,
                               1 << 30, None) == 6
    assert lib.semicrf_fwd_bwd(P, P, P, P, 2, 10, 4, 4, 0, -3, None, P, P, P, P, None, P,
                               1 << 30, None) == 6
    assert lib.semicrf_logz_fwd(P, P, P, P, -1, 10, 4, 4, 0, P, P, 1 << 30, None) == 2


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2)
    with pytest.raises(ValueError):
        bd.semicrf_logz_fwd(x, torch.ones(1, dtype=torch.int32), torch.zeros(2, 2), torch.zeros(3, 2))


def test_weight_vectors_must_be_contiguous():
    """grad_logz / weights are read as contiguous [B] float32 memory: a
    strided view (w[::2]) would silently weight the wrong sequences."""
    import torch
    dev = torch.device("cpu")
    bd._check_weights("grad_logz", None, 3, dev)
    bd._check_weights("grad_logz", torch.ones(3), 3, dev)
    with pytest.raises(ValueError):
        bd._check_weights("grad_logz", torch.ones(6)[::2], 3, dev)
    with pytest.raises(ValueError):
        bd._check_weights("grad_logz", torch.ones(3, dtype=torch.float64), 3, dev)
    with pytest.raises(ValueError):
        bd._check_weights("weights", torch.ones(4), 3, dev)


def test_fwd_bwd_ex_and_path_score_validate_before_launch(lib):
    P = FAKE
    need = bd.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 10, 4, 4)
    # fwd_bwd_ex: boundary and phase events optional; the rest as fwd_bwd
    assert lib.semicrf_fwd_bwd_ex(P, P, P, P, 2, 10, 4, 4, 0, 0, None, P, P, P, None, None, None,
                                  P, need, None, None) == 1
    assert lib.semicrf_fwd_bwd_ex(P, P, P, P, 2, 10, 4, 4, 0, 0, None, P, P, P, P, None, None,
                                  P, need - 1, None, None) == 4
    assert lib.semicrf_fwd_bwd_ex(P, P, P, P, 2, 10, 300, 4, 0, 0, None, P, P, P, P, None, P,
                                  P, need, None, None) == 3
    # path score: inputs, segments and score required; gradients optional
    need = bd.semicrf_workspace_size(bd.OP_PATH_SCORE, 2, 10, 4, 4)
    assert need > 0
    base = [P, P, P, P, 2, 10, 4, 4, 0, P, P, P, P, None, P, None, None, None, P, need, None]
    for idx in (0, 1, 2, 3, 9, 10, 11, 12, 14):
        args = list(base)
        args[idx] = None
        assert lib.semicrf_path_score(*args) == 1
    args = list(base)
    args[19] = need - 1
    assert lib.semicrf_path_score(*args) == 4
    args = list(base)
    args[8] = 8  # unknown flag
    assert lib.semicrf_path_score(*args) == 6
    args = list(base)
    args[4] = 0
    assert lib.semicrf_path_score(*args) == 2


def test_low_memory_workspace_is_sublinear(lib):
    """SEMICRF_LOW_MEMORY keeps checkpoint records and one window of rows:
    beyond the cumulative scores (8 bytes per position and label) its
    workspace grows more slowly than T, while the default keeps per-position
    rows."""
    C, K = 64, 256

    def beyond_scores(T, flags):
        n = bd.semicrf_workspace_size(bd.OP_FWD_BWD, 1, T, C, K, flags)
        return n - (T + 1) * C * 8

    for T in (1 << 16, 1 << 18, 1 << 20):
        assert beyond_scores(T, bd.LOW_MEMORY) < beyond_scores(T, 0) / 2
    assert beyond_scores(1 << 20, bd.LOW_MEMORY) < beyond_scores(1 << 20, 0) / 6
    # 16x the positions: ~T^(3/4) (8x) for the windows, ~T for the rows
    g_low = beyond_scores(1 << 20, bd.LOW_MEMORY) / beyond_scores(1 << 16, bd.LOW_MEMORY)
    g_all = beyond_scores(1 << 20, 0) / beyond_scores(1 << 16, 0)
    assert g_all > 8 and g_low < 6, (g_all, g_low)
    n = ctypes.c_size_t(0)
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 3, 0, ctypes.byref(n)) == 0
    assert lib.semicrf_workspace_size(bd.OP_FWD_BWD, 2, 100, 4, 8, 8, 0, ctypes.byref(n)) == 6
