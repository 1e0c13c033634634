"""GPU parity of the float32-ring sweep engine (64 < C <= 256, K <= 64): a
lane pair per label, each lane holding 32 durations, so the shapes below put
K at the edges of that split (K = 1, 31, 32, 33, 64), C at the edges of the
wave slices (65, 96, 129, 200, 256: waves with some, all or no real labels),
the ring's wrap at every offset (T not a multiple of K, K > T), intervals
that start with a burn-in, frequent rebases (emission scale 30), replay
windows and the log Z-only operation -- every element against the float64
oracle, and the same calls with SEMICRF_FLOAT64 (the float64 engine) next to
it.
"""
import numpy as np
import pytest

import oracle
from semi_markov_crf_zero_amd.workloads import make_random
from tests.gpu_util import assert_fwd_bwd_close, gpu_fwd_bwd, gpu_logz, logz_rel_err

pytestmark = pytest.mark.gpu

# (B, T, C, K, lengths, interval)
SHAPES = [
    (3, 500, 65, 1, [500, 499, 2], 0),           # K = 1: lane 0's newest term only; C = 65
    (2, 400, 96, 31, [400, 271], 0),             # K < 32: lane 1 idle
    (2, 420, 129, 32, [420, 419], 96),           # lane 0 full
    (2, 410, 200, 33, [410, 333], 0),            # lane 1 holds one duration
    (2, 700, 256, 64, [700, 517], 512),          # K = 64, an interval with a burn-in
    (2, 200, 256, 64, [200, 37], 0),             # K > L
    (4, 300, 160, 50, [300, 298, 297, 1], 0),    # several residues of the ring, L = 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_sweep256_shapes(shape):
    B, T, C, K, lengths, ckpt = shape
    inp = make_random(B, T, C, K, seed=11 * T + C + K, lengths=lengths, tsd=0.3, dsd=0.3)
    print("case", shape[:4], flush=True)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=ckpt)
    errs = assert_fwd_bwd_close(g, o, label=shape[:4])
    print(shape[:4], errs)
    f = gpu_fwd_bwd(inp, ckpt=ckpt, float64=True)
    assert_fwd_bwd_close(f, o, label=(shape[:4], "float64"))
    lz = gpu_logz(inp)
    assert logz_rel_err(lz, oracle.logz(inp)).max() <= 1e-5


@pytest.mark.parametrize("K,ckpt", [(40, 320), (64, 600)])
def test_sweep256_rebases_and_burn_in(K, ckpt):
    """Emission scale 30: labels rebase on most steps, also on the burn-in's
    last step and on interval ends."""
    inp = make_random(2, 1500, 256, K, seed=41 + K, sigma=30.0, tsd=1.0, dsd=1.0,
                      lengths=[1500, 1207])
    print("case rebases", K, ckpt, flush=True)
    o = oracle.fwd_bwd(inp)
    for c in (0, ckpt):
        assert_fwd_bwd_close(gpu_fwd_bwd(inp, ckpt=c), o, label=(K, c))


def test_sweep256_low_memory_windows():
    """Replay windows (start rows from records, rows window-relative)."""
    inp = make_random(2, 3000, 192, 60, seed=9, lengths=[3000, 2222], tsd=0.3, dsd=0.3)
    print("case lowmem", flush=True)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=200, low_memory=True)
    assert_fwd_bwd_close(g, o, label="lowmem")
    f = gpu_fwd_bwd(inp, ckpt=200)
    for k in ("grad_emissions", "marginals", "boundary"):
        assert np.abs(g[k] - f[k]).max() <= 1e-5, k
