"""GPU parity of the eight-wave sweep engine (32 < C <= 64, K <= 256): each
wave owns 32 durations of every label, so the shapes below put K at the
edges of that split (K = 1, 31, 32, 33, 64, 255, 256), the ring's wrap at
every offset (T not a multiple of K, K > T), checkpoint intervals that start
with a burn-in, frequent rebases (emission scale 30), the row flushes every
8 steps (lengths of every residue mod 8), low-memory replay windows and the
log Z-only operation -- every element against the float64 oracle.
"""
import numpy as np
import pytest

import oracle
from semi_markov_crf_zero_amd.workloads import make_random
from tests.gpu_util import assert_fwd_bwd_close, gpu_fwd_bwd, gpu_logz, logz_rel_err

pytestmark = pytest.mark.gpu

# (B, T, C, K, lengths, interval)
SHAPES = [
    (3, 500, 64, 1, [500, 499, 2], 0),           # K = 1: wave 0's newest term only
    (2, 400, 33, 31, [400, 271], 0),             # K < 32, C = 33
    (2, 420, 64, 32, [420, 419], 96),            # wave 0 full, the others idle
    (2, 410, 40, 33, [410, 333], 0),             # wave 1 holds one duration
    (2, 700, 48, 64, [700, 517], 512),           # two waves, an interval with a burn-in
    (2, 900, 64, 255, [900, 641], 512),          # 8 waves, the last one short
    (2, 1100, 64, 256, [1100, 1093], 0),         # K = 256, the largest ring
    (1, 4500, 64, 256, [4400], 2048),            # K = 256 with burn-in intervals
    (2, 200, 64, 256, [200, 37], 0),             # K > T
    (4, 300, 57, 100, [300, 298, 297, 1], 0),    # lengths of several residues mod 8, L = 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dT%dC%dK%d" % s[:4])
def test_sweep64_shapes(shape):
    B, T, C, K, lengths, ckpt = shape
    inp = make_random(B, T, C, K, seed=7 * T + C + K, lengths=lengths, tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    errs = assert_fwd_bwd_close(gpu_fwd_bwd(inp, ckpt=ckpt), o, label=shape[:4])
    print(shape[:4], errs)
    lz = gpu_logz(inp)
    assert logz_rel_err(lz, oracle.logz(inp)).max() <= 1e-5


@pytest.mark.parametrize("K,ckpt", [(40, 320), (256, 300)])
def test_sweep64_rebases_and_burn_in(K, ckpt):
    """Emission scale 30: labels rebase on most steps, also on the burn-in's
    last step (which stores the interval's start record; intervals of 8K
    positions or more) and on interval ends."""
    inp = make_random(2, 1500, 64, K, seed=31 + K, sigma=30.0, tsd=1.0, dsd=1.0,
                      lengths=[1500, 1207])
    o = oracle.fwd_bwd(inp)
    for ckpt in (0, ckpt):
        assert_fwd_bwd_close(gpu_fwd_bwd(inp, ckpt=ckpt), o, label=(K, ckpt))


def test_sweep64_low_memory_windows():
    """Replay windows (start rows from records, rows window-relative)."""
    inp = make_random(2, 3000, 64, 120, seed=5, lengths=[3000, 2222], tsd=0.3, dsd=0.3)
    o = oracle.fwd_bwd(inp)
    g = gpu_fwd_bwd(inp, ckpt=200, low_memory=True)
    assert_fwd_bwd_close(g, o, label="lowmem")
    f = gpu_fwd_bwd(inp, ckpt=200)
    for k in ("grad_emissions", "marginals", "boundary"):
        assert np.abs(g[k] - f[k]).max() <= 1e-5, k
