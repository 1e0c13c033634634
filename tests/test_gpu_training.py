"""GPU tests of the training path: semicrf_path_score through the C ABI and
the autograd loss log Z - score(gold) (semi_markov_crf_zero_amd/training.py)
against the float64 oracle (oracle.fwd_bwd minus oracle.path_score), plus a
short optimisation run whose loss must fall (technical summary of
"Streaming Structured Inference with Flash-SemiCRF", section 3: training)."""
import numpy as np
import pytest
import torch

import oracle
from semi_markov_crf_zero_amd import binding as bd
from semi_markov_crf_zero_amd.training import semicrf_log_partition, semicrf_nll
from semi_markov_crf_zero_amd.workloads import make_inputs, make_random, segment_arrays
from tests.gpu_util import DEV, TOL_GRAD, gpu_viterbi, param_excess, to_dev

pytestmark = pytest.mark.gpu


def _gold_dev(seg):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in seg.items()}


def _seg_dict(seglists, T):
    B = len(seglists)
    out = {k: np.full((B, T), -1, np.int32) for k in ("seg_start", "seg_len", "seg_label")}
    out["num_segs"] = np.zeros(B, np.int32)
    for b, segs in enumerate(seglists):
        for j, (s, k, c) in enumerate(segs):
            out["seg_start"][b, j], out["seg_len"][b, j], out["seg_label"][b, j] = s, k, c
        out["num_segs"][b] = len(segs)
    return out


def test_path_score_invalid_segmentations():
    inp = make_random(7, 8, 3, 4, seed=1, lengths=[8, 8, 8, 8, 8, 8, 9])
    bad = [
        [(0, 4, 0), (4, 3, 1)],
        [(0, 4, 0), (3, 5, 1)],
        [(0, 5, 0), (5, 3, 1)],
        [(0, 4, 3), (4, 4, 1)],
        [(1, 4, 0), (5, 3, 1)],
        [(0, 4, 0), (4, 4, 2)],   # valid
        [(0, 4, 0), (4, 4, 2)],   # length 9 > T: invalid length
    ]
    seg = _seg_dict(bad, 8)
    t = to_dev(inp)
    out = bd.semicrf_path_score(t["emissions"], t["lengths"], t["trans"], t["dur"],
                                _gold_dev(seg), want_grads=True)
    torch.cuda.synchronize()
    sc = out["score"].cpu().numpy()
    assert np.all(np.isnan(sc[[0, 1, 2, 3, 4, 6]])) and np.isfinite(sc[5])
    o = oracle.path_score(inp, seg)
    assert abs(sc[5] - o["score"][5]) <= 1e-5 * max(1.0, abs(o["score"][5]))
    gx = out["grad_emissions"].cpu().numpy()
    assert np.all(gx[[0, 1, 2, 3, 4, 6]] == 0)
    np.testing.assert_allclose(gx, o["grad_emissions"], atol=1e-6)
    np.testing.assert_allclose(out["grad_trans"].cpu().numpy(), o["grad_trans"], atol=0)
    np.testing.assert_allclose(out["grad_dur"].cpu().numpy(), o["grad_dur"], atol=0)


@pytest.mark.parametrize("name", ["tiny", "nlp"])
def test_viterbi_path_scores_best_score(name):
    inp = make_inputs(name)
    v = gpu_viterbi(inp)
    t = to_dev(inp)
    seg = {k: v[k] for k in ("seg_start", "seg_len", "seg_label", "num_segs")}
    out = bd.semicrf_path_score(t["emissions"], t["lengths"], t["trans"], t["dur"],
                                _gold_dev(seg))
    torch.cuda.synchronize()
    np.testing.assert_allclose(out["score"].cpu().numpy(), v["best_score"], rtol=2e-6)


@pytest.mark.parametrize("name", ["tiny", "nlp", "speech"])
@pytest.mark.parametrize("weighted", [False, True])
def test_nll_autograd_matches_oracle(name, weighted):
    inp = make_inputs(name)
    t = to_dev(inp)
    x = t["emissions"].clone().requires_grad_(True)
    tr = t["trans"].clone().requires_grad_(True)
    du = t["dur"].clone().requires_grad_(True)
    loss = semicrf_nll(x, t["lengths"], tr, du, _gold_dev(inp["gold"]))
    w = (np.linspace(0.25, 2.0, inp["B"]) if weighted else np.ones(inp["B"])).astype(np.float32)
    (loss * torch.from_numpy(w).to(DEV)).sum().backward()
    torch.cuda.synchronize()
    o = oracle.fwd_bwd(inp, grad_logz=w.astype(np.float64))
    p = oracle.path_score(inp, inp["gold"], weights=w)
    ref_loss = o["logz"] - p["score"]
    got = loss.detach().cpu().numpy().astype(np.float64)
    # the loss is a difference of two float32 outputs of magnitude |log Z|
    bar = 4 * np.spacing(np.abs(o["logz"]).astype(np.float32)).astype(np.float64) + 1e-5
    assert np.all(np.abs(got - ref_loss) <= bar), (got - ref_loss, bar)
    gx = x.grad.cpu().numpy().astype(np.float64)
    assert np.abs(gx - (o["grad_emissions"] - p["grad_emissions"])).max() <= 2 * TOL_GRAD
    for g, k in ((tr.grad, "grad_trans"), (du.grad, "grad_dur")):
        ref = o[k] - p[k]
        gv = g.cpu().numpy().astype(np.float64)
        # each term has the one-ulp bar of its own magnitude
        bar = (np.maximum(TOL_GRAD, np.spacing(np.abs(o[k]).astype(np.float32)))
               + np.maximum(1e-6, np.spacing(np.abs(p[k]).astype(np.float32))))
        assert np.all(np.abs(gv - ref) <= bar), (k, np.abs(gv - ref).max())


def test_log_partition_autograd():
    inp = make_inputs("nlp")
    t = to_dev(inp)
    x = t["emissions"].clone().requires_grad_(True)
    lz = semicrf_log_partition(x, t["lengths"], t["trans"], t["dur"])
    w = torch.linspace(-1.0, 1.0, inp["B"], device=DEV)
    (lz * w).sum().backward()
    o = oracle.fwd_bwd(inp, grad_logz=w.cpu().numpy().astype(np.float64))
    assert np.abs(x.grad.cpu().numpy() - o["grad_emissions"]).max() <= TOL_GRAD
    assert np.abs(lz.detach().cpu().numpy() - o["logz"]).max() <= 1e-5 * np.abs(o["logz"]).max()


def test_training_reduces_loss():
    """A linear emission model plus transition and duration scores, fitted by
    Adam on NLP-shaped synthetic data (features = noisy one-hot of the gold
    label): the training loss falls, and the Viterbi decoding of the trained
    model agrees with the gold labels on most positions."""
    B, T, C, K, F = 16, 256, 6, 12, 16
    rng = np.random.default_rng(0)
    lengths = rng.integers(T // 2, T + 1, size=B).astype(np.int32)
    paths = []
    for _ in range(B):
        lens = rng.integers(1, K + 1, size=T)
        labels = rng.integers(0, C, size=T)
        paths.append((lens, labels))
    gold = segment_arrays(paths, lengths, T)
    lab = np.zeros((B, T), np.int64)
    for b in range(B):
        for j in range(gold["num_segs"][b]):
            s, k, c = gold["seg_start"][b, j], gold["seg_len"][b, j], gold["seg_label"][b, j]
            lab[b, s:s + k] = c
    proj = rng.normal(size=(C, F))
    feats = proj[lab] + rng.normal(scale=1.5, size=(B, T, F))
    feats_t = torch.tensor(feats, dtype=torch.float32, device=DEV)
    W = torch.zeros((F, C), device=DEV, requires_grad=True)
    tr = torch.zeros((C, C), device=DEV, requires_grad=True)
    du = torch.zeros((K, C), device=DEV, requires_grad=True)
    opt = torch.optim.Adam([W, tr, du], lr=0.05)
    L_t = torch.from_numpy(lengths).to(DEV)
    g_t = _gold_dev(gold)
    losses = []
    for _ in range(40):
        opt.zero_grad()
        x = (feats_t @ W).contiguous()
        loss = semicrf_nll(x, L_t, tr, du, g_t).sum() / float(lengths.sum())
        loss.backward()
        opt.step()
        losses.append(float(loss))
    print("loss per position", losses[0], "->", losses[-1])
    assert losses[-1] < 0.6 * losses[0]
    assert all(np.isfinite(losses))
    with torch.no_grad():
        x = (feats_t @ W).contiguous()
        v = bd.semicrf_viterbi(x, L_t, tr.detach().contiguous(), du.detach().contiguous())
    torch.cuda.synchronize()
    agree = total = 0
    for b in range(B):
        pred = np.zeros(T, np.int64)
        n = int(v["num_segs"][b])
        for j in range(n):
            s, k, c = (int(v["seg_start"][b, j]), int(v["seg_len"][b, j]),
                       int(v["seg_label"][b, j]))
            pred[s:s + k] = c
        agree += int((pred[:lengths[b]] == lab[b, :lengths[b]]).sum())
        total += int(lengths[b])
    print("label accuracy", agree / total)
    assert agree / total > 0.8
