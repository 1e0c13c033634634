"""ctypes binding of libsemicrf.so (the C ABI in include/semicrf.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of the library.  Functions carry the C names; tensors must be CUDA
(HIP) tensors, contiguous, float32 (emissions, trans, dur, grad_logz) and
int32 (lengths).  Outputs and the workspace are allocated with torch on the
input's device and the work is enqueued on torch's current stream.

If the library has not been built this module raises at the first call;
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsemicrf.so")

OP_SCAN, OP_LOGZ, OP_FWD_BWD, OP_VITERBI, OP_PATH_SCORE = 0, 1, 2, 3, 4
NO_CENTER = 1
LOW_MEMORY = 2  # fwd_bwd / viterbi: checkpoint records only, replayed in windows
FLOAT64 = 4  # logz_fwd / fwd_bwd: float64 sweeps for 64 < C <= 256, K <= 64 as well

STATUS = {
    0: "SEMICRF_OK", 1: "SEMICRF_ERR_NULL", 2: "SEMICRF_ERR_SHAPE",
    3: "SEMICRF_ERR_UNSUPPORTED", 4: "SEMICRF_ERR_WORKSPACE", 5: "SEMICRF_ERR_HIP",
    6: "SEMICRF_ERR_ARG", 7: "SEMICRF_ERR_SCRATCH",
}
STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = (
    "semicrf_status_string", "semicrf_default_checkpoint_interval", "semicrf_checkpoint_interval",
    "semicrf_workspace_size",
    "semicrf_cumulative_scores", "semicrf_logz_fwd", "semicrf_fwd_bwd", "semicrf_fwd_bwd_ex",
    "semicrf_viterbi", "semicrf_path_score", "semicrf_fwd_bwd_static",
)
FWD_BWD_PHASES = ("cumulative_scores", "sweep_first", "sweep_rest", "posteriors", "reductions")


class SemiCRFError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(code, code), status_string(code)))


_lib = None


def load():
    """Load libsemicrf.so and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsemicrf.so is not built (run: python -m semi_markov_crf_zero_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, U, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.semicrf_status_string.argtypes = [I]
    lib.semicrf_status_string.restype = ctypes.c_char_p
    lib.semicrf_default_checkpoint_interval.argtypes = [I, I]
    lib.semicrf_default_checkpoint_interval.restype = I
    lib.semicrf_checkpoint_interval.argtypes = [I, I, I, I]
    lib.semicrf_checkpoint_interval.restype = I
    lib.semicrf_workspace_size.argtypes = [I, I, I, I, I, U, I, ctypes.POINTER(Z)]
    lib.semicrf_workspace_size.restype = I
    lib.semicrf_cumulative_scores.argtypes = [P, P, I, I, I, U, P, P, P, Z, P]
    lib.semicrf_cumulative_scores.restype = I
    lib.semicrf_logz_fwd.argtypes = [P, P, P, P, I, I, I, I, U, P, P, Z, P]
    lib.semicrf_logz_fwd.restype = I
    lib.semicrf_fwd_bwd.argtypes = [P, P, P, P, I, I, I, I, U, I, P, P, P, P, P, P, P, Z, P]
    lib.semicrf_fwd_bwd.restype = I
    lib.semicrf_fwd_bwd_ex.argtypes = [P, P, P, P, I, I, I, I, U, I, P, P, P, P, P, P, P, P, Z,
                                       P, P]
    lib.semicrf_fwd_bwd_ex.restype = I
    lib.semicrf_path_score.argtypes = [P, P, P, P, I, I, I, I, U, P, P, P, P, P, P, P, P, P, P, Z,
                                       P]
    lib.semicrf_path_score.restype = I
    lib.semicrf_fwd_bwd_static.argtypes = [P, P, P, P, I, I, I, I, U, I, P, P, P, P, P, P, P]
    lib.semicrf_fwd_bwd_static.restype = I
    lib.semicrf_viterbi.argtypes = [P, P, P, P, I, I, I, I, U, P, P, P, P, P, P, Z, P]
    lib.semicrf_viterbi.restype = I
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().semicrf_status_string(int(code)).decode()


def semicrf_default_checkpoint_interval(T: int, K: int) -> int:
    return int(load().semicrf_default_checkpoint_interval(int(T), int(K)))


def semicrf_checkpoint_interval(B: int, T: int, C: int, K: int) -> int:
    """Interval used by logz / fwd_bwd when given 0 (see semicrf.h)."""
    return load().semicrf_checkpoint_interval(int(B), int(T), int(C), int(K))


def semicrf_workspace_size(op: int, B: int, T: int, C: int, K: int, flags: int = 0,
                           checkpoint_interval: int = 0) -> int:
    n = ctypes.c_size_t(0)
    rc = load().semicrf_workspace_size(op, B, T, C, K, flags, checkpoint_interval, ctypes.byref(n))
    if rc:
        raise SemiCRFError(rc, "semicrf_workspace_size")
    return int(n.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check_inputs(emissions, lengths, trans=None, dur=None):
    if emissions.dim() != 3:
        raise ValueError("emissions must be [B, T, C]")
    B, T, C = emissions.shape
    dev = emissions.device
    if dev.type != "cuda":
        raise ValueError("semicrf runs on the GPU only; got a %s tensor" % dev.type)
    for name, t, dt in (("emissions", emissions, torch.float32), ("lengths", lengths, torch.int32),
                        ("trans", trans, torch.float32), ("dur", dur, torch.float32)):
        if t is None:
            continue
        if t.device != dev or t.dtype != dt or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s tensor on %s" % (name, dt, dev))
    if lengths.shape != (B,):
        raise ValueError("lengths must be [B]")
    K = None
    if trans is not None and trans.shape != (C, C):
        raise ValueError("trans must be [C, C]")
    if dur is not None:
        if dur.dim() != 2 or dur.shape[1] != C:
            raise ValueError("dur must be [K, C]")
        K = dur.shape[0]
    return B, T, C, K, dev


def _check_weights(name, w, B, dev):
    """A per-sequence weight vector: None, or a contiguous float32 [B] tensor
    on `dev` (the kernels read w[b] as contiguous memory)."""
    if w is None:
        return
    if (w.shape != (B,) or w.dtype != torch.float32 or w.device != dev
            or not w.is_contiguous()):
        raise ValueError("%s must be a contiguous float32 [%d] tensor on %s" % (name, B, dev))


def _workspace(op, B, T, C, K, flags, ckpt, dev):
    n = semicrf_workspace_size(op, B, T, C, K, flags, ckpt)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev), n


def semicrf_cumulative_scores(emissions, lengths, center: bool = True):
    """Row (a): returns (nu [B,C] float64, S [B,T+1,C] float64)."""
    B, T, C, _, dev = _check_inputs(emissions, lengths)
    flags = 0 if center else NO_CENTER
    ws, n = _workspace(OP_SCAN, B, T, C, 1, flags, 0, dev)
    nu = torch.empty((B, C), dtype=torch.float64, device=dev)
    S = torch.empty((B, T + 1, C), dtype=torch.float64, device=dev)
    rc = load().semicrf_cumulative_scores(_ptr(emissions), _ptr(lengths), B, T, C, flags, _ptr(nu),
                                          _ptr(S), _ptr(ws), n, _stream(dev))
    if rc:
        raise SemiCRFError(rc, "semicrf_cumulative_scores")
    return nu, S


def semicrf_logz_fwd(emissions, lengths, trans, dur, center: bool = True, float64: bool = False):
    """log Z [B] float32.  float64: float64 sweeps for every shape (SEMICRF_FLOAT64)."""
    return LogzPlan(emissions, lengths, trans, dur, center, float64).run()


class FwdBwdPlan:
    """Preallocated outputs + workspace for repeated semicrf_fwd_bwd calls on
    one shape (the benchmark times `run()` alone)."""

    def __init__(self, emissions, lengths, trans, dur, center=True, grad_logz=None,
                 checkpoint_interval=0, want_marginals=False, want_boundary=False,
                 low_memory=False, float64=False):
        B, T, C, K, dev = _check_inputs(emissions, lengths, trans, dur)
        _check_weights("grad_logz", grad_logz, B, dev)
        self.args = (emissions, lengths, trans, dur)
        self.B, self.T, self.C, self.K = B, T, C, K
        self.flags = ((0 if center else NO_CENTER) | (LOW_MEMORY if low_memory else 0)
                      | (FLOAT64 if float64 else 0))
        self.ckpt = int(checkpoint_interval)
        self.grad_logz = grad_logz
        self.dev = dev
        self.ws, self.ws_bytes = _workspace(OP_FWD_BWD, B, T, C, K, self.flags, self.ckpt, dev)
        self.logz = torch.empty(B, dtype=torch.float32, device=dev)
        self.grad_emissions = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        self.grad_trans = torch.empty((C, C), dtype=torch.float32, device=dev)
        self.grad_dur = torch.empty((K, C), dtype=torch.float32, device=dev)
        self.marginals = (torch.empty((B, T, C), dtype=torch.float32, device=dev)
                          if want_marginals else None)
        self.boundary = (torch.empty((B, T), dtype=torch.float32, device=dev)
                         if want_boundary else None)

    def run(self, stream=None, phase_events=None):
        """Enqueue one fwd+bwd.  phase_events: optional list of
        len(FWD_BWD_PHASES)+1 recorded torch.cuda.Event(enable_timing=True)
        objects; the library re-records them around its phases."""
        e, l, t, d = self.args
        st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(self.dev)
        evs = None
        if phase_events is not None:
            if len(phase_events) != len(FWD_BWD_PHASES) + 1:
                raise ValueError("need %d events" % (len(FWD_BWD_PHASES) + 1))
            evs = (ctypes.c_void_p * len(phase_events))(*[ev.cuda_event for ev in phase_events])
        rc = load().semicrf_fwd_bwd_ex(
            _ptr(e), _ptr(l), _ptr(t), _ptr(d), self.B, self.T, self.C, self.K, self.flags,
            self.ckpt, _ptr(self.grad_logz), _ptr(self.logz), _ptr(self.grad_emissions),
            _ptr(self.grad_trans), _ptr(self.grad_dur), _ptr(self.marginals),
            _ptr(self.boundary), _ptr(self.ws), self.ws_bytes, st, evs)
        if rc:
            raise SemiCRFError(rc, "semicrf_fwd_bwd")
        return self

    def outputs(self):
        out = dict(logz=self.logz, grad_emissions=self.grad_emissions,
                   grad_trans=self.grad_trans, grad_dur=self.grad_dur)
        if self.marginals is not None:
            out["marginals"] = self.marginals
        if self.boundary is not None:
            out["boundary"] = self.boundary
        return out


def semicrf_fwd_bwd(emissions, lengths, trans, dur, center: bool = True, grad_logz=None,
                    checkpoint_interval: int = 0, want_marginals: bool = False,
                    want_boundary: bool = False, low_memory: bool = False,
                    float64: bool = False):
    """Returns dict(logz, grad_emissions, grad_trans, grad_dur[, marginals][, boundary]).
    low_memory: keep only the checkpoint records and replay the intervals in
    windows for the posteriors (SEMICRF_LOW_MEMORY).  float64: float64 sweeps
    for every shape (SEMICRF_FLOAT64)."""
    plan = FwdBwdPlan(emissions, lengths, trans, dur, center, grad_logz, checkpoint_interval,
                      want_marginals, want_boundary, low_memory, float64)
    return plan.run().outputs()


def semicrf_fwd_bwd_static(emissions, lengths, trans, dur, center: bool = True, grad_logz=None,
                           checkpoint_interval: int = 0, want_marginals: bool = False, out=None):
    """semicrf_fwd_bwd on the library's static device scratch (no workspace
    argument; see semicrf.h).  `out` may hold preallocated outputs (a dict as
    returned), so that repeated calls allocate nothing on the torch side
    either.  Returns dict(logz, grad_emissions, grad_trans, grad_dur[,
    marginals])."""
    B, T, C, K, dev = _check_inputs(emissions, lengths, trans, dur)
    _check_weights("grad_logz", grad_logz, B, dev)
    if out is None:
        out = dict(logz=torch.empty(B, dtype=torch.float32, device=dev),
                   grad_emissions=torch.empty((B, T, C), dtype=torch.float32, device=dev),
                   grad_trans=torch.empty((C, C), dtype=torch.float32, device=dev),
                   grad_dur=torch.empty((K, C), dtype=torch.float32, device=dev))
        if want_marginals:
            out["marginals"] = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    flags = 0 if center else NO_CENTER
    rc = load().semicrf_fwd_bwd_static(
        _ptr(emissions), _ptr(lengths), _ptr(trans), _ptr(dur), B, T, C, K, flags,
        int(checkpoint_interval), _ptr(grad_logz), _ptr(out["logz"]), _ptr(out["grad_emissions"]),
        _ptr(out["grad_trans"]), _ptr(out["grad_dur"]), _ptr(out.get("marginals")), _stream(dev))
    if rc:
        raise SemiCRFError(rc, "semicrf_fwd_bwd_static")
    return out


def _check_segments(segments, B, T, dev):
    names = ("seg_start", "seg_len", "seg_label", "num_segs")
    shapes = ((B, T), (B, T), (B, T), (B,))
    for n, shp in zip(names, shapes):
        t = segments[n]
        if t.device != dev or t.dtype != torch.int32 or not t.is_contiguous() or t.shape != shp:
            raise ValueError("%s must be a contiguous int32 %s tensor on %s" % (n, shp, dev))
    return [segments[n] for n in names]


def semicrf_path_score(emissions, lengths, trans, dur, segments, center: bool = True,
                       weights=None, want_grads: bool = False):
    """Score of the segmentations `segments` (dict of seg_start, seg_len,
    seg_label [B,T] and num_segs [B] int32, the Viterbi output layout).
    Returns dict(score [B] f32[, grad_emissions, grad_trans, grad_dur]): the
    gradients of sum_b weights_b score_b (weights [B] float32 or None = 1)."""
    B, T, C, K, dev = _check_inputs(emissions, lengths, trans, dur)
    ss, sl, sc, ns = _check_segments(segments, B, T, dev)
    _check_weights("weights", weights, B, dev)
    flags = 0 if center else NO_CENTER
    ws, n = _workspace(OP_PATH_SCORE, B, T, C, K, flags, 0, dev)
    score = torch.empty(B, dtype=torch.float32, device=dev)
    out = dict(score=score)
    gx = gt = gd = None
    if want_grads:
        gx = torch.empty((B, T, C), dtype=torch.float32, device=dev)
        gt = torch.empty((C, C), dtype=torch.float32, device=dev)
        gd = torch.empty((K, C), dtype=torch.float32, device=dev)
        out.update(grad_emissions=gx, grad_trans=gt, grad_dur=gd)
    rc = load().semicrf_path_score(_ptr(emissions), _ptr(lengths), _ptr(trans), _ptr(dur), B, T,
                                   C, K, flags, _ptr(ss), _ptr(sl), _ptr(sc), _ptr(ns),
                                   _ptr(weights), _ptr(score), _ptr(gx), _ptr(gt), _ptr(gd),
                                   _ptr(ws), n, _stream(dev))
    if rc:
        raise SemiCRFError(rc, "semicrf_path_score")
    return out


class LogzPlan:
    """Preallocated output + workspace for repeated semicrf_logz_fwd calls."""

    def __init__(self, emissions, lengths, trans, dur, center=True, float64=False):
        B, T, C, K, dev = _check_inputs(emissions, lengths, trans, dur)
        self.args = (emissions, lengths, trans, dur)
        self.B, self.T, self.C, self.K = B, T, C, K
        self.flags = (0 if center else NO_CENTER) | (FLOAT64 if float64 else 0)
        self.dev = dev
        self.ws, self.ws_bytes = _workspace(OP_LOGZ, B, T, C, K, self.flags, 0, dev)
        self.logz = torch.empty(B, dtype=torch.float32, device=dev)

    def run(self):
        e, l, t, d = self.args
        rc = load().semicrf_logz_fwd(_ptr(e), _ptr(l), _ptr(t), _ptr(d), self.B, self.T, self.C,
                                     self.K, self.flags, _ptr(self.logz), _ptr(self.ws),
                                     self.ws_bytes, _stream(self.dev))
        if rc:
            raise SemiCRFError(rc, "semicrf_logz_fwd")
        return self.logz


class ViterbiPlan:
    """Preallocated outputs + workspace for repeated semicrf_viterbi calls."""

    def __init__(self, emissions, lengths, trans, dur, center=True, low_memory=False):
        B, T, C, K, dev = _check_inputs(emissions, lengths, trans, dur)
        self.args = (emissions, lengths, trans, dur)
        self.B, self.T, self.C, self.K = B, T, C, K
        self.flags = (0 if center else NO_CENTER) | (LOW_MEMORY if low_memory else 0)
        self.dev = dev
        self.ws, self.ws_bytes = _workspace(OP_VITERBI, B, T, C, K, self.flags, 0, dev)
        self.best = torch.empty(B, dtype=torch.float32, device=dev)
        self.seg_start = torch.empty((B, T), dtype=torch.int32, device=dev)
        self.seg_len = torch.empty((B, T), dtype=torch.int32, device=dev)
        self.seg_label = torch.empty((B, T), dtype=torch.int32, device=dev)
        self.num_segs = torch.empty(B, dtype=torch.int32, device=dev)

    def run(self):
        e, l, t, d = self.args
        rc = load().semicrf_viterbi(_ptr(e), _ptr(l), _ptr(t), _ptr(d), self.B, self.T, self.C,
                                    self.K, self.flags, _ptr(self.best), _ptr(self.seg_start),
                                    _ptr(self.seg_len), _ptr(self.seg_label),
                                    _ptr(self.num_segs), _ptr(self.ws), self.ws_bytes,
                                    _stream(self.dev))
        if rc:
            raise SemiCRFError(rc, "semicrf_viterbi")
        return dict(best_score=self.best, seg_start=self.seg_start, seg_len=self.seg_len,
                    seg_label=self.seg_label, num_segs=self.num_segs)


def semicrf_viterbi(emissions, lengths, trans, dur, center: bool = True,
                    low_memory: bool = False):
    """Returns dict(best_score [B] f32, seg_start/seg_len/seg_label [B,T] i32, num_segs [B] i32).
    low_memory: recompute the decisions window by window (SEMICRF_LOW_MEMORY)."""
    return ViterbiPlan(emissions, lengths, trans, dur, center, low_memory).run()


# short aliases
cumulative_scores = semicrf_cumulative_scores
logz = semicrf_logz_fwd
fwd_bwd = semicrf_fwd_bwd
viterbi = semicrf_viterbi
path_score = semicrf_path_score
workspace_size = semicrf_workspace_size
