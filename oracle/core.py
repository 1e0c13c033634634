"""ctypes front end of the float64 C oracle (``semicrf_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  The C file states the
definitions it implements and the pages it follows; this module only
marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "semicrf_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE float64, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared",
               "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_prefix.argtypes = [I, I, I, P, P, I, P, P]
        lib.oracle_fwd_bwd.argtypes = [I, I, I, I, P, P, P, P, I, P, P, P, P, P, P, P, P, I]
        lib.oracle_viterbi.argtypes = [I, I, I, I, P, P, P, P, I, P, P, P, P, P, P, I]
        for f in (lib.oracle_prefix, lib.oracle_fwd_bwd, lib.oracle_viterbi):
            f.restype = I
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _inputs(inp):
    x = np.ascontiguousarray(inp["emissions"], dtype=np.float32)
    lengths = np.ascontiguousarray(inp["lengths"], dtype=np.int32)
    trans = np.ascontiguousarray(inp["trans"], dtype=np.float32)
    dur = np.ascontiguousarray(inp["dur"], dtype=np.float32)
    B, T, C = x.shape
    K = dur.shape[0]
    assert trans.shape == (C, C) and dur.shape == (K, C) and lengths.shape == (B,)
    return x, lengths, trans, dur, B, T, C, K


def prefix(inp, center=True):
    """Return (nu [B,C], S [B,T+1,C]) in float64."""
    x, lengths, _, _, B, T, C, _ = _inputs(inp)
    nu = np.zeros((B, C))
    S = np.zeros((B, T + 1, C))
    rc = _load().oracle_prefix(B, T, C, _p(x), _p(lengths), int(center), _p(nu), _p(S))
    if rc:
        raise ValueError("oracle_prefix failed with code %d" % rc)
    return nu, S


def fwd_bwd(inp, center=True, grad_logz=None, nthreads=0, want_grads=True):
    """Full forward-backward.  Returns a dict of float64 arrays:
    logz [B], logz_bwd [B], grad_emissions [B,T,C], grad_trans [C,C],
    grad_dur [K,C], marginals [B,T,C], boundary [B,T] (probability that a
    segment starts at t)."""
    x, lengths, trans, dur, B, T, C, K = _inputs(inp)
    logz = np.zeros(B)
    logz_bwd = np.zeros(B)
    w = None if grad_logz is None else np.ascontiguousarray(grad_logz, dtype=np.float64)
    if want_grads:
        gx = np.zeros((B, T, C))
        gt = np.zeros((C, C))
        gd = np.zeros((K, C))
        mu = np.zeros((B, T, C))
        bnd = np.zeros((B, T))
    else:
        gx = gt = gd = mu = bnd = None
    rc = _load().oracle_fwd_bwd(B, T, C, K, _p(x), _p(lengths), _p(trans), _p(dur),
                                int(center), _p(w), _p(logz), _p(logz_bwd), _p(gx),
                                _p(gt), _p(gd), _p(mu), _p(bnd), int(nthreads))
    if rc:
        raise RuntimeError("oracle_fwd_bwd failed with code %d" % rc)
    out = dict(logz=logz, logz_bwd=logz_bwd)
    if want_grads:
        out.update(grad_emissions=gx, grad_trans=gt, grad_dur=gd, marginals=mu, boundary=bnd)
    return out


def logz(inp, center=True, nthreads=0):
    """Forward pass only: log Z [B]."""
    x, lengths, trans, dur, B, T, C, K = _inputs(inp)
    out = np.zeros(B)
    rc = _load().oracle_fwd_bwd(B, T, C, K, _p(x), _p(lengths), _p(trans), _p(dur),
                                int(center), None, _p(out), None, None, None, None, None,
                                None, int(nthreads))
    if rc:
        raise RuntimeError("oracle_fwd_bwd failed with code %d" % rc)
    return out


def viterbi(inp, center=True, nthreads=0):
    """Max-semiring decoding.  Returns dict with best_score [B] f64,
    seg_start/seg_len/seg_label [B,T] i32 (-1 padded), num_segs [B] i32,
    min_margin [B] f64."""
    x, lengths, trans, dur, B, T, C, K = _inputs(inp)
    score = np.zeros(B)
    ss = np.zeros((B, T), dtype=np.int32)
    sl = np.zeros((B, T), dtype=np.int32)
    sc = np.zeros((B, T), dtype=np.int32)
    ns = np.zeros(B, dtype=np.int32)
    mm = np.zeros(B)
    rc = _load().oracle_viterbi(B, T, C, K, _p(x), _p(lengths), _p(trans), _p(dur),
                                int(center), _p(score), _p(ss), _p(sl), _p(sc), _p(ns),
                                _p(mm), int(nthreads))
    if rc:
        raise RuntimeError("oracle_viterbi failed with code %d" % rc)
    return dict(best_score=score, seg_start=ss, seg_len=sl, seg_label=sc, num_segs=ns,
                min_margin=mm)
