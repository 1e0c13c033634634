"""Training loss of the semi-CRF as a torch.autograd.Function over the C ABI.

The loss of a labelled segmentation y of sequence b is its negative
log-likelihood, log Z_b - score_b(y) ("Streaming Structured Inference with
Flash-SemiCRF", technical summary at gist.science, section 3: training on
labelled segmentations).  Both terms and their exact gradients come from the
HIP library: semicrf_fwd_bwd (log Z and dlogZ/d{x, trans, dur}) and
semicrf_path_score (the gold score and its count gradients).  This module
only marshals tensors: no semi-CRF arithmetic runs here beyond subtracting
the two library outputs.

    loss = semicrf_nll(emissions, lengths, trans, dur, gold)   # [B]
    loss.sum().backward()

`gold` holds seg_start / seg_len / seg_label [B, T] and num_segs [B] int32
(the layout semicrf_viterbi returns).  Gradients flow to emissions, trans and
dur (float32, contiguous, on the GPU).
"""
from __future__ import annotations

import torch

from . import binding as bd

_SEG_KEYS = ("seg_start", "seg_len", "seg_label", "num_segs")


class SemiCRFNLL(torch.autograd.Function):
    """Per-sequence log Z - score(gold).  The forward pass runs one
    semicrf_fwd_bwd (unit weights) and one semicrf_path_score with gradients
    when any input needs a gradient (log Z and the score alone otherwise);
    the backward pass scales those gradients when every sequence receives
    the same upstream weight (loss.sum(), loss.mean()), and otherwise calls
    both again with the upstream weights."""

    @staticmethod
    def forward(ctx, emissions, trans, dur, lengths, seg_start, seg_len, seg_label, num_segs,
                center, checkpoint_interval):
        gold = dict(zip(_SEG_KEYS, (seg_start, seg_len, seg_label, num_segs)))
        need = any(ctx.needs_input_grad[:3])
        if need:
            out = bd.semicrf_fwd_bwd(emissions, lengths, trans, dur, center=center,
                                     checkpoint_interval=checkpoint_interval)
            ps = bd.semicrf_path_score(emissions, lengths, trans, dur, gold, center=center,
                                       want_grads=True)
            logz = out["logz"]
            ctx.grads = (out["grad_emissions"] - ps["grad_emissions"],
                         out["grad_trans"] - ps["grad_trans"],
                         out["grad_dur"] - ps["grad_dur"])
            ctx.save_for_backward(emissions, trans, dur, lengths, seg_start, seg_len, seg_label,
                                  num_segs)
        else:
            logz = bd.semicrf_logz_fwd(emissions, lengths, trans, dur, center=center)
            ps = bd.semicrf_path_score(emissions, lengths, trans, dur, gold, center=center)
        ctx.center = center
        ctx.ckpt = checkpoint_interval
        return logz - ps["score"]

    @staticmethod
    def backward(ctx, g):
        g = g.contiguous().float()
        uniform = bool((g == g[0]).all().item()) if g.numel() else True
        if uniform:
            s = g[0] if g.numel() else g.new_zeros(())
            gx, gt, gd = (t * s for t in ctx.grads)
        else:
            (emissions, trans, dur, lengths, seg_start, seg_len, seg_label,
             num_segs) = ctx.saved_tensors
            gold = dict(zip(_SEG_KEYS, (seg_start, seg_len, seg_label, num_segs)))
            out = bd.semicrf_fwd_bwd(emissions, lengths, trans, dur, center=ctx.center,
                                     grad_logz=g, checkpoint_interval=ctx.ckpt)
            ps = bd.semicrf_path_score(emissions, lengths, trans, dur, gold, center=ctx.center,
                                       weights=g, want_grads=True)
            gx = out["grad_emissions"] - ps["grad_emissions"]
            gt = out["grad_trans"] - ps["grad_trans"]
            gd = out["grad_dur"] - ps["grad_dur"]
        ctx.grads = None
        return gx, gt, gd, None, None, None, None, None, None, None


def semicrf_nll(emissions, lengths, trans, dur, gold, center: bool = True,
                checkpoint_interval: int = 0):
    """Negative log-likelihood [B] of the segmentations `gold` (dict of
    seg_start, seg_len, seg_label [B,T] and num_segs [B], int32 on the
    device); NaN for an invalid length or segmentation."""
    return SemiCRFNLL.apply(emissions, trans, dur, lengths,
                            *(gold[k] for k in _SEG_KEYS), center, int(checkpoint_interval))


class SemiCRFLogPartition(torch.autograd.Function):
    """log Z [B] with its exact gradients (semicrf_fwd_bwd with the upstream
    weights as grad_logz)."""

    @staticmethod
    def forward(ctx, emissions, trans, dur, lengths, center, checkpoint_interval):
        ctx.save_for_backward(emissions, trans, dur, lengths)
        ctx.center = center
        ctx.ckpt = checkpoint_interval
        return bd.semicrf_logz_fwd(emissions, lengths, trans, dur, center=center)

    @staticmethod
    def backward(ctx, g):
        emissions, trans, dur, lengths = ctx.saved_tensors
        out = bd.semicrf_fwd_bwd(emissions, lengths, trans, dur, center=ctx.center,
                                 grad_logz=g.contiguous().float(), checkpoint_interval=ctx.ckpt)
        return out["grad_emissions"], out["grad_trans"], out["grad_dur"], None, None, None


def semicrf_log_partition(emissions, lengths, trans, dur, center: bool = True,
                          checkpoint_interval: int = 0):
    return SemiCRFLogPartition.apply(emissions, trans, dur, lengths, center,
                                     int(checkpoint_interval))
