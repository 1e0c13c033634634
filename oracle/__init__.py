"""Float64 CPU oracle for the semi-CRF hot path.

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``semi_markov_crf_zero_amd`` and never imports it.

Contents
  oracle.core        ctypes front end of ``semicrf_oracle.c`` (full-table
                     forward-backward, posteriors, gradients, Viterbi)
  oracle.bruteforce  explicit enumeration of every segmentation (tiny inputs)
  oracle.linear_chain  an independent textbook linear-chain CRF (the K=1 case)
  oracle.closed_form   log Z for zero potentials at any length
  oracle.path        score of a given segmentation and its gradients (the
                     gold-path term of the training loss)
"""
from .core import build, prefix, fwd_bwd, logz, viterbi  # noqa: F401
from .path import path_score  # noqa: F401
