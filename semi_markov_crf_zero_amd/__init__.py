"""MI355X-native semi-CRF hot path (exact forward-backward, Viterbi).

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI of
include/semicrf.h (libsemicrf.so); ``binding`` marshals torch tensors into
it.  ``workloads`` draws the seeded synthetic inputs.  Importing the package
does not load the library; the first call does, and fails loudly if it has
not been built.
"""
__all__ = ["binding", "workloads"]
