"""MI355X-native SAS gated block-sparse attention.

The compute lives in ``libsas.so`` (hand-written HIP for gfx950 behind a C
ABI declared in ``include/sas.h``).  :mod:`gated_block_sparse_sas_amd.ops`
marshals torch tensors into that ABI; it never computes anything itself.
Import the submodules directly (``ops``, ``synth``); importing the package
loads nothing.
"""
