"""sas_sparse_fwd_noalloc (the sparse forward with its workspace in the
library's fixed per-GPU scratch array) against sas_sparse_fwd (a workspace
the caller allocates), both through the C ABI: the same outputs on calls in a
row, each later call smaller than the one before, over the block-stationary
prefill path (which uses the scratch) and the row path (decode); shapes
whose workspace exceeds the array are rejected before anything runs.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
from gpu_common import DEV, inputs, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# calls in this order: each smaller than the one before
CASES = [
    ("prefill_2048", W["prefill_32k_top16"].with_(batch=1, hq=8, hkv=2, tq=2048, tk=2048,
                                                  topk=8)),
    ("chunk_384", W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=1, tq=384, tk=1024, topk=5)),
    ("decode_4k", W["decode_64k_top8"].with_(batch=4, tk=4096, topk=8)),
]


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_workspace_entry_point():
    lib = ops.load()
    assert lib.sas_noalloc_scratch_bytes() == 256 << 20
    for name, w in CASES:
        say("noalloc", name, w)
        cpu, dev, _ = inputs(w, ("q", "k", "v", "qs", "ks"))
        idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk)
        sh = ops.make_shape(w.batch, w.hq, w.hkv, w.tq, w.tk, w.d, 32, 64, w.hkv)
        need = ops.sparse_workspace_bytes(sh, w.topk)
        assert need <= lib.sas_noalloc_scratch_bytes()
        say("  workspace bytes", need)
        o_ref, l_ref = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.sas_sparse_fwd_noalloc(ctypes.byref(sh), w.topk, _p(dev["q"]), _p(dev["k"]),
                                        _p(dev["v"]), _p(idx), _p(bias), _p(o), _p(lse), st)
        assert rc == 0, rc
        torch.cuda.synchronize()
        eo = float((o.float() - o_ref.float()).abs().max())
        el = float((lse - l_ref).abs().max())
        say("  max-abs O %.3e lse %.3e, bit-equal %s" % (eo, el, torch.equal(o, o_ref)))
        assert eo <= 2e-2 and el <= 1e-3
        assert torch.isfinite(o.float()).all().item()


def test_noalloc_rejects_workspace_beyond_scratch():
    lib = ops.load()
    A = ctypes.c_void_p(0x10000)
    w = W["prefill_32k_top16"]  # top-16 prefill at 32k needs several GB of partials
    sh = ops.make_shape(w.batch, w.hq, w.hkv, w.tq, w.tk, w.d, 32, 64, w.hkv)
    assert ops.sparse_workspace_bytes(sh, w.topk) > lib.sas_noalloc_scratch_bytes()
    assert lib.sas_sparse_fwd_noalloc(ctypes.byref(sh), w.topk, A, A, A, A, A, A, None,
                                      None) == 6  # SAS_ERR_WORKSPACE, nothing enqueued
