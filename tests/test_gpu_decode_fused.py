"""Selection and decode in one launch (sas_topk_decode, sas_paged_topk_decode).

The fused call ranks the same scores in the same order as the separate Top-K
call and attends with the same row routine as the separate decode: its
blocks must equal the separate call's on every row, its biases agree up to
the order in which the normaliser's sum is taken (the waves of a row sum
their shares first), and its output must equal, bit for bit, the separate
decode run over its own selection.  It is also checked against the oracle
directly (tie-free
rows: the oracle's blocks; O max-abs <= 2e-2, lse <= 1e-3 over the GPU's
selection), with rows that have fewer historical blocks than K (padding),
both bias modes, 16-token units, d 64 and several query rows per call; the
paged form at the serving mix and at edge lengths (1 token, past the table).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, inputs, max_abs, oshape, say, tie_free_rows

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
PW = synth.PAGED_WORKLOADS


def _separate(dev, w, renorm=0):
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk, block=w.block, renorm=renorm)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias, block=w.block)
    return o, lse, idx, bias


def _bias_close(a, b):
    """Equal padding (-inf) and finite entries within 1e-5 of the largest."""
    a, b = host(a), host(b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert np.array_equal(fa, fb) and np.array_equal(a[~fa], b[~fb])
    if fb.any():
        assert max_abs(a[fa], b[fb]) <= 1e-5 * max(1.0, float(np.abs(b[fb]).max()))


def test_fused_decode_full_size_equals_separate():
    w = W["decode_64k_top8"]
    say("fused decode", w.batch, "x", w.tk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    o, lse, idx, bias = ops.topk_decode(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], w.topk)
    o2, l2, i2, b2 = _separate(dev, w)
    o4, l4 = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2)
    _bias_close(bias, b2)
    assert torch.equal(o, o4) and torch.equal(lse, l4)
    assert max_abs(host(o), host(o2)) <= 1e-3


SMALL = {
    # tk 256: three historical blocks, fewer than K (padding)
    "short": W["decode_64k_top8"].with_(batch=3, tk=256, topk=8),
    "decode_4k": W["decode_64k_top8"].with_(batch=2, tk=4096, topk=12),
    "units16": W["decode_64k_top8"].with_(batch=2, tk=4096, block=16, topk=16),
    "d64": W["decode_64k_top8"].with_(batch=2, tk=2048, d=64, ds=16, topk=5),
    "rows5": W["decode_64k_top8"].with_(batch=1, tq=5, tk=1024, topk=6),
    # wave counts around the slot assignment of the row kernels: K = 7 (the
    # last of 8 waves holds only the current block), K = 9 (10 waves) and
    # K = 16 (16 waves, the last one taking the current block and slot 15)
    "k7": W["decode_64k_top8"].with_(batch=2, tk=4096, topk=7),
    "k9": W["decode_64k_top8"].with_(batch=2, tk=4096, topk=9),
    "k16": W["decode_64k_top8"].with_(batch=2, tk=4096, topk=16),
}


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("name", list(SMALL))
def test_fused_decode_small(name, renorm):
    w = SMALL[name]
    say("fused decode", name, renorm)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    o, lse, idx, bias = ops.topk_decode(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"],
                                        w.topk, block=w.block, renorm=renorm)
    o2, l2, i2, b2 = _separate(dev, w, renorm)
    # the separate decode over the fused call's own selection
    o4, l4 = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias, block=w.block)
    o3, l3, i3, b3 = ops.topk_decode(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], w.topk,
                                     block=w.block, renorm=renorm, with_sel=False, with_lse=False)
    torch.cuda.synchronize()
    # same blocks; the bias equal up to the order of the normaliser's sum (K >= 16
    # takes the radix-select kernel in the separate call)
    assert torch.equal(idx, i2)
    _bias_close(bias, b2)
    assert torch.equal(o, o4) and torch.equal(lse, l4) and torch.equal(o, o3)
    assert i3 is None and l3 is None
    # against the oracle: its selection on tie-free rows, its decode over the GPU's selection
    S = oshape(w)
    rows = w.batch * w.hq * w.tq
    idx_ref, _ = oracle.topk_blocks(S, w.topk, f["qs"], f["ks"], renorm=renorm)
    z, _, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    c = np.tile((np.arange(w.tq) + w.tk - w.tq) // w.block, w.batch * w.hq)
    ok = tie_free_rows(z.reshape(rows, -1), c, w.topk)
    assert ok.mean() > 0.8
    ig = idx.cpu().numpy().reshape(rows, -1)
    assert np.array_equal(ig[ok], idx_ref.reshape(rows, -1)[ok])
    bg = host(bias)
    o_ref, l_ref = oracle.sparse_fwd(S, w.topk, f["q"], f["k"], f["v"], idx.cpu().numpy(), bg)
    e = max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1))
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-3


def _dev(t):
    return {n: x.to(DEV) for n, x in t.items()}


@pytest.mark.parametrize("renorm", [0, 1])
def test_fused_paged_mix_equals_separate(renorm):
    pw = PW["decode_paged_mix"]
    t = synth.draw_paged(pw)
    d = _dev(t)
    o, lse, idx, bias = ops.paged_topk_decode(d["q"], d["k_pool"], d["v_pool"], d["qs"],
                                              d["ks_pool"], d["block_table"], d["seq_len"],
                                              pw.topk, renorm=renorm)
    i2, b2 = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk,
                            renorm=renorm)
    o2, l2 = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2)
    _bias_close(bias, b2)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_fused_paged_edge_lengths():
    # the first token of a sequence, a full table, a block-aligned length,
    # 65 tokens, and a length past the table (no keys: o = 0, lse = -inf)
    pw = PW["decode_paged_mix"].with_(batch=5, max_len=64 * 12, topk=4)
    t = synth.draw_paged(pw, lens=[1, 64 * 12, 64 * 5, 65, 64 * 12])
    d = _dev(t)
    d["seq_len"][4] = 64 * 12 + 1
    o, lse, idx, bias = ops.paged_topk_decode(d["q"], d["k_pool"], d["v_pool"], d["qs"],
                                              d["ks_pool"], d["block_table"], d["seq_len"],
                                              pw.topk)
    i2, b2 = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    o2, l2 = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2)
    _bias_close(bias, b2)
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    assert (idx[4] == -1).all().item() and torch.isneginf(lse[4]).all().item()
    assert torch.equal(o[4].float().cpu(), torch.zeros(pw.hq, pw.d))
