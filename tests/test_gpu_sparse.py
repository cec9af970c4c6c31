"""GPU top-K sparse forward (prefill and decode) vs fp64 oracle.

Prefill takes one of two paths by the share of history the selection keeps:
selections keeping at least 3/16 of the average row's history run the dense
query-stationary kernel with the selection as a per-(block, row) bias
(-inf where not attended); sparser ones the block-stationary path (gather,
partials, merge).  The small cases below sit on both sides of that line
(block path: "block_4096_k2", "chunk_block").

Both sides attend the same selection: the oracle's top-K (idx, bias) is the
input to the GPU kernel and to the oracle's sparse forward (bias rounded to
fp32 for both).  End-to-end GPU top-K -> GPU sparse is compared on the rows
whose selection is tie-free.  Bar: bf16 output max-abs <= 2e-2, lse abs <= 1e-3.
"""

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import (DEV, host, inputs, max_abs, oshape, rel_l2, sample_rows, say,
                        tie_free_rows)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SMALL = {
    "prefill_1088": W["prefill_32k_top16"].with_(name="prefill_1088", batch=2, hq=8, hkv=2,
                                                 tq=1088, tk=1088, topk=4),
    "chunk_q": W["prefill_32k_top16"].with_(name="chunk_q", batch=1, hq=4, hkv=1, tq=100,
                                            tk=2048, topk=6),
    "decode_8k": W["decode_64k_top8"].with_(name="decode_8k", batch=3, tk=8192, topk=8),
    "big_budget": W["prefill_32k_top16"].with_(name="big_budget", batch=1, hq=4, hkv=2, tq=640,
                                               tk=640, topk=12),
    "d64": W["prefill_32k_top16"].with_(name="d64", batch=1, hq=4, hkv=2, tq=512, tk=512, d=64,
                                        topk=3),
    "quarter_2048": W["prefill_32k_top25pct"].with_(name="quarter_2048", batch=1, hq=8, hkv=2,
                                                    tq=2048, tk=2048, topk=8),
    # block-stationary path: 2 blocks of a 2048-key average history
    "block_4096_k2": W["prefill_32k_top16"].with_(name="block_4096_k2", batch=1, hq=4, hkv=1,
                                                  tq=4096, tk=4096, topk=2),
    # chunked prefill on the block-stationary path (query offset 3584)
    "chunk_block": W["prefill_32k_top16"].with_(name="chunk_block", batch=1, hq=4, hkv=2,
                                                tq=512, tk=4096, topk=4),
    # chunked prefill on the dense-kernel path (query offset 768, 6 of ~14 blocks)
    "chunk_dense": W["prefill_32k_top16"].with_(name="chunk_dense", batch=2, hq=4, hkv=1,
                                                tq=256, tk=1024, topk=6),
}


def _oracle_selection(w, f, renorm=0):
    if w.frac > 0:
        idx, bias = oracle.topk_budget(oshape(w), w.topk, w.frac, f["qs"], f["ks"], renorm=renorm)
    else:
        idx, bias = oracle.topk_blocks(oshape(w), w.topk, f["qs"], f["ks"], renorm=renorm)
    bias32 = bias.astype(np.float32)
    return idx, bias32


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("name", list(SMALL))
def test_sparse_small(name, renorm):
    w = SMALL[name]
    say("sparse", name, renorm)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f, renorm)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_fwd(oshape(w), w.topk, f["q"], f["k"], f["v"], idx,
                                     bias32.astype(np.float64))
    e = max_abs(host(o), o_ref)
    say("  O max-abs", e, "lse", max_abs(host(lse), l_ref))
    assert e <= 2e-2
    assert max_abs(host(lse), l_ref) <= 1e-3


def test_sparse_end_to_end_tie_free():
    w = SMALL["prefill_1088"]
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx_g, bias_g = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk)
    o, _ = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx_g, bias_g)
    torch.cuda.synchronize()
    idx, bias = oracle.topk_blocks(oshape(w), w.topk, f["qs"], f["ks"])
    o_ref, _ = oracle.sparse_fwd(oshape(w), w.topk, f["q"], f["k"], f["v"], idx, bias)
    z, _, _ = oracle.gate_scores(oshape(w), f["qs"], f["ks"])
    c = np.tile((np.arange(w.tq) + w.tk - w.tq) // 64, w.batch * w.hq)
    ok = tie_free_rows(z.reshape(-1, w.nb), c, w.topk)
    assert ok.mean() > 0.9
    assert max_abs(host(o).reshape(-1, w.d)[ok], o_ref.reshape(-1, w.d)[ok]) <= 2e-2


def test_sparse_full_budget_equals_dense():
    # K >= c(t) for every row: the sparse forward is the dense-active forward
    w = SMALL["prefill_1088"].with_(topk=17)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx_g, bias_g = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk)
    o_s, l_s = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx_g, bias_g)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk)
    o_d, l_d = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam)
    torch.cuda.synchronize()
    assert max_abs(host(o_s), host(o_d)) <= 2e-2
    assert max_abs(host(l_s), host(l_d)) <= 1e-3


def test_sparse_skips_invalid_entries():
    # entries that are -1 or not before c(t) are skipped, never read
    w = SMALL["chunk_q"]
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f)
    bad = idx.copy()
    bad[..., -1] = 10_000  # far out of range
    o1, _ = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(bad).to(DEV),
                           torch.from_numpy(bias32).to(DEV))
    good = idx.copy()
    good[..., -1] = -1
    o2, _ = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(good).to(DEV),
                           torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["prefill_1088", "block_4096_k2"])
def test_sparse_prefill_skips_invalid_entries(name):
    # both prefill paths: entries that are -1, past the row's history or out of
    # range are skipped
    w = SMALL[name]
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f)
    c = (np.arange(w.tq) + w.tk - w.tq) // 64
    bad = idx.copy()
    bad[..., -1] = np.where(np.arange(w.tq) % 2 == 0, 10_000, c)[None, None, :]
    o1, l1 = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(bad).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    good = idx.copy()
    good[..., -1] = -1
    o2, l2 = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(good).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = oracle.sparse_fwd(oshape(w), w.topk, f["q"], f["k"], f["v"], good,
                                     bias32.astype(np.float64))
    assert max_abs(host(o2), o_ref) <= 2e-2 and max_abs(host(l2), l_ref) <= 1e-3


def test_sparse_prefill_full_size_sampled():
    w = W["prefill_32k_top16"]
    say("sparse prefill full")
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    rows = sample_rows(w, 256, seed=17)
    o_ref, l_ref = oracle.sparse_fwd(oshape(w), w.topk, f["q"], f["k"], f["v"], idx,
                                     bias32.astype(np.float64), rows=rows)
    e = max_abs(host(o).reshape(-1, w.d)[rows], o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1)[rows], l_ref) <= 1e-3
    assert torch.isfinite(o).all().item()


def test_sparse_quarter_budget_full_size_sampled():
    # 32k prefill at a quarter of each row's history (up to 128 blocks per row)
    w = W["prefill_32k_top25pct"]
    say("sparse prefill 25% full")
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f, renorm=1)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    rows = sample_rows(w, 192, seed=23)
    o_ref, l_ref = oracle.sparse_fwd(oshape(w), w.topk, f["q"], f["k"], f["v"], idx,
                                     bias32.astype(np.float64), rows=rows)
    e = max_abs(host(o).reshape(-1, w.d)[rows], o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1)[rows], l_ref) <= 1e-3
    assert torch.isfinite(o).all().item()


def test_sparse_decode_full_size():
    w = W["decode_64k_top8"]
    say("sparse decode full")
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias32 = _oracle_selection(w, f)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx).to(DEV),
                            torch.from_numpy(bias32).to(DEV))
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    worst = 0.0
    for b in range(w.batch):
        for g in range(w.hkv):
            hs = slice(g * 4, g * 4 + 4)
            S1 = oracle.OracleShape(1, 4, 1, 1, w.tk, w.d, w.ds, 64)
            kk = synth.to_f64(cpu["k"][b:b + 1, g:g + 1])
            vv = synth.to_f64(cpu["v"][b:b + 1, g:g + 1])
            o_ref, l_ref = oracle.sparse_fwd(S1, w.topk, f["q"][b:b + 1, hs], kk, vv,
                                             idx[b:b + 1, hs], bias32[b:b + 1, hs].astype(np.float64))
            worst = max(worst, max_abs(og[b, hs], o_ref))
            assert max_abs(lg[b, hs], l_ref) <= 1e-3
    say("  O max-abs", worst)
    assert worst <= 2e-2

