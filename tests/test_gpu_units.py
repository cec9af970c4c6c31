"""Smaller context units: gate blocks of 1 .. 32 tokens against the oracle.

fp32 training path (gate, forward, backward incl. dz, dqs, dks) at blocks
1, 4, 16, 32; bf16 selection (gate, Top-K, threshold) and the sparse forward
at blocks 1, 2, 4, 8, 16 and 32, prefill, chunked prefill and decode.  Same bars as the
64-token cases: fp32 max-abs / rel-L2 <= 1e-4; bf16 O <= 2e-2, lse <= 1e-3;
selections exact on rows clear of ties / of the threshold.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, inputs, max_abs, oshape, rel_l2, say, tie_free_rows

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TINY = W["tiny_fp32"]


@pytest.mark.parametrize("blk", [1, 4, 16, 32])
def test_f32_units_fwd_bwd(blk):
    w = TINY.with_(name="tiny_b%d" % blk, batch=1, hq=2, hkv=1, tq=320, tk=384, block=blk)
    say("f32 units", blk)
    cpu, dev, f = inputs(w)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam,
                     block=blk)
    torch.cuda.synchronize()
    S = oshape(w)
    _, lam_ref, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    fin = np.isfinite(lam_ref)
    assert max_abs(host(lam)[fin], lam_ref[fin]) <= 1e-4
    assert np.array_equal(np.isneginf(host(lam)), np.isneginf(lam_ref))
    o_ref, l_ref = oracle.attn_fwd(S, f["q"], f["k"], f["v"], f["qs"], f["ks"])
    say("  O max-abs", max_abs(host(o), o_ref))
    assert max_abs(host(o), o_ref) <= 1e-4
    assert max_abs(host(lse), l_ref) <= 1e-4
    ref = oracle.attn_bwd(S, f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"])
    for n in ("dq", "dk", "dv", "dz", "dqs", "dks"):
        e = rel_l2(host(g[n]), ref[n])
        say("  %s rel-L2 %.2e" % (n, e))
        assert e <= 1e-4, n


SMALL = {
    "prefill_b16": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=1024, tk=1024,
                                                block=16, topk=12),
    "prefill_b32": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=1024, tk=1024,
                                                block=32, topk=6),
    "chunk_b16": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=200, tk=1024, block=16,
                                             topk=8),
    "decode_b16": W["decode_64k_top8"].with_(batch=3, tk=4096, block=16, topk=16),
    # bf16 token-level and 2 .. 8-token units (pair path for the sparse forward)
    "prefill_b1": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=320, tk=320, block=1,
                                               topk=24),
    "chunk_b2": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=136, tk=448, block=2,
                                             topk=40),
    "prefill_b4": W["prefill_32k_top16"].with_(batch=2, hq=4, hkv=1, tq=512, tk=512, block=4,
                                               topk=16),
    "prefill_b8": W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=640, tk=640, block=8,
                                               topk=10),
    "decode_b1": W["decode_64k_top8"].with_(batch=2, tk=1024, block=1, topk=32),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_units_selection_and_sparse(name):
    w = SMALL[name]
    say("units", name)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    S = oshape(w)
    rows = w.batch * w.hq * w.tq
    c = np.tile((np.arange(w.tq) + w.tk - w.tq) // w.block, w.batch * w.hq)
    # gate normaliser
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=w.block)
    z, lam_ref, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    fin = np.isfinite(lam_ref)
    torch.cuda.synchronize()
    assert max_abs(host(lam)[fin], lam_ref[fin]) <= 1e-4
    # Top-K on tie-free rows
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk, block=w.block)
    torch.cuda.synchronize()
    idx_ref, bias_ref = oracle.topk_blocks(S, w.topk, f["qs"], f["ks"])
    ok = tie_free_rows(z.reshape(rows, -1), c, w.topk)
    assert ok.mean() > 0.8
    ig = idx.cpu().numpy().reshape(rows, -1)
    assert np.array_equal(ig[ok], idx_ref.reshape(rows, -1)[ok])
    # threshold selection: counts on every row clear of the threshold
    theta = 0.01
    rp, col, tb = ops.threshold_blocks(dev["qs"], dev["ks"], theta, w.tk, block=w.block)
    cnt, _, _ = oracle.threshold_blocks(S, theta, f["qs"], f["ks"])
    lt = math.log(float(np.float32(theta)))
    with np.errstate(invalid="ignore"):  # rows without history: -inf - -inf
        zl = z.reshape(rows, -1) - lam_ref.reshape(-1, 1)
    clear = np.array([c[r] == 0 or np.min(np.abs(zl[r, :c[r]] - lt)) > 1e-4
                      for r in range(rows)])
    assert np.array_equal(np.diff(rp.cpu().numpy())[clear], cnt.reshape(-1)[clear])
    # sparse forward over the oracle's selection (pair path for units below 64)
    b32 = bias_ref.astype(np.float32)
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx_ref).to(DEV),
                            torch.from_numpy(b32).to(DEV), block=w.block)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_fwd(S, w.topk, f["q"], f["k"], f["v"], idx_ref,
                                     b32.astype(np.float64))
    e = max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1))
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-3


def test_token_units_selection_and_sparse():
    # token-level units (block 1): every earlier token is a context unit
    w = W["tiny_fp32"].with_(batch=1, hq=2, hkv=1, tq=256, tk=256, block=1, topk=24)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    S = oshape(w)
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk, block=1)
    torch.cuda.synchronize()
    idx_ref, bias_ref = oracle.topk_blocks(S, w.topk, f["qs"], f["ks"])
    z, _, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    rows = w.batch * w.hq * w.tq
    ok = tie_free_rows(z.reshape(rows, -1), np.tile(np.arange(w.tq), w.hq), w.topk)
    assert np.array_equal(idx.cpu().numpy().reshape(rows, -1)[ok], idx_ref.reshape(rows, -1)[ok])
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx_ref).to(DEV),
                            torch.from_numpy(bias_ref.astype(np.float32)).to(DEV), block=1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_fwd(S, w.topk, f["q"], f["k"], f["v"], idx_ref,
                                     bias_ref.astype(np.float32).astype(np.float64))
    assert max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1)) <= 1e-4
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-4


def test_units_full_budget_equals_dense_f32():
    # K covering every unit: the sparse forward is the dense-active forward
    w = TINY.with_(batch=1, hq=2, hkv=1, tq=320, tk=384, block=16)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    K = w.tk // 16
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], K, w.tk, block=16)
    o_s, l_s = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias, block=16)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=16)
    o_d, l_d = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=16)
    torch.cuda.synchronize()
    assert max_abs(host(o_s), host(o_d)) <= 1e-4
    assert max_abs(host(l_s), host(l_d)) <= 1e-4


@pytest.mark.parametrize("blk", [16, 32])
@pytest.mark.parametrize("shape", [(1024, 1024), (300, 1024), (1088, 1088)])
def test_bf16_units_fwd(blk, shape):
    # the bf16 MFMA forward with 2 or 4 gate units per 64-key tile
    tq, tk = shape
    w = W["train_8k"].with_(name="fwd_b%d" % blk, batch=2, hq=4, hkv=2, tq=tq, tk=tk, block=blk)
    if tk % 64:
        w = w.with_(tk=((tk + 63) // 64) * 64, tq=tq)
    say("bf16 units fwd", blk, w.tq, w.tk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(oshape(w), f["q"], f["k"], f["v"], f["qs"], f["ks"])
    e = max_abs(host(o), o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse), l_ref) <= 1e-3


@pytest.mark.parametrize("blk", [16, 32])
def test_bf16_units_fwd_full_size_sampled(blk):
    w = W["train_32k"].with_(block=blk)
    say("bf16 units fwd 32k", blk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    torch.cuda.synchronize()
    from gpu_common import sample_rows
    rows = sample_rows(w, 96, seed=31)
    o_ref, l_ref = oracle.attn_fwd(oshape(w), f["q"], f["k"], f["v"], f["qs"], f["ks"], rows=rows)
    e = max_abs(host(o).reshape(-1, w.d)[rows], o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1)[rows], l_ref) <= 1e-3


def _fwd_bwd_units(dev, w, blk):
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam,
                     block=blk)
    torch.cuda.synchronize()
    return g


BWD_SMALL = {
    "gqa_576": dict(batch=2, hq=8, hkv=2, tq=576, tk=576),
    "q_offset": dict(batch=1, hq=4, hkv=1, tq=160, tk=1024),
    "ragged_q": dict(batch=1, hq=4, hkv=2, tq=200, tk=448),
    "ds64_hks": dict(batch=1, hq=4, hkv=2, hks=4, tq=320, tk=320, ds=64),
    "ds16_q520": dict(batch=1, hq=4, hkv=2, tq=520, tk=576, ds=16),
}


@pytest.mark.parametrize("blk", [16, 32])
@pytest.mark.parametrize("name", list(BWD_SMALL))
def test_bf16_units_bwd(name, blk):
    # the bf16 MFMA backward (dq/dz/dqs and dk/dv kernels, dks) with 2 or 4 units per tile
    w = W["train_8k"].with_(name=name, block=blk, **BWD_SMALL[name])
    say("bf16 units bwd", name, blk)
    cpu, dev, f = inputs(w)
    g = _fwd_bwd_units(dev, w, blk)
    ref = oracle.attn_bwd(oshape(w), f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"])
    for n in ("dq", "dk", "dv", "dz", "dqs", "dks"):
        e = rel_l2(host(g[n]), ref[n])
        say("  %s rel-L2 %.3e" % (n, e))
        assert e <= 5e-2, n
    dz = host(g["dz"])
    c = (np.arange(w.tq) + w.tk - w.tq) // blk
    for i in range(w.tq):
        assert np.all(dz[:, :, i, c[i]:] == 0.0)


@pytest.mark.parametrize("blk", [16, 32])
def test_bf16_units_bwd_full_size_sampled(blk):
    w = W["train_32k"].with_(block=blk)
    say("bf16 units bwd 32k", blk)
    cpu, dev, f = inputs(w)
    g = _fwd_bwd_units(dev, w, blk)
    from gpu_common import sample_rows
    rows = sample_rows(w, 16, seed=13)
    keys = np.array([(b * w.hkv + kh) * w.tk + u for b in range(w.batch) for kh in range(w.hkv)
                     for u in range(w.tk - 128, w.tk, 9)], dtype=np.int64)
    sblk = np.array([(b * w.kheads + s) * w.nb + j for b in range(w.batch)
                     for s in range(w.kheads) for j in (w.nb - 2, w.nb - 5)], dtype=np.int64)
    ref = oracle.attn_bwd(oshape(w), f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"],
                          rows=rows, keys=keys, sblocks=sblk)
    got = {
        "dq": host(g["dq"]).reshape(-1, w.d)[rows],
        "dz": host(g["dz"]).reshape(-1, w.nb)[rows],
        "dqs": host(g["dqs"]).reshape(-1, w.ds)[rows],
        "dk": host(g["dk"]).reshape(-1, w.d)[keys],
        "dv": host(g["dv"]).reshape(-1, w.d)[keys],
        "dks": host(g["dks"]).reshape(-1, w.ds)[sblk],
    }
    for n in got:
        e = rel_l2(got[n], ref[n])
        say("  %s rel-L2 %.3e" % (n, e))
        assert e <= 5e-2, n


@pytest.mark.parametrize("blk", [16, 32])
def test_units_csr_and_full_budget_bf16(blk):
    # block-stationary path at 16 / 32-token units: a threshold (CSR) selection
    # against the oracle, and K covering every unit == the dense forward
    w = W["prefill_32k_top16"].with_(batch=1, hq=4, hkv=2, tq=640, tk=1024, block=blk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    S = oshape(w)
    rows = w.batch * w.hq * w.tq
    rp, col, tb = ops.threshold_blocks(dev["qs"], dev["ks"], 0.01, w.tk, block=blk)
    o, lse = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, col, tb, block=blk)
    torch.cuda.synchronize()
    rph, colh, tbh = rp.cpu().numpy(), col.cpu().numpy(), tb.cpu().numpy()
    width = max(1, int(np.diff(rph).max()))
    pi = np.full((rows, width), -1, dtype=np.int32)
    pb = np.full((rows, width), -np.inf)
    for r in range(rows):
        n = rph[r + 1] - rph[r]
        pi[r, :n] = colh[rph[r]:rph[r + 1]]
        pb[r, :n] = tbh[rph[r]:rph[r + 1]]
    o_ref, l_ref = oracle.sparse_fwd(S, width, f["q"], f["k"], f["v"], pi, pb)
    e = max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1))
    say("  csr O max-abs", e, "nnz", len(colh))
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-3
    K = w.tk // blk
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], K, w.tk, block=blk)
    o_s, l_s = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias, block=blk)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o_d, l_d = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    torch.cuda.synchronize()
    assert max_abs(host(o_s), host(o_d)) <= 2e-2
    assert max_abs(host(l_s), host(l_d)) <= 1e-3
