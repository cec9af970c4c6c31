"""Dynamic-threshold selection (CSR) and the sparse forward over a CSR
selection, against the oracle.

A row is compared exactly when no gate of the row lies within a margin of
the threshold (both sides then take every decision the same way: the GPU's
fp32 log-gate differs from the oracle's fp64 one by ~1e-6); elsewhere the
kept set may differ at the boundary, and only the row's consistency is
checked.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, inputs, max_abs, oshape, sample_rows, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
MARGIN = 1e-4


def _csr_host(row_ptr, col, bias):
    return (row_ptr.cpu().numpy(), col.cpu().numpy(), bias.cpu().numpy())


def _padded(rp, col, bias, rows, width):
    """CSR -> padded [rows, width] idx (-1) / bias (-inf) for the oracle."""
    idx = np.full((rows, width), -1, dtype=np.int32)
    b = np.full((rows, width), -np.inf)
    for r in range(rows):
        n = rp[r + 1] - rp[r]
        idx[r, :n] = col[rp[r]:rp[r + 1]]
        b[r, :n] = bias[rp[r]:rp[r + 1]]
    return idx, b


def _clear_rows(z, lam, c, theta):
    """Rows whose log-gates z - lam all sit farther than MARGIN from log theta."""
    ok = np.ones(z.shape[0], dtype=bool)
    if theta <= 0:
        return ok  # every historical block is kept: no boundary
    lt = math.log(float(np.float32(theta)))
    for r in range(z.shape[0]):
        if c[r] and np.min(np.abs(z[r, :c[r]] - lam[r] - lt)) <= MARGIN:
            ok[r] = False
    return ok


SMALL = {
    "prefill_1088": W["prefill_32k_theta"].with_(batch=2, hq=4, hkv=2, tq=1088, tk=1088),
    "chunk_q": W["prefill_32k_theta"].with_(batch=1, hq=8, hkv=2, tq=300, tk=2048),
    "decode": W["prefill_32k_theta"].with_(batch=3, hq=8, hkv=2, tq=1, tk=4096),
    # the other selector widths of the matrix-core selection: ds 16 with a
    # query offset, ds 64 with selector keys per query head (a ragged last
    # 256-row workgroup in both)
    "ds16_q504": W["prefill_32k_theta"].with_(batch=1, hq=4, hkv=2, tq=520, tk=1024, ds=16),
    "ds64_hks": W["prefill_32k_theta"].with_(batch=1, hq=4, hkv=2, tq=640, tk=640, ds=64, hks=4),
}


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("theta", [0.0, 0.01, 0.1])
@pytest.mark.parametrize("name", list(SMALL))
def test_threshold_small(name, theta, renorm):
    w = SMALL[name]
    say("threshold", name, theta, renorm)
    cpu, dev, f = inputs(w, ("qs", "ks"))
    rp, col, bias = _csr_host(*ops.threshold_blocks(dev["qs"], dev["ks"], theta, w.tk,
                                                    renorm=renorm))
    S = oshape(w)
    cnt, idx, b_ref = oracle.threshold_blocks(S, theta, f["qs"], f["ks"], renorm=renorm)
    z, lam, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    rows = w.batch * w.hq * w.tq
    c = np.tile((np.arange(w.tq) + w.tk - w.tq) // 64, w.batch * w.hq)
    ok = _clear_rows(z.reshape(rows, -1), lam.reshape(-1), c, theta)
    say("  clear rows", int(ok.sum()), "of", rows, "nnz", int(rp[-1]))
    assert ok.mean() > 0.9
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == len(col)
    g_cnt = np.diff(rp)
    r_cnt = cnt.reshape(-1)
    idx = idx.reshape(rows, -1)
    b_ref = b_ref.reshape(rows, -1)
    assert np.array_equal(g_cnt[ok], r_cnt[ok])
    for r in np.nonzero(ok)[0]:
        n = g_cnt[r]
        assert np.array_equal(col[rp[r]:rp[r + 1]], idx[r, :n]), r
        assert max_abs(bias[rp[r]:rp[r + 1]], b_ref[r, :n]) <= 1e-4
    # every row: kept blocks ascending, historical
    for r in range(rows):
        seg = col[rp[r]:rp[r + 1]]
        assert np.all(np.diff(seg) > 0) and (len(seg) == 0 or (seg[0] >= 0 and seg[-1] < c[r]))


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("name", ["prefill_1088", "chunk_q", "decode"])
def test_sparse_csr_small(name, renorm):
    # the oracle's threshold selection, as CSR, through the GPU CSR forward
    w = SMALL[name]
    say("sparse csr", name, renorm)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    S = oshape(w)
    cnt, idx, b_ref = oracle.threshold_blocks(S, 0.01, f["qs"], f["ks"], renorm=renorm)
    rows = w.batch * w.hq * w.tq
    cnt = cnt.reshape(-1)
    rp = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
    idx = idx.reshape(rows, -1)
    b32 = b_ref.reshape(rows, -1).astype(np.float32)
    col = np.concatenate([idx[r, :cnt[r]] for r in range(rows)]).astype(np.int32)
    bias = np.concatenate([b32[r, :cnt[r]] for r in range(rows)]).astype(np.float32)
    o, lse = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], torch.from_numpy(rp).to(DEV),
                                torch.from_numpy(col).to(DEV), torch.from_numpy(bias).to(DEV))
    torch.cuda.synchronize()
    width = max(1, int(cnt.max()))
    pi, pb = _padded(rp, col, bias.astype(np.float64), rows, width)
    o_ref, l_ref = oracle.sparse_fwd(S, width, f["q"], f["k"], f["v"], pi, pb)
    e = max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1))
    say("  O max-abs", e, "nnz", len(col))
    assert e <= 2e-2
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-3


@pytest.mark.parametrize("tq,topk,bits", [(4096, 4, True), (2048, 8, False)])
def test_sparse_csr_equals_fixed(tq, topk, bits):
    # a Top-K selection written as CSR (pads dropped): where the fixed-budget
    # call takes the block-stationary path too (4096 tokens, 4 blocks) the
    # bits are equal; where it takes the dense-kernel path (2048 tokens, 8 of
    # ~16 blocks) the two paths agree to the bf16 bar
    w = W["prefill_32k_top16"].with_(batch=1, hq=8, hkv=2, tq=tq, tk=tq, topk=topk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk)
    o1, l1 = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias)
    keep = (idx >= 0).reshape(-1, w.topk)
    rp = torch.zeros(keep.shape[0] + 1, dtype=torch.int64, device=DEV)
    rp[1:] = torch.cumsum(keep.sum(-1), 0)
    col = idx.reshape(-1, w.topk)[keep].contiguous()
    b = bias.reshape(-1, w.topk)[keep].contiguous()
    o2, l2 = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, col, b)
    torch.cuda.synchronize()
    if bits:
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)
    else:
        assert max_abs(host(o1), host(o2)) <= 2e-2
        assert max_abs(host(l1), host(l2)) <= 1e-3


def test_sparse_csr_empty_selection():
    # theta above every gate: nnz = 0, each row attends its current block only
    w = SMALL["prefill_1088"]
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    rp, col, bias = ops.threshold_blocks(dev["qs"], dev["ks"], 2.0, w.tk)
    assert int(rp[-1].item()) == 0 and col.numel() == 0
    o, lse = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, col, bias)
    torch.cuda.synchronize()
    S = oshape(w)
    rows = w.batch * w.hq * w.tq
    o_ref, l_ref = oracle.sparse_fwd(S, 1, f["q"], f["k"], f["v"],
                                     np.full((rows, 1), -1, np.int32), np.full((rows, 1), -np.inf))
    assert max_abs(host(o).reshape(rows, -1), o_ref.reshape(rows, -1)) <= 2e-2
    assert max_abs(host(lse).reshape(-1), l_ref.reshape(-1)) <= 1e-3


def test_threshold_full_size():
    # 32k prefill, theta = 0.01: selection on sampled rows (one-row oracle
    # shapes), then the CSR forward over the GPU's selection on sampled rows
    w = W["prefill_32k_theta"]
    say("threshold full")
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    row_ptr, col_d, bias_d = ops.threshold_blocks(dev["qs"], dev["ks"], w.theta, w.tk)
    o, lse = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], row_ptr, col_d, bias_d)
    torch.cuda.synchronize()
    rp, col, bias = _csr_host(row_ptr, col_d, bias_d)
    rows_all = w.batch * w.hq * w.tq
    say("  nnz", int(rp[-1]), "mean per row", float(rp[-1]) / rows_all)
    rows = sample_rows(w, 600, seed=11)
    qs = f["qs"].reshape(-1, w.ds)
    o_gpu, l_gpu = host(o).reshape(-1, w.d), host(lse).reshape(-1)
    n_clear, e_o = 0, 0.0
    for r in rows:
        i = r % w.tq
        h = (r // w.tq) % w.hq
        b = r // (w.tq * w.hq)
        t = w.tk - w.tq + i
        nb1 = (t + 1 + 63) // 64
        ks1 = f["ks"][b, h // (w.hq // w.kheads)][None, None, :nb1]
        S1 = oracle.OracleShape(1, 1, 1, 1, t + 1, w.d, w.ds, 64)
        q1 = qs[r][None, None, None, :]
        cnt, idx, br = oracle.threshold_blocks(S1, w.theta, q1, ks1)
        z, lam, _ = oracle.gate_scores(S1, q1, ks1)
        if not _clear_rows(z.reshape(1, -1), lam.reshape(-1), np.array([t // 64]), w.theta)[0]:
            continue
        n_clear += 1
        n = int(cnt.reshape(-1)[0])
        assert rp[r + 1] - rp[r] == n, r
        assert np.array_equal(col[rp[r]:rp[r + 1]], idx.reshape(-1)[:n])
        assert max_abs(bias[rp[r]:rp[r + 1]], br.reshape(-1)[:n]) <= 1e-4
        # the row's output: the oracle's forward over its own selection (the
        # GPU's equals it on this row), on the row's key prefix
        g = h // (w.hq // w.hkv)
        k1 = f["k"][b, g][None, None, :t + 1]
        v1 = f["v"][b, g][None, None, :t + 1]
        qq = f["q"].reshape(-1, w.d)[r][None, None, None, :]
        width = max(n, 1)
        pi = idx.reshape(1, 1, 1, -1)[..., :width].astype(np.int32)
        pb = br.reshape(1, 1, 1, -1)[..., :width].astype(np.float32).astype(np.float64)
        o1, l1 = oracle.sparse_fwd(S1, width, qq, k1, v1, pi, pb)
        e_o = max(e_o, max_abs(o_gpu[r], o1.reshape(-1)))
        assert abs(l_gpu[r] - float(l1.reshape(-1)[0])) <= 1e-3
    assert n_clear >= 0.9 * len(rows)
    say("  O max-abs", e_o, "over", n_clear, "rows")
    assert e_o <= 2e-2


def test_threshold_bounded_capacity():
    # count -> fill -> CSR forward enqueued with a capacity instead of the
    # count read back: with room to spare the same selection and output; with
    # too little room nothing is written past the capacity and the forward
    # sees each row's kept blocks below it
    w = SMALL["prefill_1088"]
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    rp, col, bias = ops.threshold_blocks(dev["qs"], dev["ks"], 0.01, w.tk)
    o, lse = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, col, bias)
    nnz = int(rp[-1].item())
    say("bounded capacity, nnz", nnz)
    cap = nnz + 777
    rp2, col2, bias2 = ops.threshold_blocks(dev["qs"], dev["ks"], 0.01, w.tk, capacity=cap)
    assert col2.numel() == cap
    o2, lse2 = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp2, col2, bias2)
    torch.cuda.synchronize()
    assert torch.equal(rp, rp2)
    assert torch.equal(col, col2[:nnz]) and torch.equal(bias, bias2[:nnz])
    assert max_abs(host(o2), host(o)) <= 2e-2 and max_abs(host(lse2), host(lse)) <= 1e-3
    say("  bit-equal output:", torch.equal(o, o2) and torch.equal(lse, lse2))
    # truncation: a sentinel-filled buffer longer than the capacity
    cap = nnz // 2
    sh = ops._thr_shape(dev["qs"], dev["ks"], w.tk, 64, None)
    colx = torch.full((cap + 256,), -7, dtype=torch.int32, device=DEV)
    biasx = torch.full((cap + 256,), 7.0, dtype=torch.float32, device=DEV)
    ops._check("sas_threshold_fill", ops.load().sas_threshold_fill(
        ops.ctypes.byref(sh), ops.ctypes.c_float(0.01), 0, ops._p(dev["qs"]), ops._p(dev["ks"]),
        ops._p(rp), ops.ctypes.c_int64(cap), ops._p(colx), ops._p(biasx), ops._stream(dev["qs"])))
    torch.cuda.synchronize()
    assert torch.equal(colx[:cap], col[:cap]) and torch.equal(biasx[:cap], bias[:cap])
    assert bool((colx[cap:] == -7).all()) and bool((biasx[cap:] == 7.0).all())
    # the forward over the truncated selection == the forward over the same
    # segments cut at the capacity
    o3, l3 = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, colx[:cap], biasx[:cap])
    rpc = torch.clamp(rp, max=cap)
    o4, l4 = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rpc, col[:cap].contiguous(),
                                bias[:cap].contiguous())
    torch.cuda.synchronize()
    assert max_abs(host(o3), host(o4)) <= 2e-2 and max_abs(host(l3), host(l4)) <= 1e-3
