"""Out-of-bounds write detection: every output and workspace of every entry
point sits inside a larger device buffer whose bands before and after it are
filled with a sentinel byte; after the call (through the C ABI) the bands
must be untouched, the inputs unchanged and the outputs equal to those of the
same call on exactly sized buffers.  Shapes are ragged where stray stores
would land: a last query tile of 8 rows (tq 520), query offsets that are not
multiples of 64 (56, 248), d 64, 4-token units in f32, 1- and 2-token units
in the bf16 training kernels, and paged sequences of 1, 65 and 128 tokens;
the fused selection + decode calls too.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
from gpu_common import DEV, inputs, say

pytestmark = pytest.mark.gpu

BAND = 4096  # sentinel bytes on each side (keeps 256-byte alignment)
PAT = 0xA5


class Guarded:
    """nbytes of device memory with a sentinel band before and after."""

    def __init__(self, nbytes: int):
        self.n = int(nbytes)
        self.buf = torch.full((self.n + 2 * BAND,), PAT, dtype=torch.uint8, device=DEV)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr() + BAND)

    def view(self, dtype, shape):
        return self.buf[BAND:BAND + self.n].view(dtype).view(shape)

    def bands_ok(self) -> bool:
        return bool((self.buf[:BAND] == PAT).all().item()
                    and (self.buf[BAND + self.n:] == PAT).all().item())


def guarded_like(t: torch.Tensor) -> Guarded:
    return Guarded(t.numel() * t.element_size())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_all(outs, refs, inputs_before, inputs_after, approx=()):
    torch.cuda.synchronize()
    for n, gbuf in outs.items():
        assert gbuf.bands_ok(), "sentinel band overwritten around " + n
    for n, ref in refs.items():
        got = outs[n].view(ref.dtype, ref.shape)
        if n in approx:
            assert torch.allclose(got.float(), ref.float(), rtol=1e-5, atol=1e-6), n
        else:
            assert torch.equal(got, ref), n
    for n in inputs_before:
        assert torch.equal(inputs_before[n], inputs_after[n]), "input changed: " + n


DENSE = {
    "tq520_off56_ds16": synth.WORKLOADS["train_8k"].with_(name="g1", batch=1, hq=4, hkv=2,
                                                          tq=520, tk=576, ds=16, topk=3),
    "tq200_off248": synth.WORKLOADS["train_8k"].with_(name="g2", batch=2, hq=4, hkv=2, tq=200,
                                                      tk=448, topk=4),
    "d64_tq200": synth.WORKLOADS["train_8k"].with_(name="g3", batch=1, hq=4, hkv=1, tq=200,
                                                   tk=448, d=64, ds=16, topk=2),
    "f32_b4_tq100": synth.WORKLOADS["tiny_fp32"].with_(name="g4", batch=1, hq=2, hkv=1, tq=100,
                                                       tk=192, block=4, topk=6),
    "tok_b1_tq520_off56": synth.WORKLOADS["train_8k"].with_(name="g5", batch=1, hq=4, hkv=2,
                                                            tq=520, tk=576, block=1, topk=5),
    "tok_b2_tq200_off248": synth.WORKLOADS["train_8k"].with_(name="g6", batch=1, hq=8, hkv=2,
                                                             tq=200, tk=448, block=2, topk=4),
}


@pytest.mark.parametrize("name", list(DENSE))
def test_guard_bands_dense_paths(name):
    w = DENSE[name]
    say("guard bands", name, w)
    lib = ops.load()
    cpu, dev, _ = inputs(w)
    keep = {n: t.clone() for n, t in dev.items()}
    sh = ops.shape_of(dev["q"], dev["k"], dev["qs"], dev["ks"], block=w.block)
    st = _stream()
    # references on exactly sized buffers
    lam, beta = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=w.block, with_bias=True)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=w.block)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam,
                     block=w.block)
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk, block=w.block)
    bidx, bbias = ops.topk_blocks_budget(dev["qs"], dev["ks"], w.topk + 1, 0.25, w.tk,
                                         block=w.block, renorm=1)
    os_, ls_ = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], idx, bias, block=w.block)
    rp, col, tb = ops.threshold_blocks(dev["qs"], dev["ks"], 0.02, w.tk, block=w.block)
    of, lf, fi, fb = ops.topk_decode(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], w.topk,
                                     block=w.block)
    torch.cuda.synchronize()

    # gate
    G = {"lam": guarded_like(lam), "beta": guarded_like(beta)}
    assert lib.sas_gate_scores(ctypes.byref(sh), _p(dev["qs"]), _p(dev["ks"]), G["lam"].ptr,
                               G["beta"].ptr, st) == 0
    _check_all(G, {"lam": lam, "beta": beta}, keep, dev)
    # forward
    G = {"o": guarded_like(o), "lse": guarded_like(lse)}
    assert lib.sas_attn_fwd(ctypes.byref(sh), _p(dev["q"]), _p(dev["k"]), _p(dev["v"]),
                            _p(dev["qs"]), _p(dev["ks"]), _p(lam), G["o"].ptr, G["lse"].ptr,
                            st) == 0
    _check_all(G, {"o": o, "lse": lse}, keep, dev)
    # backward, with the workspace guarded too (size from the query)
    need = ops.bwd_workspace_bytes(sh, True)
    G = {n: guarded_like(g[n]) for n in ("dq", "dk", "dv", "dqs", "dks", "dz")}
    G["ws"] = Guarded(need)
    n = ctypes.c_size_t(need)
    assert lib.sas_attn_bwd(ctypes.byref(sh), _p(dev["q"]), _p(dev["k"]), _p(dev["v"]), _p(o),
                            _p(dev["dout"]), _p(lse), _p(dev["qs"]), _p(dev["ks"]), _p(lam),
                            G["dq"].ptr, G["dk"].ptr, G["dv"].ptr, G["dqs"].ptr, G["dks"].ptr,
                            G["dz"].ptr, G["ws"].ptr, ctypes.byref(n), st) == 0
    _check_all(G, {k: g[k] for k in ("dq", "dk", "dv", "dqs", "dks", "dz")}, keep, dev,
               approx=("dks",))
    # top-K and the budgeted top-K
    G = {"idx": guarded_like(idx), "bias": guarded_like(bias)}
    assert lib.sas_topk_blocks(ctypes.byref(sh), w.topk, 0, _p(dev["qs"]), _p(dev["ks"]),
                               G["idx"].ptr, G["bias"].ptr, st) == 0
    _check_all(G, {"idx": idx, "bias": bias}, keep, dev)
    G = {"idx": guarded_like(bidx), "bias": guarded_like(bbias)}
    assert lib.sas_topk_blocks_budget(ctypes.byref(sh), w.topk + 1, 1, 4, 1, _p(dev["qs"]),
                                      _p(dev["ks"]), G["idx"].ptr, G["bias"].ptr, st) == 0
    _check_all(G, {"idx": bidx, "bias": bbias}, keep, dev)
    # sparse forward (guarded workspace)
    need = ops.sparse_workspace_bytes(sh, w.topk)
    G = {"o": guarded_like(os_), "lse": guarded_like(ls_), "ws": Guarded(need)}
    n = ctypes.c_size_t(need)
    assert lib.sas_sparse_fwd(ctypes.byref(sh), w.topk, _p(dev["q"]), _p(dev["k"]), _p(dev["v"]),
                              _p(idx), _p(bias), G["o"].ptr, G["lse"].ptr, G["ws"].ptr,
                              ctypes.byref(n), st) == 0
    _check_all(G, {"o": os_, "lse": ls_}, keep, dev)
    # selection and decode in one launch (every row of the call)
    G = {"o": guarded_like(of), "lse": guarded_like(lf), "idx": guarded_like(fi),
         "bias": guarded_like(fb)}
    assert lib.sas_topk_decode(ctypes.byref(sh), w.topk, 0, _p(dev["q"]), _p(dev["k"]),
                               _p(dev["v"]), _p(dev["qs"]), _p(dev["ks"]), G["idx"].ptr,
                               G["bias"].ptr, G["o"].ptr, G["lse"].ptr, st) == 0
    _check_all(G, {"o": of, "lse": lf, "idx": fi, "bias": fb}, keep, dev)
    # threshold count / fill and the CSR forward (64-token units, bf16 only)
    nnz = int(col.numel())
    if w.block == 64 and w.dtype == "bf16":
        nws = ctypes.c_size_t(0)
        assert lib.sas_threshold_count(ctypes.byref(sh), ctypes.c_float(0.02), None, None, None,
                                       None, ctypes.byref(nws), st) == 0
        G = {"row_ptr": guarded_like(rp), "ws": Guarded(nws.value)}
        assert lib.sas_threshold_count(ctypes.byref(sh), ctypes.c_float(0.02), _p(dev["qs"]),
                                       _p(dev["ks"]), G["row_ptr"].ptr, G["ws"].ptr,
                                       ctypes.byref(nws), st) == 0
        _check_all(G, {"row_ptr": rp}, keep, dev)
        G = {"col": Guarded(4 * nnz), "bias": Guarded(4 * nnz)}
        assert lib.sas_threshold_fill(ctypes.byref(sh), ctypes.c_float(0.02), 0, _p(dev["qs"]),
                                      _p(dev["ks"]), _p(rp), ctypes.c_int64(nnz), G["col"].ptr,
                                      G["bias"].ptr, st) == 0
        _check_all(G, {"col": col, "bias": tb}, keep, dev)
        oc, lc = ops.sparse_fwd_csr(dev["q"], dev["k"], dev["v"], rp, col, tb)
        torch.cuda.synchronize()
        need = ops.sparse_csr_workspace_bytes(sh, nnz)
        G = {"o": guarded_like(oc), "lse": guarded_like(lc), "ws": Guarded(need)}
        n = ctypes.c_size_t(need)
        assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), ctypes.c_int64(nnz), _p(rp), _p(col),
                                      _p(tb), _p(dev["q"]), _p(dev["k"]), _p(dev["v"]),
                                      G["o"].ptr, G["lse"].ptr, G["ws"].ptr, ctypes.byref(n),
                                      st) == 0
        _check_all(G, {"o": oc, "lse": lc}, keep, dev)


def test_guard_bands_paged():
    pw = synth.PAGED_WORKLOADS["decode_paged_mix"].with_(batch=4, hq=8, hkv=2, max_len=4096,
                                                         topk=3)
    t = synth.draw_paged(pw, lens=[1, 65, 128, 4096])
    d = {n: x.to(DEV) for n, x in t.items()}
    lib = ops.load()
    pages, hkv, _, dd = d["k_pool"].shape
    sh = ops.make_paged_shape(pw.batch, pw.hq, pw.hkv, pw.d, pw.ds, pw.max_blocks, pages,
                              dtype=ops.SAS_BF16)
    st = _stream()
    keep = {n: x.clone() for n, x in d.items()}
    idx, bias = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    o, lse = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    of, lf, fi, fb = ops.paged_topk_decode(d["q"], d["k_pool"], d["v_pool"], d["qs"],
                                           d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    torch.cuda.synchronize()
    G = {"o": guarded_like(of), "lse": guarded_like(lf), "idx": guarded_like(fi),
         "bias": guarded_like(fb)}
    assert lib.sas_paged_topk_decode(ctypes.byref(sh), pw.topk, 0, _p(d["seq_len"]),
                                     _p(d["block_table"]), _p(d["q"]), _p(d["k_pool"]),
                                     _p(d["v_pool"]), _p(d["qs"]), _p(d["ks_pool"]), G["idx"].ptr,
                                     G["bias"].ptr, G["o"].ptr, G["lse"].ptr, st) == 0
    _check_all(G, {"o": of, "lse": lf, "idx": fi, "bias": fb}, keep, d)
    G = {"idx": guarded_like(idx), "bias": guarded_like(bias)}
    assert lib.sas_paged_topk(ctypes.byref(sh), pw.topk, 0, _p(d["seq_len"]),
                              _p(d["block_table"]), _p(d["qs"]), _p(d["ks_pool"]), G["idx"].ptr,
                              G["bias"].ptr, st) == 0
    _check_all(G, {"idx": idx, "bias": bias}, keep, d)
    need = ops.paged_workspace_bytes(sh, pw.topk)
    G = {"o": guarded_like(o), "lse": guarded_like(lse), "ws": Guarded(need)}
    n = ctypes.c_size_t(need)
    assert lib.sas_paged_decode(ctypes.byref(sh), pw.topk, _p(d["seq_len"]), _p(d["block_table"]),
                                _p(d["q"]), _p(d["k_pool"]), _p(d["v_pool"]), _p(idx), _p(bias),
                                G["o"].ptr, G["lse"].ptr, G["ws"].ptr, ctypes.byref(n), st) == 0
    _check_all(G, {"o": o, "lse": lse}, keep, d)
    # append into guarded pools: the pools are outputs here, every other byte of
    # them must keep its value
    kp, vp, ksp = (Guarded(x.numel() * x.element_size()) for x in
                   (d["k_pool"], d["v_pool"], d["ks_pool"]))
    for gbuf, x in ((kp, d["k_pool"]), (vp, d["v_pool"]), (ksp, d["ks_pool"])):
        gbuf.view(x.dtype, x.shape).copy_(x)
    pos = (d["seq_len"] - 1).clamp(min=0).to(torch.int32)  # the last cached token of each
    pos[1] = 63  # completes a block: the selector key is written too
    kn = torch.randn(pw.batch, pw.hkv, pw.d, device=DEV).to(torch.bfloat16)
    vn = torch.randn(pw.batch, pw.hkv, pw.d, device=DEV).to(torch.bfloat16)
    ksn = torch.randn(pw.batch, pw.kheads, pw.ds, device=DEV).to(torch.bfloat16)
    ash = ops.make_paged_shape(pw.batch, pw.hkv, pw.hkv, pw.d, pw.ds, pw.max_blocks, pages,
                               pw.kheads, dtype=ops.SAS_BF16)
    assert lib.sas_paged_append(ctypes.byref(ash), _p(pos), _p(d["block_table"]), _p(kn), _p(vn),
                                _p(ksn), kp.ptr, vp.ptr, ksp.ptr, st) == 0
    ref_k, ref_v, ref_ks = d["k_pool"].clone(), d["v_pool"].clone(), d["ks_pool"].clone()
    ops.paged_append(pos, d["block_table"], kn, vn, ref_k, ref_v, ksn, ref_ks)
    torch.cuda.synchronize()
    for gbuf, ref in ((kp, ref_k), (vp, ref_v), (ksp, ref_ks)):
        assert gbuf.bands_ok()
        assert torch.equal(gbuf.view(ref.dtype, ref.shape), ref)
