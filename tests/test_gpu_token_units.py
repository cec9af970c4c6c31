"""bf16 training with context units of 1, 2, 4 and 8 tokens against the oracle.

The gate, forward and backward of the MFMA kernels when the gate bias changes
from key to key inside a 64-key tile (NeurIPS abstract: a query selects a
small set of context units, tokens or blocks; here every unit is active, as
in training).  Small shapes are compared over whole tensors: lam, O and lse
element-wise, every gradient (dq, dk, dv, dz, dqs, dks) by its relative L2
and by a bound per row.  Shapes cover kv groups of 4 heads, a query offset,
a ragged last query tile, selector heads finer and coarser than the kv heads
(the dK/dV kernel then changes selector head between query heads, or several
workgroups add into one dks row), explicit scales and large logits.  At 32k
(token units, the full training workload) sampled query rows, keys of the
first blocks and of the middle of kv group 0 (all 4 x 32768 rows reach them)
and selector rows are compared, without the dense dz.
Bars as for 64-token units: O max-abs <= 2e-2, lse <= 1e-3, gradients rel-L2
<= 5e-2 and every row within 0.1 of its norm.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import (check_train, gpu_train, host, inputs, max_abs, oshape, rel_l2, row_bound,
                        sample_rows, say)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
BASE = W["train_8k"]
SMALL = {
    "gqa_576": dict(batch=2, hq=8, hkv=2, tq=576, tk=576),
    "q_offset": dict(batch=1, hq=4, hkv=1, tq=160, tk=1024),
    "ragged_q": dict(batch=1, hq=4, hkv=2, tq=200, tk=448),
    "hks_fine": dict(batch=1, hq=8, hkv=2, hks=4, tq=320, tk=320),
    "hks_coarse": dict(batch=1, hq=8, hkv=4, hks=1, tq=384, tk=384),
}


@pytest.mark.parametrize("blk", [1, 2, 4, 8])
@pytest.mark.parametrize("name", list(SMALL))
def test_token_units_train(name, blk):
    w = BASE.with_(name="%s_b%d" % (name, blk), block=blk, **SMALL[name])
    say("token units train", name, blk)
    cpu, dev, f = inputs(w)
    lam, o, lse, g = gpu_train(dev, w)
    check_train(w, f, lam, o, lse, g, oshape(w))
    dz = host(g["dz"])
    c = (np.arange(w.tq) + w.tk - w.tq) // blk
    for i in range(w.tq):
        assert np.all(dz[:, :, i, c[i]:] == 0.0)


@pytest.mark.parametrize("blk,name,sm,sel", [
    (1, "scales", 0.3, 2.0),
    (4, "large_logits", None, None),
])
def test_token_units_stressed(blk, name, sm, sel):
    w = BASE.with_(name=name, batch=1, hq=8, hkv=2, tq=448, tk=512, block=blk)
    if name == "large_logits":
        w = w.with_(scales={"q": 2.0, "k": 2.0, "v": 0.5})
    say("token units stressed", name, blk)
    cpu, dev, f = inputs(w)
    S = oshape(w)
    if sm is not None:
        S = oracle.OracleShape(w.batch, w.hq, w.hkv, w.tq, w.tk, w.d, w.ds, w.block,
                               hks=w.kheads, sm_scale=float(np.float32(sm)),
                               sel_scale=float(np.float32(sel)))
    lam, o, lse, g = gpu_train(dev, w, sm, sel)
    check_train(w, f, lam, o, lse, g, S)


@pytest.mark.parametrize("d,ds", [(128, 16), (128, 64), (64, 32)])
@pytest.mark.parametrize("blk", [1, 8])
def test_token_units_fwd_other_dims(d, ds, blk):
    # the forward takes every (d, ds); the backward of these units needs d = 128, ds = 32
    w = BASE.with_(name="fwd_d%d_ds%d" % (d, ds), batch=1, hq=4, hkv=2, tq=300, tk=512, d=d,
                   ds=ds, block=blk)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(oshape(w), f["q"], f["k"], f["v"], f["qs"], f["ks"])
    e = max_abs(host(o), o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse), l_ref) <= 1e-3


def test_token_units_bwd_unsupported_selector_width():
    w = BASE.with_(batch=1, hq=2, hkv=1, tq=128, tk=128, ds=16, block=4)
    cpu, dev, f = inputs(w)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=4)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=4)
    with pytest.raises(RuntimeError, match="not supported"):
        ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"],
                     lam, block=4)


def test_token_units_dz_optional_same_grads():
    w = BASE.with_(batch=1, hq=8, hkv=2, tq=576, tk=576, block=2)
    cpu, dev, f = inputs(w)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=2)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=2)
    args = (dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam)
    g1 = ops.attn_bwd(*args, block=2, with_dz=True)
    g2 = ops.attn_bwd(*args, block=2, with_dz=False)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dqs"):
        assert torch.equal(g1[n], g2[n]), n
    # dks sums fp32 atomics: equal up to their order
    assert rel_l2(host(g2["dks"]), host(g1["dks"])) <= 1e-5


@pytest.mark.timeout(900)
@pytest.mark.parametrize("blk", [1, 8])
def test_token_units_full_size_sampled(blk):
    w = W["train_32k"].with_(name="train_32k_b%d" % blk, block=blk)
    say("token units 32k", blk)
    cpu, dev, _ = inputs(w)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=blk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=blk)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam,
                     block=blk, with_dz=False)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dqs", "dks"):
        assert torch.isfinite(g[n]).all().item(), n
    # kv group 0 (query heads 0 .. 3): rows of every head, keys of the first
    # two 64-key tiles and of the middle one, selector rows at the same places
    hpg = w.hq // w.hkv
    pick = {"q": slice(0, hpg), "qs": slice(0, hpg), "dout": slice(0, hpg), "k": slice(0, 1),
            "v": slice(0, 1), "ks": slice(0, 1)}
    f = {n: synth.to_f64(cpu[n][:, pick[n]].contiguous()) for n in pick}
    S = oracle.OracleShape(1, hpg, 1, w.tq, w.tk, w.d, w.ds, blk, hks=1)
    w1 = w.with_(hq=hpg, hkv=1)
    rows = sample_rows(w1, 24, seed=23)
    tiles = (0, 1, w.tk // 128)
    keys = np.array([u for j in tiles for u in range(64 * j, 64 * j + 64, 3)], dtype=np.int64)
    units = np.unique(keys // blk)
    o_ref, l_ref = oracle.attn_fwd(S, f["q"], f["k"], f["v"], f["qs"], f["ks"], rows=rows)
    og = host(o[:, :hpg]).reshape(-1, w.d)[rows]
    e = max_abs(og, o_ref)
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse[:, :hpg]).reshape(-1)[rows], l_ref) <= 1e-3
    ref = oracle.attn_bwd(S, f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"], rows=rows,
                          keys=keys, sblocks=units)
    got = {
        "dq": host(g["dq"][:, :hpg]).reshape(-1, w.d)[rows],
        "dqs": host(g["dqs"][:, :hpg]).reshape(-1, w.ds)[rows],
        "dk": host(g["dk"][0, 0])[keys],
        "dv": host(g["dv"][0, 0])[keys],
        "dks": host(g["dks"][0, 0])[units],
    }
    for n in got:
        e = rel_l2(got[n], ref[n])
        say("  %s rel-L2 %.3e" % (n, e))
        assert e <= 5e-2, n
    for n in ("dk", "dv", "dks"):
        row_bound(n, got[n], ref[n])
