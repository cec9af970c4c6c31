"""GPU backward vs fp64 oracle: dq, dk, dv, dz, dqs, dks.

Bar: relative L2 <= 5e-2 per gradient tensor (bf16); dz is also checked
against the exact structure (zero for j >= c(t)).
"""

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, inputs, max_abs, oshape, rel_l2, sample_rows, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
SMALL = {
    "gqa_576": W["train_8k"].with_(name="gqa_576", batch=2, hq=8, hkv=2, tq=576, tk=576),
    "q_offset": W["train_8k"].with_(name="q_offset", batch=1, hq=4, hkv=1, tq=160, tk=1024),
    "ragged_q": W["train_8k"].with_(name="ragged_q", batch=1, hq=4, hkv=2, tq=200, tk=448),
    "d64_ds16": W["train_8k"].with_(name="d64_ds16", batch=1, hq=4, hkv=2, tq=448, tk=448, d=64,
                                    ds=16),
    "ds64_hks": W["train_8k"].with_(name="ds64_hks", batch=1, hq=4, hkv=2, hks=4, tq=320,
                                    tk=320, ds=64),
    "one_block": W["train_8k"].with_(name="one_block", batch=1, hq=2, hkv=1, tq=64, tk=64),
    # d = 128 with a 16-dim selector: three 256-row dQ workgroups, the last
    # with 8 rows, and a query offset of 56
    "ds16_q520": W["train_8k"].with_(name="ds16_q520", batch=1, hq=4, hkv=2, tq=520, tk=576,
                                     ds=16),
}


def _gpu_fwd_bwd(dev, w, with_dz=True):
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"],
                     lam, with_dz=with_dz)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd_small_full(name):
    w = SMALL[name]
    say("bwd", name, w)
    cpu, dev, f = inputs(w)
    g = _gpu_fwd_bwd(dev, w)
    ref = oracle.attn_bwd(oshape(w), f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"])
    for n in ("dq", "dk", "dv", "dz", "dqs", "dks"):
        e = rel_l2(host(g[n]), ref[n])
        say("  %s rel-L2 %.3e" % (n, e))
        assert e <= 5e-2, n
    dz = host(g["dz"])
    c = (np.arange(w.tq) + w.tk - w.tq) // 64
    for i in range(w.tq):
        assert np.all(dz[:, :, i, c[i]:] == 0.0)
    assert np.allclose(dz.sum(-1), 0.0, atol=5e-2 * np.abs(dz).max() + 1e-6)


def test_bwd_dz_in_workspace_gives_same_dks():
    w = SMALL["gqa_576"]
    cpu, dev, f = inputs(w)
    g1 = _gpu_fwd_bwd(dev, w, with_dz=True)
    g2 = _gpu_fwd_bwd(dev, w, with_dz=False)
    for n in ("dq", "dk", "dv", "dqs"):
        assert torch.equal(g1[n], g2[n]), n
    assert rel_l2(host(g2["dks"]), host(g1["dks"])) <= 1e-6


def test_bwd_deterministic():
    w = SMALL["gqa_576"]
    cpu, dev, f = inputs(w)
    g1 = _gpu_fwd_bwd(dev, w)
    g2 = _gpu_fwd_bwd(dev, w)
    for n in ("dq", "dk", "dv", "dz", "dqs"):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("name", ["train_8k", "train_32k"])
def test_bwd_full_size_sampled(name):
    w = W[name]
    say("bwd full", name)
    cpu, dev, f = inputs(w)
    g = _gpu_fwd_bwd(dev, w)
    rows = sample_rows(w, 24, seed=11)
    # keys of the last two blocks of every kv head (their rows are cheap to sum)
    keys = np.array([(b * w.hkv + kh) * w.tk + u for b in range(w.batch) for kh in range(w.hkv)
                     for u in range(w.tk - 128, w.tk, 7)], dtype=np.int64)
    sblk = np.array([(b * w.kheads + s) * w.nb + j for b in range(w.batch)
                     for s in range(w.kheads) for j in (w.nb - 2, w.nb - 3)], dtype=np.int64)
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
    for n in ("dq", "dk", "dv", "dqs", "dks"):
        assert torch.isfinite(g[n]).all().item(), n
