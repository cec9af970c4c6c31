"""GPU fp32 path (the tiny fp32 workload: T=512, d=64, one head) vs the oracle.

Bar for fp32: max-abs <= 1e-4 on outputs, relative L2 <= 1e-4 on gradients,
top-K indices bit-exact on tie-free rows.
"""

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, inputs, max_abs, oshape, rel_l2, say, tie_free_rows

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_fp32"]
GQA = TINY.with_(name="tiny_gqa", batch=2, hq=4, hkv=2, tq=320, tk=384)


@pytest.mark.parametrize("w", [TINY, GQA], ids=["tiny_fp32", "tiny_gqa"])
def test_f32_fwd_bwd(w):
    say("f32", w.name)
    cpu, dev, f = inputs(w)
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam)
    torch.cuda.synchronize()
    S = oshape(w)
    o_ref, l_ref = oracle.attn_fwd(S, f["q"], f["k"], f["v"], f["qs"], f["ks"])
    say("  O max-abs", max_abs(host(o), o_ref))
    assert max_abs(host(o), o_ref) <= 1e-4
    assert max_abs(host(lse), l_ref) <= 1e-4
    ref = oracle.attn_bwd(S, f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"])
    for n in ("dq", "dk", "dv", "dz", "dqs", "dks"):
        e = rel_l2(host(g[n]), ref[n])
        say("  %s rel-L2 %.2e max-abs %.2e" % (n, e, max_abs(host(g[n]), ref[n])))
        assert e <= 1e-4, n


def test_f32_topk_sparse():
    w = TINY.with_(topk=3)
    cpu, dev, f = inputs(w, ("q", "k", "v", "qs", "ks"))
    idx, bias = ops.topk_blocks(dev["qs"], dev["ks"], w.topk, w.tk)
    torch.cuda.synchronize()
    S = oshape(w)
    idx_ref, bias_ref = oracle.topk_blocks(S, w.topk, f["qs"], f["ks"])
    z, _, _ = oracle.gate_scores(S, f["qs"], f["ks"])
    ok = tie_free_rows(z.reshape(-1, w.nb), (np.arange(w.tq)) // 64, w.topk)
    assert np.array_equal(idx.cpu().numpy().reshape(-1, 3)[ok], idx_ref.reshape(-1, 3)[ok])
    o, lse = ops.sparse_fwd(dev["q"], dev["k"], dev["v"], torch.from_numpy(idx_ref).to(DEV),
                            torch.from_numpy(bias_ref.astype(np.float32)).to(DEV))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_fwd(S, 3, f["q"], f["k"], f["v"], idx_ref,
                                     bias_ref.astype(np.float32).astype(np.float64))
    assert max_abs(host(o), o_ref) <= 1e-4
    assert max_abs(host(lse), l_ref) <= 1e-4
