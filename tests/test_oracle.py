"""Pins of the fp64 CPU oracle against things other than itself.

* brute force: the whole bias matrix + torch ``scaled_dot_product_attention``
  and autograd (``bruteforce.py``), on tiny shapes;
* special cases that reduce to textbook attention (no history, dominant block);
* closed forms (zero query => L = log(B + n_cur), uniform gate => -log c);
* central finite differences of the oracle's own forward;
* invariants (shift of the scores, sum of dz, GQA == repeated MHA,
  sparse == dense when the budget covers every block, decode == last prefill row).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp, softmax

import bruteforce as bf
from oracle import OracleShape
import oracle

RNG = np.random.default_rng(1234)


def make(batch=1, hq=2, hkv=1, tq=40, tk=40, d=8, ds=4, block=8, hks=None, seed=0, qscale=0.7):
    rng = np.random.default_rng(seed)
    hks_ = hks if hks else hkv
    nb = (tk + block - 1) // block
    x = dict(
        q=rng.standard_normal((batch, hq, tq, d)) * qscale,
        k=rng.standard_normal((batch, hkv, tk, d)) * qscale,
        v=rng.standard_normal((batch, hkv, tk, d)),
        qs=rng.standard_normal((batch, hq, tq, ds)),
        ks=rng.standard_normal((batch, hks_, nb, ds)),
        dout=rng.standard_normal((batch, hq, tq, d)),
    )
    S = OracleShape(batch, hq, hkv, tq, tk, d, ds, block, hks=hks)
    return S, x


def T(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


SHAPES = [
    dict(),                                           # MHA-like 2 heads on 1 kv head
    dict(hq=4, hkv=2, tq=37, tk=37, block=8),         # GQA 2:1, ragged last block
    dict(hq=4, hkv=1, tq=33, tk=33, block=4),         # GQA 4:1
    dict(hq=4, hkv=2, hks=4, tq=24, tk=24, block=2),  # selector keys per query head
    dict(batch=2, hq=2, hkv=2, tq=16, tk=16, block=1),  # token-level units
    dict(hq=2, hkv=1, tq=9, tk=30, block=8),          # queries at the end (q_off > 0)
    dict(hq=2, hkv=2, tq=1, tk=29, block=4),          # one decode-like row
]


# ---------------------------------------------------------------- gate scores
def test_gate_scores_vs_numpy():
    S, x = make(hq=4, hkv=2, tq=37, tk=37, block=8)
    z, lam, beta = oracle.gate_scores(S, x["qs"], x["ks"])
    ksr = np.repeat(x["ks"], 2, axis=1)
    zref = np.einsum("bhte,bhje->bhtj", x["qs"], ksr) / math.sqrt(S.ds)
    c = (np.arange(S.tq) + S.tk - S.tq) // S.block
    for t in range(S.tq):
        h = slice(0, c[t])
        np.testing.assert_allclose(z[..., t, h], zref[..., t, h], rtol=1e-13, atol=1e-13)
        assert np.all(np.isneginf(z[..., t, c[t]:]))
        if c[t] == 0:
            assert np.all(np.isneginf(lam[..., t]))
        else:
            np.testing.assert_allclose(lam[..., t], logsumexp(zref[..., t, h], axis=-1), rtol=1e-13)
            np.testing.assert_allclose(np.exp(beta[..., t, h]).sum(-1), 1.0, rtol=1e-13)
        if c[t] < S.nb:
            assert np.all(beta[..., t, c[t]] == 0.0)
        assert np.all(np.isneginf(beta[..., t, c[t] + 1:]))


def test_gate_uniform_when_keys_zero():
    S, x = make(tq=40, tk=40, block=8)
    x["ks"][:] = 0.0
    _, lam, beta = oracle.gate_scores(S, x["qs"], x["ks"])
    for t in range(S.tq):
        c = t // S.block
        for j in range(c):
            np.testing.assert_allclose(beta[..., t, j], -math.log(c), rtol=1e-14)
        if c >= 1:
            np.testing.assert_allclose(lam[..., t], math.log(c), rtol=1e-14)


def test_single_history_block_has_zero_bias():
    S, x = make(tq=40, tk=40, block=8)
    _, _, beta = oracle.gate_scores(S, x["qs"], x["ks"])
    assert np.all(beta[..., 8:16, 0] == 0.0)  # c = 1 -> softmax over one block


# ------------------------------------------------------------------- forward
@pytest.mark.parametrize("kw", SHAPES)
def test_fwd_vs_bruteforce(kw):
    S, x = make(**kw)
    o, lse = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    ob, lb = bf.gated(T(x["q"]), T(x["k"]), T(x["v"]), T(x["qs"]), T(x["ks"]), block=S.block)
    np.testing.assert_allclose(o, ob.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lb.numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_short_sequence_is_plain_causal():
    # T <= 2B: block 0 has no history, block 1 has one block with bias 0.
    S, x = make(hq=4, hkv=2, tq=16, tk=16, block=8)
    o, _ = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    kr = T(x["k"]).repeat_interleave(2, dim=1)
    vr = T(x["v"]).repeat_interleave(2, dim=1)
    ref = F.scaled_dot_product_attention(T(x["q"]), kr, vr, is_causal=True)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_zero_query_closed_form():
    # q = 0: logits are the bias only; weights g_j per historical key, 1 per
    # current key, so L = log(B + n_cur) (log n_cur without history) and
    # O = (sum_j g_j sum_{u in j} v_u + sum_cur v_u) / (B + n_cur).
    S, x = make(hq=2, hkv=1, tq=37, tk=37, block=8)
    x["q"][:] = 0.0
    o, lse = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    B = S.block
    for h in range(S.hq):
        for t in range(S.tq):
            c, ncur = t // B, t % B + 1
            v = x["v"][0, 0]
            if c == 0:
                np.testing.assert_allclose(lse[0, h, t], math.log(ncur), rtol=1e-14)
                ref = v[:t + 1].sum(0) / ncur
            else:
                z = x["qs"][0, h, t] @ x["ks"][0, 0, :c].T / math.sqrt(S.ds)
                g = softmax(z)
                np.testing.assert_allclose(lse[0, h, t], math.log(B + ncur), rtol=1e-14)
                hist = sum(g[j] * v[j * B:(j + 1) * B].sum(0) for j in range(c))
                ref = (hist + v[c * B:t + 1].sum(0)) / (B + ncur)
            np.testing.assert_allclose(o[0, h, t], ref, rtol=1e-12, atol=1e-13)


def test_fwd_dominant_block_is_masked_attention():
    # Scores-in with one block at 0 and the rest at -1e4: the gate is one-hot,
    # so each row attends exactly that block (bias 0) plus its current block.
    S, x = make(hq=2, hkv=1, tq=40, tk=40, block=8)
    nb = S.nb
    z = np.full((1, S.hq, S.tq, nb), -1e4)
    pick = np.zeros((S.hq, S.tq), dtype=int)
    for h in range(S.hq):
        for t in range(S.tq):
            c = t // S.block
            if c:
                pick[h, t] = RNG.integers(0, c)
                z[0, h, t, pick[h, t]] = 0.0
    o, _ = oracle.attn_fwd(S, x["q"], x["k"], x["v"], z=z)
    mask = torch.zeros(1, S.hq, S.tq, S.tk, dtype=torch.bool)
    for h in range(S.hq):
        for t in range(S.tq):
            c = t // S.block
            mask[0, h, t, c * S.block:t + 1] = True
            if c:
                mask[0, h, t, pick[h, t] * S.block:(pick[h, t] + 1) * S.block] = True
    ref = F.scaled_dot_product_attention(T(x["q"]), T(x["k"]).expand(1, 2, -1, -1),
                                         T(x["v"]).expand(1, 2, -1, -1), attn_mask=mask)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_score_shift_invariance():
    S, x = make(hq=2, hkv=1, tq=40, tk=40, block=8)
    z, _, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    z = np.where(np.isneginf(z), 0.0, z)
    a = RNG.standard_normal((1, S.hq, S.tq, 1)) * 5
    o1, l1 = oracle.attn_fwd(S, x["q"], x["k"], x["v"], z=z)
    o2, l2 = oracle.attn_fwd(S, x["q"], x["k"], x["v"], z=z + a)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
    # the same through the selector vectors: qs' = [qs, a/sigma], ks' = [ks, 1]
    sig = 1.0 / math.sqrt(S.ds)
    S2 = OracleShape(1, 2, 1, 40, 40, S.d, S.ds + 1, 8, sel_scale=sig)
    qs2 = np.concatenate([x["qs"], np.broadcast_to(a / sig, (1, 2, 40, 1))], axis=-1)
    ks2 = np.concatenate([x["ks"], np.ones((1, 1, S.nb, 1))], axis=-1)
    o3, _ = oracle.attn_fwd(S2, x["q"], x["k"], x["v"], qs2, ks2)
    np.testing.assert_allclose(o1, o3, rtol=1e-11, atol=1e-12)


def test_fwd_gqa_equals_repeated_mha():
    S, x = make(hq=4, hkv=2, tq=30, tk=30, block=4)
    o, l = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    S2 = OracleShape(1, 4, 4, 30, 30, S.d, S.ds, 4)
    rep = lambda a: np.repeat(a, 2, axis=1)
    o2, l2 = oracle.attn_fwd(S2, x["q"], rep(x["k"]), rep(x["v"]), x["qs"], rep(x["ks"]))
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_fwd_rows_subset_matches_full():
    S, x = make(hq=4, hkv=2, tq=37, tk=37, block=8)
    o, l = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    rows = np.array([0, 5, 36, 37 + 12, 3 * 37 + 36])
    os_, ls_ = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"], rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, S.d)[rows])
    np.testing.assert_array_equal(ls_, l.reshape(-1)[rows])


# ------------------------------------------------------------------ backward
@pytest.mark.parametrize("kw", SHAPES)
def test_bwd_vs_autograd(kw):
    S, x = make(**kw)
    g = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"])
    ref = bf.grads(T(x["q"]), T(x["k"]), T(x["v"]), T(x["dout"]), T(x["qs"]), T(x["ks"]),
                   block=S.block)
    for n in ("q", "k", "v", "qs", "ks"):
        np.testing.assert_allclose(g["d" + n], ref[n].numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


@pytest.mark.parametrize("kw", SHAPES[:4])
def test_bwd_dz_vs_autograd_scores_in(kw):
    S, x = make(**kw)
    z, _, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    z = np.where(np.isneginf(z), RNG.standard_normal(z.shape), z)  # unused entries: arbitrary
    g = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], z=z)
    ref = bf.grads(T(x["q"]), T(x["k"]), T(x["v"]), T(x["dout"]), z=T(z), block=S.block)
    np.testing.assert_allclose(g["dz"], ref["z"].numpy(), rtol=1e-9, atol=1e-11)
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(g["d" + n], ref[n].numpy(), rtol=1e-9, atol=1e-11)


def _loss(S, x, z=None):
    if z is None:
        o, _ = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    else:
        o, _ = oracle.attn_fwd(S, x["q"], x["k"], x["v"], z=z)
    return float((o * x["dout"]).sum())


def test_bwd_finite_differences():
    S, x = make(hq=4, hkv=2, tq=21, tk=21, block=4, d=4, ds=3)
    g = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"])
    h = 1e-6
    rng = np.random.default_rng(7)
    for n in ("q", "k", "v", "qs", "ks"):
        for _ in range(6):
            ix = tuple(rng.integers(0, m) for m in x[n].shape)
            xp = {a: b.copy() for a, b in x.items()}
            xm = {a: b.copy() for a, b in x.items()}
            xp[n][ix] += h
            xm[n][ix] -= h
            fd = (_loss(S, xp) - _loss(S, xm)) / (2 * h)
            assert abs(fd - g["d" + n][ix]) <= 1e-6 * max(1.0, abs(fd)), (n, ix, fd, g["d" + n][ix])
    z, _, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    z = np.where(np.isneginf(z), 0.0, z)
    gz = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], z=z)["dz"]
    for _ in range(10):
        b_, hh, t = 0, rng.integers(0, S.hq), rng.integers(S.block, S.tq)
        j = rng.integers(0, t // S.block)
        zp, zm = z.copy(), z.copy()
        zp[b_, hh, t, j] += h
        zm[b_, hh, t, j] -= h
        fd = (_loss(S, x, zp) - _loss(S, x, zm)) / (2 * h)
        assert abs(fd - gz[b_, hh, t, j]) <= 1e-6 * max(1.0, abs(fd))


def test_bwd_dz_rows_sum_to_zero_and_shift_invariant():
    S, x = make(hq=2, hkv=1, tq=40, tk=40, block=8)
    z, _, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    z = np.where(np.isneginf(z), 0.0, z)
    dz = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], z=z)["dz"]
    np.testing.assert_allclose(dz.sum(-1), 0.0, atol=1e-13)
    for t in range(S.tq):
        assert np.all(dz[..., t, t // S.block:] == 0.0)
    a = RNG.standard_normal((1, S.hq, S.tq, 1)) * 3
    dz2 = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], z=z + a)["dz"]
    np.testing.assert_allclose(dz, dz2, rtol=1e-9, atol=1e-12)


def test_bwd_gqa_dkdv_is_sum_of_heads():
    S, x = make(hq=4, hkv=2, tq=30, tk=30, block=4)
    g = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"])
    S2 = OracleShape(1, 4, 4, 30, 30, S.d, S.ds, 4)
    rep = lambda a: np.repeat(a, 2, axis=1)
    g2 = oracle.attn_bwd(S2, x["q"], rep(x["k"]), rep(x["v"]), x["dout"], x["qs"], rep(x["ks"]))
    for n in ("dk", "dv", "dks"):
        summed = g2[n].reshape(1, 2, 2, *g2[n].shape[2:]).sum(2)
        np.testing.assert_allclose(g[n], summed, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["dq"], g2["dq"], rtol=1e-13, atol=1e-15)


def test_bwd_sampled_matches_full():
    S, x = make(batch=2, hq=4, hkv=2, tq=37, tk=37, block=8)
    full = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"])
    rows = np.array([3, 40, 2 * 4 * 37 - 1, 4 * 37 + 20])
    keys = np.array([0, 36, 37 + 5, 3 * 37 + 30])
    sblk = np.array([0, 4, 5 + 2, 3 * 5 + 3])
    sm = oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"],
                         rows=rows, keys=keys, sblocks=sblk)
    np.testing.assert_array_equal(sm["dq"], full["dq"].reshape(-1, S.d)[rows])
    np.testing.assert_array_equal(sm["dz"], full["dz"].reshape(-1, S.nb)[rows])
    np.testing.assert_array_equal(sm["dqs"], full["dqs"].reshape(-1, S.ds)[rows])
    np.testing.assert_array_equal(sm["dk"], full["dk"].reshape(-1, S.d)[keys])
    np.testing.assert_array_equal(sm["dv"], full["dv"].reshape(-1, S.d)[keys])
    np.testing.assert_array_equal(sm["dks"], full["dks"].reshape(-1, S.ds)[sblk])


# --------------------------------------------------------------------- top-K
@pytest.mark.parametrize("renorm", [0, 1])
def test_topk_vs_sort(renorm):
    S, x = make(hq=4, hkv=2, tq=70, tk=70, block=4)
    K = 5
    idx, bias = oracle.topk_blocks(S, K, x["qs"], x["ks"], renorm=renorm)
    z, lam, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    for h in range(S.hq):
        for t in range(S.tq):
            c = t // S.block
            zz = z[0, h, t, :c]
            order = np.lexsort((np.arange(c), -zz))[:K]
            n = len(order)
            np.testing.assert_array_equal(idx[0, h, t, :n], order)
            assert np.all(idx[0, h, t, n:] == -1) and np.all(np.isneginf(bias[0, h, t, n:]))
            norm = logsumexp(zz[order]) if renorm else lam[0, h, t]
            np.testing.assert_allclose(bias[0, h, t, :n], zz[order] - norm, rtol=1e-12, atol=1e-12)


def test_topk_tie_goes_to_smaller_block():
    S, x = make(hq=1, hkv=1, tq=40, tk=40, block=4)
    z = np.zeros((1, 1, 40, S.nb))
    idx, _ = oracle.topk_blocks(S, 3, z=z)
    for t in range(40):
        c = t // 4
        np.testing.assert_array_equal(idx[0, 0, t, :min(3, c)], np.arange(min(3, c)))


@pytest.mark.parametrize("renorm", [0, 1])
@pytest.mark.parametrize("num,den", [(1, 4), (3, 10), (7, 10)])
def test_topk_budget_vs_sort(renorm, num, den):
    S, x = make(hq=4, hkv=2, tq=90, tk=90, block=4)
    kmax = 5
    idx, bias = oracle.topk_budget(S, kmax, (num, den), x["qs"], x["ks"], renorm=renorm)
    z, lam, _ = oracle.gate_scores(S, x["qs"], x["ks"])
    for h in range(S.hq):
        for t in range(S.tq):
            c = t // S.block
            n = min(kmax, c, -(-num * c // den))  # exact ceiling of num c / den
            zz = z[0, h, t, :c]
            order = np.lexsort((np.arange(c), -zz))[:n]
            np.testing.assert_array_equal(idx[0, h, t, :n], order)
            assert np.all(idx[0, h, t, n:] == -1) and np.all(np.isneginf(bias[0, h, t, n:]))
            norm = logsumexp(zz[order]) if renorm else lam[0, h, t]
            np.testing.assert_allclose(bias[0, h, t, :n], zz[order] - norm, rtol=1e-12, atol=1e-12)


def test_topk_budget_quarter_counts():
    # frac = 1/4: a row with c = 4m historical blocks keeps exactly m (cap aside)
    S, x = make(hq=1, hkv=1, tq=130, tk=130, block=4)
    idx, _ = oracle.topk_budget(S, 64, 0.25, x["qs"], x["ks"])
    for t in range(130):
        c = t // 4
        assert int((idx[0, 0, t] >= 0).sum()) == -(-c // 4)


def test_topk_budget_exact_decimal_counts():
    # the fraction is an exact ratio: 30 % of 10 blocks is 3 (a float32 0.3 is
    # slightly above 3/10 and would round the count up to 4); 70 % of 10 is 7
    # (0.7 * 10 is 7.000000000000001 in double)
    S, x = make(hq=1, hkv=1, tq=64, tk=64, block=2)
    for frac, want in ((0.3, {10: 3, 20: 6, 30: 9, 31: 10}), (0.7, {10: 7, 20: 14, 31: 22}),
                       ((1, 3), {3: 1, 9: 3, 10: 4})):
        idx, _ = oracle.topk_budget(S, 32, frac, x["qs"], x["ks"])
        for c, n in want.items():
            for t in (2 * c, 2 * c + 1):
                assert int((idx[0, 0, t] >= 0).sum()) == n, (frac, c)
    assert oracle.budget_ratio(0.3) == (3, 10) and oracle.budget_ratio(0.25) == (1, 4)
    assert oracle.budget_ratio(0.0) == (0, 1) and oracle.budget_ratio(-1.0) == (0, 1)


def test_topk_budget_nonpositive_frac_is_fixed_budget():
    S, x = make(hq=2, hkv=1, tq=50, tk=50, block=4)
    a = oracle.topk_budget(S, 4, 0.0, x["qs"], x["ks"], renorm=1)
    b = oracle.topk_blocks(S, 4, x["qs"], x["ks"], renorm=1)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# -------------------------------------------------------------------- sparse
@pytest.mark.parametrize("renorm", [0, 1])
def test_sparse_full_budget_equals_dense(renorm):
    S, x = make(hq=4, hkv=2, tq=37, tk=37, block=4)
    K = S.nb  # covers every historical block
    idx, bias = oracle.topk_blocks(S, K, x["qs"], x["ks"], renorm=renorm)
    o, l = oracle.sparse_fwd(S, K, x["q"], x["k"], x["v"], idx, bias)
    od, ld = oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    np.testing.assert_allclose(o, od, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, ld, rtol=1e-12)


@pytest.mark.parametrize("renorm", [0, 1])
def test_sparse_vs_bruteforce(renorm):
    S, x = make(hq=4, hkv=2, tq=45, tk=45, block=4)
    K = 3
    idx, bias = oracle.topk_blocks(S, K, x["qs"], x["ks"], renorm=renorm)
    o, l = oracle.sparse_fwd(S, K, x["q"], x["k"], x["v"], idx, bias)
    keep = torch.zeros(1, S.hq, S.tq, S.nb, dtype=torch.bool)
    for h in range(S.hq):
        for t in range(S.tq):
            for j in idx[0, h, t]:
                if j >= 0:
                    keep[0, h, t, j] = True
    z = bf.scores(T(x["qs"]), T(x["ks"]), S.hq, 1.0 / math.sqrt(S.ds))
    bias_m = bf.bias_matrix(z, S.tq, S.tk, S.block, restrict=keep, renorm=bool(renorm))
    ob, lb = bf.attention(T(x["q"]), T(x["k"]), T(x["v"]), bias_m, 1.0 / math.sqrt(S.d))
    np.testing.assert_allclose(o, ob.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lb.numpy(), rtol=1e-12)


@pytest.mark.parametrize("renorm", [0, 1])
def test_sparse_budget_vs_bruteforce(renorm):
    S, x = make(hq=4, hkv=2, tq=61, tk=61, block=4)
    kmax = 6
    idx, bias = oracle.topk_budget(S, kmax, 0.25, x["qs"], x["ks"], renorm=renorm)
    o, l = oracle.sparse_fwd(S, kmax, x["q"], x["k"], x["v"], idx, bias)
    keep = torch.zeros(1, S.hq, S.tq, S.nb, dtype=torch.bool)
    for h in range(S.hq):
        for t in range(S.tq):
            for j in idx[0, h, t]:
                if j >= 0:
                    keep[0, h, t, j] = True
    z = bf.scores(T(x["qs"]), T(x["ks"]), S.hq, 1.0 / math.sqrt(S.ds))
    bias_m = bf.bias_matrix(z, S.tq, S.tk, S.block, restrict=keep, renorm=bool(renorm))
    ob, lb = bf.attention(T(x["q"]), T(x["k"]), T(x["v"]), bias_m, 1.0 / math.sqrt(S.d))
    np.testing.assert_allclose(o, ob.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lb.numpy(), rtol=1e-12)


def test_sparse_decode_row_equals_last_prefill_row():
    S, x = make(hq=4, hkv=2, tq=45, tk=45, block=4)
    K = 3
    idx, bias = oracle.topk_blocks(S, K, x["qs"], x["ks"])
    o, l = oracle.sparse_fwd(S, K, x["q"], x["k"], x["v"], idx, bias)
    Sd = OracleShape(1, 4, 2, 1, 45, S.d, S.ds, 4)
    idx_d, bias_d = oracle.topk_blocks(Sd, K, x["qs"][:, :, -1:], x["ks"])
    np.testing.assert_array_equal(idx_d[:, :, 0], idx[:, :, -1])
    od, ld = oracle.sparse_fwd(Sd, K, x["q"][:, :, -1:], x["k"], x["v"], idx_d, bias_d)
    np.testing.assert_allclose(od[:, :, 0], o[:, :, -1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ld[:, :, 0], l[:, :, -1], rtol=1e-14)


def test_sparse_rejects_bad_index():
    S, x = make(hq=1, hkv=1, tq=20, tk=20, block=4)
    idx = np.full((1, 1, 20, 2), -1, dtype=np.int32)
    bias = np.zeros((1, 1, 20, 2))
    idx[0, 0, 5, 0] = 1  # row t=5 has c=1: block 1 is not historical
    with pytest.raises(ValueError):
        oracle.sparse_fwd(S, 2, x["q"], x["k"], x["v"], idx, bias)
    idx[0, 0, 5, 0] = -1
    idx[0, 0, 12, :] = [1, 1]  # duplicate
    with pytest.raises(ValueError):
        oracle.sparse_fwd(S, 2, x["q"], x["k"], x["v"], idx, bias)


# ------------------------------------------------------- dynamic threshold
def _log_gates_bruteforce(S, x):
    """log g [B,Hq,Tq,NB] from torch: scores by matmul, masked log_softmax over
    the historical blocks of each query (-inf elsewhere)."""
    z = bf.scores(T(x["qs"]), T(x["ks"]), S.hq, 1.0 / math.sqrt(S.ds))
    t, _, ct, _ = bf.positions(S.tq, S.tk, S.block)
    hist = torch.arange(S.nb)[None, :] < ct[:, None]
    zm = torch.where(hist, z, torch.full_like(z, -math.inf))
    ls = torch.log_softmax(zm, dim=-1)
    return torch.where(hist, ls, torch.full_like(ls, -math.inf)).numpy(), ct.numpy()


@pytest.mark.parametrize("theta", [0.02, 0.1, 0.3])
@pytest.mark.parametrize("renorm", [0, 1])
def test_threshold_vs_bruteforce(theta, renorm):
    S, x = make(hq=4, hkv=2, tq=90, tk=90, block=4)
    cnt, idx, bias = oracle.threshold_blocks(S, theta, x["qs"], x["ks"], renorm=renorm)
    lg, ct = _log_gates_bruteforce(S, x)
    th = math.log(float(np.float32(theta)))
    checked = 0
    for h in range(S.hq):
        for i in range(S.tq):
            c = int(ct[i])
            g = lg[0, h, i, :c]
            if c and np.min(np.abs(g - th)) < 1e-9:
                continue  # a gate on the threshold: either answer is right
            checked += 1
            want = np.nonzero(g >= th)[0]
            n = len(want)
            assert cnt[0, h, i] == n
            np.testing.assert_array_equal(idx[0, h, i, :n], want)
            assert np.all(idx[0, h, i, n:] == -1) and np.all(np.isneginf(bias[0, h, i, n:]))
            ref = g[want] - (logsumexp(g[want]) if renorm else 0.0)
            np.testing.assert_allclose(bias[0, h, i, :n], ref, rtol=1e-11, atol=1e-11)
    assert checked > 0.95 * S.hq * S.tq


def test_threshold_special_cases():
    S, x = make(hq=2, hkv=1, tq=70, tk=70, block=4)
    ct = (np.arange(S.tq)) // S.block
    # theta <= 0 keeps every historical block, in order
    cnt, idx, _ = oracle.threshold_blocks(S, 0.0, x["qs"], x["ks"])
    for i in range(S.tq):
        assert cnt[0, 0, i] == ct[i]
        np.testing.assert_array_equal(idx[0, 0, i, :ct[i]], np.arange(ct[i]))
    # a gate never exceeds 1, and equals 1 only with a single historical block
    cnt, _, _ = oracle.threshold_blocks(S, 1.5, x["qs"], x["ks"])
    assert not cnt.any()
    cnt, _, _ = oracle.threshold_blocks(S, 1.0, x["qs"], x["ks"])
    np.testing.assert_array_equal(cnt[0, 0], (ct == 1).astype(np.int32))
    # ks = 0: every gate is 1/c, kept iff 1/c >= theta (0.13: c <= 7)
    z0 = dict(x, ks=np.zeros_like(x["ks"]))
    cnt, _, bias = oracle.threshold_blocks(S, 0.13, z0["qs"], z0["ks"])
    np.testing.assert_array_equal(cnt[0, 0], np.where(ct <= 7, ct, 0))
    for i in range(S.tq):
        if 0 < ct[i] <= 7:
            np.testing.assert_allclose(bias[0, 0, i, :ct[i]], -math.log(ct[i]), rtol=1e-13)


def test_threshold_nested_and_topk_prefix():
    S, x = make(hq=2, hkv=1, tq=120, tk=120, block=4, seed=3)
    c1, i1, _ = oracle.threshold_blocks(S, 0.05, x["qs"], x["ks"])
    c2, i2, _ = oracle.threshold_blocks(S, 0.12, x["qs"], x["ks"])
    ik, _ = oracle.topk_blocks(S, S.nb, x["qs"], x["ks"])
    for h in range(S.hq):
        for i in range(S.tq):
            s1 = set(i1[0, h, i, :c1[0, h, i]].tolist())
            s2 = set(i2[0, h, i, :c2[0, h, i]].tolist())
            assert s2 <= s1  # a higher threshold keeps a subset
            # the kept set is the best-scored prefix of the Top-K order
            n = int(c1[0, h, i])
            assert s1 == set(ik[0, h, i, :n].tolist())


def test_threshold_renorm_bias_sums_to_one():
    S, x = make(hq=2, hkv=1, tq=80, tk=80, block=4, seed=5)
    cnt, _, bias = oracle.threshold_blocks(S, 0.04, x["qs"], x["ks"], renorm=1)
    for h in range(S.hq):
        for i in range(S.tq):
            n = int(cnt[0, h, i])
            if n:
                assert abs(logsumexp(bias[0, h, i, :n])) < 1e-12


@pytest.mark.parametrize("renorm", [0, 1])
def test_sparse_threshold_vs_bruteforce(renorm):
    S, x = make(hq=4, hkv=2, tq=45, tk=45, block=4)
    cnt, idx, bias = oracle.threshold_blocks(S, 0.08, x["qs"], x["ks"], renorm=renorm)
    o, l = oracle.sparse_fwd(S, S.nb, x["q"], x["k"], x["v"], idx, bias)
    keep = torch.zeros(1, S.hq, S.tq, S.nb, dtype=torch.bool)
    for h in range(S.hq):
        for t in range(S.tq):
            for j in idx[0, h, t]:
                if j >= 0:
                    keep[0, h, t, j] = True
    z = bf.scores(T(x["qs"]), T(x["ks"]), S.hq, 1.0 / math.sqrt(S.ds))
    bias_m = bf.bias_matrix(z, S.tq, S.tk, S.block, restrict=keep, renorm=bool(renorm))
    ob, lb = bf.attention(T(x["q"]), T(x["k"]), T(x["v"]), bias_m, 1.0 / math.sqrt(S.d))
    np.testing.assert_allclose(o, ob.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, lb.numpy(), rtol=1e-12)
