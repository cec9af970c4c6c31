"""Decode over a block-paged cache (serving shape) against the oracle.

The oracle knows nothing of pages: each sequence's blocks are gathered from
the pools into a contiguous [1, hkv, len, d] cache (pure data movement) and
the oracle's decode row (t = len - 1) is the reference.  Append is checked
bit-exactly against a numpy scatter.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from gpu_common import DEV, host, max_abs, say, tie_free_rows

pytestmark = pytest.mark.gpu

PW = synth.PAGED_WORKLOADS


def _contig(pool: np.ndarray, table_row: np.ndarray, n_tok: int) -> np.ndarray:
    """[pages, heads, 64, d] pool -> [heads, n_tok, d] for one sequence."""
    nblk = (n_tok + 63) // 64
    blocks = pool[table_row[:nblk]]                  # [nblk, heads, 64, d]
    seq = np.transpose(blocks, (1, 0, 2, 3)).reshape(pool.shape[1], nblk * 64, -1)
    return seq[:, :n_tok]


def _ks_contig(ks_pool: np.ndarray, table_row: np.ndarray, n_blk: int) -> np.ndarray:
    """[pages, hks, ds] -> [hks, n_blk, ds]."""
    return np.transpose(ks_pool[table_row[:n_blk]], (1, 0, 2))


def _seq_shape(pw, n_tok):
    return oracle.OracleShape(1, pw.hq, pw.hkv, 1, n_tok, pw.d, pw.ds, 64, hks=pw.kheads)


def _f64(t):
    return {n: synth.to_f64(t[n]) for n in ("k_pool", "v_pool", "ks_pool", "q", "qs")}


def _oracle_rows(pw, t, renorm=0, f=None):
    """Per sequence: the oracle's selection and its decode output over it."""
    lens = t["seq_len"].numpy()
    table = t["block_table"].numpy()
    f = _f64(t) if f is None else f
    out = []
    for b, n_tok in enumerate(lens):
        S = _seq_shape(pw, int(n_tok))
        nblk = (int(n_tok) + 63) // 64
        k = _contig(f["k_pool"], table[b], int(n_tok))[None]
        v = _contig(f["v_pool"], table[b], int(n_tok))[None]
        ks = _ks_contig(f["ks_pool"], table[b], nblk)[None]
        q = f["q"][b][None, :, None, :]
        qs = f["qs"][b][None, :, None, :]
        idx, bias = oracle.topk_blocks(S, pw.topk, qs, ks, renorm=renorm)
        bias = bias.astype(np.float32).astype(np.float64)
        o, lse = oracle.sparse_fwd(S, pw.topk, q, k, v, idx, bias)
        z, _, _ = oracle.gate_scores(S, qs, ks)
        out.append(dict(idx=idx.reshape(pw.hq, pw.topk), bias=bias.reshape(pw.hq, pw.topk),
                        o=o.reshape(pw.hq, pw.d), lse=lse.reshape(pw.hq),
                        z=z.reshape(pw.hq, -1), c=(int(n_tok) - 1) // 64))
    return out


def _dev(t):
    return {n: x.to(DEV) for n, x in t.items()}


SMALL = PW["decode_paged_mix"].with_(batch=6, max_len=3000, topk=5)


def test_paged_append_exact():
    pw = SMALL
    t = synth.draw_paged(pw)
    d = _dev(t)
    k_pool = torch.zeros_like(d["k_pool"])
    v_pool = torch.zeros_like(d["v_pool"])
    ks_pool = torch.zeros_like(d["ks_pool"])
    lens = t["seq_len"].numpy()
    # positions: the last token of each sequence, except two that end a block
    pos = (lens - 1).astype(np.int32)
    pos[1] = 63
    pos[4] = 64 * 3 + 63
    pos[5] = -1  # out of range: skipped
    g = torch.Generator().manual_seed(3)
    k_new = torch.randn(pw.batch, pw.hkv, pw.d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(pw.batch, pw.hkv, pw.d, generator=g).to(torch.bfloat16)
    ks_new = torch.randn(pw.batch, pw.kheads, pw.ds, generator=g).to(torch.bfloat16)
    ops.paged_append(torch.from_numpy(pos).to(DEV), d["block_table"], k_new.to(DEV),
                     v_new.to(DEV), k_pool, v_pool, ks_new.to(DEV), ks_pool)
    torch.cuda.synchronize()
    ek = torch.zeros_like(t["k_pool"])
    ev = torch.zeros_like(t["v_pool"])
    eks = torch.zeros_like(t["ks_pool"])
    table = t["block_table"].numpy()
    for b in range(pw.batch):
        p = int(pos[b])
        if p < 0:
            continue
        pg = int(table[b, p // 64])
        ek[pg, :, p % 64] = k_new[b]
        ev[pg, :, p % 64] = v_new[b]
        if p % 64 == 63:
            eks[pg] = ks_new[b]
    assert torch.equal(k_pool.cpu(), ek)
    assert torch.equal(v_pool.cpu(), ev)
    assert torch.equal(ks_pool.cpu(), eks)
    assert int((eks != 0).any(dim=(1, 2)).sum()) >= 2  # the two block ends wrote a row


@pytest.mark.parametrize("renorm", [0, 1])
def test_paged_decode_vs_oracle(renorm):
    pw = SMALL
    say("paged decode small", renorm)
    t = synth.draw_paged(pw)
    ref = _oracle_rows(pw, t, renorm)
    d = _dev(t)
    idx = torch.from_numpy(np.stack([r["idx"] for r in ref])).to(DEV)
    bias = torch.from_numpy(np.stack([r["bias"] for r in ref]).astype(np.float32)).to(DEV)
    o, lse = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    torch.cuda.synchronize()
    e = max_abs(host(o), np.stack([r["o"] for r in ref]))
    say("  O max-abs", e)
    assert e <= 2e-2
    assert max_abs(host(lse), np.stack([r["lse"] for r in ref])) <= 1e-3


@pytest.mark.parametrize("renorm", [0, 1])
def test_paged_topk_vs_oracle(renorm):
    pw = SMALL.with_(topk=7)
    t = synth.draw_paged(pw)
    ref = _oracle_rows(pw, t, renorm)
    d = _dev(t)
    idx, bias = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk,
                               renorm=renorm)
    torch.cuda.synchronize()
    ig, bg = idx.cpu().numpy(), bias.cpu().numpy()
    n_ok = 0
    for b, r in enumerate(ref):
        ok = tie_free_rows(r["z"], np.full(pw.hq, r["c"]), pw.topk)
        n_ok += int(ok.sum())
        assert np.array_equal(ig[b][ok], r["idx"][ok])
        fin = np.isfinite(r["bias"][ok])
        assert max_abs(bg[b][ok][fin], r["bias"][ok][fin]) <= 1e-4
        assert np.array_equal((ig[b] >= 0).sum(-1), (r["idx"] >= 0).sum(-1))
    assert n_ok >= 0.9 * pw.batch * pw.hq


def test_paged_equals_contiguous_decode():
    # equal lengths: the same blocks laid out contiguously through the
    # contiguous entry point give the same bits
    pw = PW["decode_paged_mix"].with_(batch=4, max_len=64 * 40, topk=6)
    L = 64 * 37
    t = synth.draw_paged(pw, lens=[L] * pw.batch)
    d = _dev(t)
    table = t["block_table"].numpy()
    kc = torch.stack([torch.from_numpy(_contig(t["k_pool"].float().numpy(), table[b], L))
                      for b in range(pw.batch)]).to(torch.bfloat16).to(DEV)
    vc = torch.stack([torch.from_numpy(_contig(t["v_pool"].float().numpy(), table[b], L))
                      for b in range(pw.batch)]).to(torch.bfloat16).to(DEV)
    ksc = torch.stack([torch.from_numpy(_ks_contig(t["ks_pool"].float().numpy(), table[b], L // 64))
                       for b in range(pw.batch)]).to(torch.bfloat16).to(DEV)
    qs4 = d["qs"][:, :, None, :].contiguous()
    q4 = d["q"][:, :, None, :].contiguous()
    i_c, b_c = ops.topk_blocks(qs4, ksc, pw.topk, L)
    i_p, b_p = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    o_c, l_c = ops.sparse_fwd(q4, kc, vc, i_c, b_c)
    o_p, l_p = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"],
                                d["seq_len"], i_p, b_p)
    torch.cuda.synchronize()
    assert torch.equal(i_c[:, :, 0], i_p)
    assert torch.equal(b_c[:, :, 0], b_p)
    assert torch.equal(o_c[:, :, 0], o_p)
    assert torch.equal(l_c[:, :, 0], l_p)


def test_paged_edge_lengths():
    # first token (len 1: only itself), a full table, a length past the table
    # (no keys: o = 0, lse = -inf, nothing selected), a block-aligned length
    pw = PW["decode_paged_mix"].with_(batch=5, max_len=64 * 12, topk=4)
    lens = [1, 64 * 12, 64 * 5, 65, 64 * 12]
    t = synth.draw_paged(pw, lens=lens)
    bad = t["seq_len"].clone()
    bad[4] = 64 * 12 + 1  # beyond the table: the row has no keys
    ref = _oracle_rows(pw, t)
    d = _dev(t)
    d["seq_len"] = bad.to(DEV)
    idx, bias = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    o, lse = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    for b in range(4):
        ok = tie_free_rows(ref[b]["z"], np.full(pw.hq, ref[b]["c"]), pw.topk)
        assert np.array_equal(ig[b][ok], ref[b]["idx"][ok])
        assert max_abs(host(o)[b][ok], ref[b]["o"][ok]) <= 2e-2
        assert max_abs(host(lse)[b][ok], ref[b]["lse"][ok]) <= 1e-3
    assert (ig[4] == -1).all()
    assert torch.equal(o[4].float().cpu(), torch.zeros(pw.hq, pw.d))
    assert torch.isneginf(lse[4]).all().item()


def test_paged_full_size_end_to_end():
    # 32 sequences, lengths 64 .. 65536 (log-uniform), 32 query / 8 kv heads,
    # K = 8: GPU selection then GPU decode.  On every tie-free row the GPU's
    # selection must be the oracle's, and its output the oracle's decode over
    # that (its own) selection
    pw = PW["decode_paged_mix"]
    say("paged full", pw.batch, "sequences")
    t = synth.draw_paged(pw)
    d = _dev(t)
    idx, bias = ops.paged_topk(d["qs"], d["ks_pool"], d["block_table"], d["seq_len"], pw.topk)
    o, lse = ops.paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["seq_len"],
                              idx, bias)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()
    og, lg = host(o), host(lse)
    ref = _oracle_rows(pw, t, f=_f64(t))
    n_ok, e = 0, 0.0
    for b, r in enumerate(ref):
        ok = tie_free_rows(r["z"], np.full(pw.hq, r["c"]), pw.topk)
        n_ok += int(ok.sum())
        assert np.array_equal(ig[b][ok], r["idx"][ok])
        e = max(e, max_abs(og[b][ok], r["o"][ok]))
        assert max_abs(lg[b][ok], r["lse"][ok]) <= 1e-3
    say("  O max-abs", e, "lens", t["seq_len"].min().item(), "..", t["seq_len"].max().item())
    assert e <= 2e-2
    assert n_ok >= 0.9 * pw.batch * pw.hq
