"""Brute-force full-matrix SAS attention in torch-CPU fp64 (test helper).

Independent of the C oracle: it builds the whole [Tq, Tk] additive bias
matrix from a masked ``log_softmax`` of the selector scores, hands it to
``scaled_dot_product_attention`` as a float mask, and gets every gradient from
autograd.  Only tiny shapes are meant for it.
"""

from __future__ import annotations

import math

import torch
import torch.nn.functional as F


def positions(tq, tk, block):
    qoff = tk - tq
    t = torch.arange(tq) + qoff
    u = torch.arange(tk)
    return t, u, t // block, u // block


def bias_matrix(z, tq, tk, block, restrict=None, renorm=False):
    """z: [..., Tq, NB] scores.  Returns the [..., Tq, Tk] additive mask:
    log_softmax over the query's historical blocks for earlier blocks, 0 inside
    the current block up to the query, -inf elsewhere.  ``restrict`` (bool
    [..., Tq, NB]) keeps only some historical blocks (sparse mode, bias still
    normalised over all history, or over the kept blocks when ``renorm``)."""
    t, u, ct, cu = positions(tq, tk, block)
    nb = z.shape[-1]
    hist = torch.arange(nb)[None, :] < ct[:, None]  # [Tq, NB]
    if restrict is not None and renorm:
        hist = hist & restrict
    zm = torch.where(hist, z, torch.full_like(z, -math.inf))
    ls = torch.log_softmax(zm, dim=-1)
    ls = torch.where(hist, ls, torch.zeros_like(ls))  # rows without history
    beta_u = ls[..., cu]  # [..., Tq, Tk] value of the key's block
    hist_u = cu[None, :] < ct[:, None]
    cur_u = (cu[None, :] == ct[:, None]) & (u[None, :] <= t[:, None])
    if restrict is not None:
        hist_u = hist_u & restrict[..., cu]
    neg = torch.full_like(beta_u, -math.inf)
    return torch.where(hist_u, beta_u, torch.where(cur_u, torch.zeros_like(beta_u), neg))


def scores(qs, ks, hq, sel_scale):
    """z = sel_scale * qs ks^T with the selector head of each query head."""
    rep = hq // ks.shape[1]
    ksr = ks.repeat_interleave(rep, dim=1)
    return sel_scale * torch.matmul(qs, ksr.transpose(-1, -2))


def attention(q, k, v, bias, sm_scale):
    rep = q.shape[1] // k.shape[1]
    kr = k.repeat_interleave(rep, dim=1)
    vr = v.repeat_interleave(rep, dim=1)
    o = F.scaled_dot_product_attention(q, kr, vr, attn_mask=bias, scale=sm_scale)
    lse = torch.logsumexp(sm_scale * torch.matmul(q, kr.transpose(-1, -2)) + bias, dim=-1)
    return o, lse


def gated(q, k, v, qs=None, ks=None, z=None, block=64, sm_scale=None, sel_scale=None):
    """Dense-active gated attention.  All inputs fp64 torch tensors."""
    tq, tk, d = q.shape[2], k.shape[2], q.shape[3]
    sm_scale = sm_scale if sm_scale else 1.0 / math.sqrt(d)
    if z is None:
        sel_scale = sel_scale if sel_scale else 1.0 / math.sqrt(qs.shape[-1])
        z = scores(qs, ks, q.shape[1], sel_scale)
    return attention(q, k, v, bias_matrix(z, tq, tk, block), sm_scale)


def grads(q, k, v, dout, qs=None, ks=None, z=None, block=64, sm_scale=None, sel_scale=None):
    """Autograd of sum(dout * O) wrt every input given."""
    leaves = {n: t.detach().clone().requires_grad_(True)
              for n, t in dict(q=q, k=k, v=v, qs=qs, ks=ks, z=z).items() if t is not None}
    o, _ = gated(leaves["q"], leaves["k"], leaves["v"], leaves.get("qs"), leaves.get("ks"),
                 leaves.get("z"), block, sm_scale, sel_scale)
    (o * dout).sum().backward()
    return {n: t.grad for n, t in leaves.items()}
