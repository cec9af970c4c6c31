"""Helpers for the GPU parity tests: device inputs, oracle calls, error metrics."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from gated_block_sparse_sas_amd import ops, synth
import oracle
from oracle import OracleShape

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oshape(w: synth.Workload) -> OracleShape:
    return OracleShape(w.batch, w.hq, w.hkv, w.tq, w.tk, w.d, w.ds, w.block, hks=w.kheads)


class LazyF64(dict):
    """Exact fp64 copies of the stored inputs, converted on first use."""

    def __init__(self, cpu):
        super().__init__()
        self._cpu = cpu

    def __missing__(self, n):
        a = synth.to_f64(self._cpu[n])
        self[n] = a
        return a


def inputs(w: synth.Workload, names=("q", "k", "v", "qs", "ks", "dout")):
    """CPU tensors (storage dtype), device copies and exact fp64 copies."""
    cpu = synth.draw_all(w, names)
    dev = {n: t.to(DEV) for n, t in cpu.items()}
    return cpu, dev, LazyF64(cpu)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / (den if den > 0 else 1.0)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def sample_rows(w: synth.Workload, n: int, seed: int = 0) -> np.ndarray:
    """Flat (b,h,i) rows spread over heads and positions, including the first
    and last rows and rows at block edges."""
    rng = np.random.default_rng(seed)
    rows = set()
    total = w.batch * w.hq * w.tq
    for r in (0, total - 1, w.tq - 1, min(w.tq, 64) - 1):
        rows.add(int(r))
    while len(rows) < n:
        b = int(rng.integers(0, w.batch))
        h = int(rng.integers(0, w.hq))
        i = int(rng.integers(0, w.tq))
        if rng.random() < 0.3:
            i = min(w.tq - 1, (i // 64) * 64 + int(rng.choice([0, 63])))
        rows.add((b * w.hq + h) * w.tq + i)
    return np.array(sorted(rows), dtype=np.int64)


def tie_free_rows(z: np.ndarray, c: np.ndarray, k: int, eps: float = 1e-4) -> np.ndarray:
    """Rows whose sorted top-(k+1) fp64 scores are separated by > eps*max(1,|z|)."""
    ok = np.ones(z.shape[0], dtype=bool)
    for r in range(z.shape[0]):
        zz = np.sort(z[r, :c[r]])[::-1][:k + 1]
        if len(zz) >= 2:
            gaps = zz[:-1] - zz[1:]
            if np.any(gaps <= eps * np.maximum(1.0, np.abs(zz[:-1]))):
                ok[r] = False
    return ok


GRADS = ("dq", "dk", "dv", "dz", "dqs", "dks")


def row_bound(name, got, ref, rel=0.1, floor=0.05, extra=None):
    """Every row of got within rel * max(|ref row|, floor * median |ref row|),
    plus extra[row] (an absolute allowance per row) when given."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    nr = np.linalg.norm(r, axis=1)
    err = np.linalg.norm(g - r, axis=1)
    pos = nr[nr > 0]
    fl = floor * (np.median(pos) if pos.size else 1.0)
    lim = rel * np.maximum(nr, fl) + 1e-30
    if extra is not None:
        lim = lim + np.asarray(extra, dtype=np.float64).reshape(-1)
    worst = float(np.max(err / lim)) if err.size else 0.0
    say("  %s worst row error / bound %.3f" % (name, worst))
    assert worst <= 1.0, name


def gpu_train(dev, w, sm_scale=None, sel_scale=None):
    lam = ops.gate_scores(dev["qs"], dev["ks"], w.tk, block=w.block, sel_scale=sel_scale)
    o, lse = ops.attn_fwd(dev["q"], dev["k"], dev["v"], dev["qs"], dev["ks"], lam, block=w.block,
                          sm_scale=sm_scale, sel_scale=sel_scale)
    g = ops.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["dout"], lse, dev["qs"], dev["ks"], lam,
                     block=w.block, sm_scale=sm_scale, sel_scale=sel_scale)
    torch.cuda.synchronize()
    return lam, o, lse, g


def dks_allowance(w, S, f, beta, lse_ref, dD):
    """Per selector unit (b, s, j): the part of dks_j the backward inherits
    from D_t's error |dD_t|.  dz_{t,j} moves by -(sum_{u in j} P_{t,u}) dD_t
    through dbeta_j and by g_{t,j} P_{t,cur} dD_t through sum dbeta (minus the
    current unit's dS sum), so |d dks_j| <= sel_scale sum_t (P_{t,j} +
    g_{t,j} P_{t,cur}) |dD_t| |qs_t|.  P, g from the fp64 inputs and the
    oracle's beta and lse (small shapes)."""
    tau = S.sm_scale or 1.0 / np.sqrt(w.d)
    sig = S.sel_scale or 1.0 / np.sqrt(w.ds)
    blk, nb, hks = w.block, w.nb, w.kheads
    out = np.zeros((w.batch, hks, nb))
    t = np.arange(w.tq) + w.tk - w.tq
    c = t // blk
    u = np.arange(w.tk)
    dD = dD.reshape(w.batch, w.hq, w.tq)
    for b in range(w.batch):
        for h in range(w.hq):
            gk, sh = h // (w.hq // w.hkv), h // (w.hq // hks)
            bt = beta[b, h]                               # [tq, nb]: z - lam, 0, -inf
            logit = tau * f["q"][b, h] @ f["k"][b, gk].T + np.repeat(bt, blk, axis=1)
            logit[u[None, :] > t[:, None]] = -np.inf
            P = np.exp(logit - lse_ref[b, h][:, None])
            pj = P.reshape(w.tq, nb, blk).sum(-1)         # [tq, nb]
            pcur = pj[np.arange(w.tq), c]
            hist = np.arange(nb)[None, :] < c[:, None]
            gj = np.where(hist, np.exp(np.where(hist, bt, 0.0)), 0.0)
            a = np.where(hist, pj + gj * pcur[:, None], 0.0)
            wq = dD[b, h] * np.linalg.norm(f["qs"][b, h], axis=-1)
            out[b, sh] += sig * (a * wq[:, None]).sum(0)
    return out


def check_train(w, f, lam, o, lse, g, S):
    _, lam_ref, beta_ref = oracle.gate_scores(S, f["qs"], f["ks"])
    fin = np.isfinite(lam_ref)
    assert np.array_equal(np.isneginf(host(lam)), np.isneginf(lam_ref))
    if fin.any():  # (no row has a historical unit when tq <= the unit)
        e = max_abs(host(lam)[fin], lam_ref[fin])
        say("  lam max-abs %.2e" % e)
        assert e <= 1e-4 * max(1.0, float(np.max(np.abs(lam_ref[fin]))))
    o_ref, l_ref = oracle.attn_fwd(S, f["q"], f["k"], f["v"], f["qs"], f["ks"])
    eo, el = max_abs(host(o), o_ref), max_abs(host(lse), l_ref)
    say("  O max-abs %.2e  lse max-abs %.2e" % (eo, el))
    assert eo <= 2e-2 and el <= 1e-3
    ref = oracle.attn_bwd(S, f["q"], f["k"], f["v"], f["dout"], f["qs"], f["ks"])
    # error of D_t = <dO_t, o_t> inherited from the forward output (Cauchy-Schwarz)
    dD = (np.linalg.norm(f["dout"], axis=-1)
          * np.linalg.norm(host(o) - o_ref, axis=-1)).reshape(-1)
    tau = S.sm_scale or 1.0 / np.sqrt(w.d)
    sig = S.sel_scale or 1.0 / np.sqrt(w.ds)
    kmax = float(np.max(np.linalg.norm(f["k"], axis=-1)))
    ksmax = float(np.max(np.linalg.norm(f["ks"], axis=-1)))
    extra = {"dq": 2 * tau * kmax * dD, "dz": 4 * dD, "dqs": 4 * sig * ksmax * dD,
             "dks": dks_allowance(w, S, f, beta_ref, l_ref, dD)}
    for n in GRADS:
        e = rel_l2(host(g[n]), ref[n])
        say("  %s rel-L2 %.3e" % (n, e))
        assert e <= 5e-2, n
        row_bound(n, host(g[n]), ref[n], extra=extra.get(n))
    return ref
