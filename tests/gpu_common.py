"""Helpers for the GPU parity tests: device inputs, oracle calls, error metrics."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from gated_block_sparse_sas_amd import synth
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
