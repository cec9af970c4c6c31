"""Seeded synthetic inputs shaped like the workloads of the SAS pages.

This module only draws random numbers: it holds none of the method's
arithmetic, and both the HIP path and the CPU oracle read the tensors it
returns.  Values are drawn as float32 standard normals from numpy's PCG64 with
``seed = 1000 * workload_id + tensor_id`` (tensor ids: q=0, k=1, v=2, qs=3,
ks=4, dout=5), multiplied by the workload's scale and then rounded
round-to-nearest-even to the storage dtype.  The oracle reads the rounded
values, so both sides see identical inputs.

The pages evaluate on reasoning, long-context and agentic suites they do not
name; none of their items are reproduced.  These tensors stand in for the
shapes only: a 32k-token context, 64-token blocks and a tight block budget.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "qs": 3, "ks": 4, "dout": 5}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtypes, value scales and mode."""

    name: str
    wid: int
    batch: int
    hq: int
    hkv: int
    tq: int
    tk: int
    d: int
    ds: int
    block: int
    dtype: str  # "f32" or "bf16"
    mode: str  # "train", "prefill" or "decode"
    topk: int = 0  # fixed budget, or the cap kmax of a proportional one
    frac: float = 0.0  # > 0: row t keeps min(topk, ceil(frac * c(t))) blocks
    theta: float = 0.0  # dynamic threshold on the normalised gate (selection by threshold)
    hks: int = 0  # 0 -> hkv
    scales: dict = field(default_factory=dict)

    @property
    def nb(self) -> int:
        return (self.tk + self.block - 1) // self.block

    @property
    def kheads(self) -> int:
        return self.hks if self.hks else self.hkv

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scale(self, name: str) -> float:
        return float(self.scales.get(name, 1.0))

    def shapes(self) -> dict:
        return {
            "q": (self.batch, self.hq, self.tq, self.d),
            "k": (self.batch, self.hkv, self.tk, self.d),
            "v": (self.batch, self.hkv, self.tk, self.d),
            "qs": (self.batch, self.hq, self.tq, self.ds),
            "ks": (self.batch, self.kheads, self.nb, self.ds),
            "dout": (self.batch, self.hq, self.tq, self.d),
        }

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_HALF = {"q": 0.5, "k": 0.5, "v": 0.5}

# The workloads: a tiny fp32 case, dense-active training at 8k and 32k,
# top-K sparse prefill at 32k (fixed budget of 16 blocks, and a budget of a
# quarter of each row's history, capped at 128 blocks) and top-K sparse
# decode at 64k.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1, 1, 512, 512, 64, 16, 64, "f32", "train"),
    "train_8k": Workload("train_8k", 2, 1, 32, 8, 8192, 8192, 128, 32, 64, "bf16", "train",
                         scales=_HALF),
    "train_32k": Workload("train_32k", 3, 1, 32, 8, 32768, 32768, 128, 32, 64, "bf16", "train",
                          scales=_HALF),
    "prefill_32k_top16": Workload("prefill_32k_top16", 4, 1, 32, 8, 32768, 32768, 128, 32, 64,
                                  "bf16", "prefill", topk=16, scales=_HALF),
    "decode_64k_top8": Workload("decode_64k_top8", 5, 16, 32, 8, 1, 65536, 128, 32, 64, "bf16",
                                "decode", topk=8, scales=_HALF),
    "prefill_32k_top25pct": Workload("prefill_32k_top25pct", 6, 1, 32, 8, 32768, 32768, 128, 32,
                                     64, "bf16", "prefill", topk=128, frac=0.25, scales=_HALF),
    # 16-token context units at prefill: 64 units = the 1024-token budget of K = 16 x 64
    "prefill_32k_b16_top64": Workload("prefill_32k_b16_top64", 10, 1, 32, 8, 32768, 32768, 128,
                                      32, 16, "bf16", "prefill", topk=64, scales=_HALF),
    # 16-token context units at decode: 32 units = the 512-token budget of K = 8 x 64
    "decode_64k_b16_top32": Workload("decode_64k_b16_top32", 9, 16, 32, 8, 1, 65536, 128, 32,
                                     16, "bf16", "decode", topk=32, scales=_HALF),
    # selection by a dynamic threshold: blocks whose normalised gate is >= 0.01
    "prefill_32k_theta": Workload("prefill_32k_theta", 8, 1, 32, 8, 32768, 32768, 128, 32, 64,
                                  "bf16", "prefill", theta=0.01, scales=_HALF),
}


def _round(a32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # round-to-nearest-even
    return t


def draw(w: Workload, name: str, seed_base: int | None = None) -> torch.Tensor:
    """One input tensor of workload ``w`` as a CPU tensor in its storage dtype."""
    wid = w.wid if seed_base is None else seed_base
    seed = 1000 * wid + TENSOR_IDS[name]
    shape = w.shapes()[name]
    rng = np.random.Generator(np.random.PCG64(seed))
    n = math.prod(shape)
    out = torch.empty(n, dtype=w.torch_dtype())
    chunk = 1 << 26
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        a = rng.standard_normal(m, dtype=np.float32)
        sc = w.scale(name)
        if sc != 1.0:
            a *= np.float32(sc)
        out[s:s + m] = _round(a, w.dtype)
    return out.view(shape)


def draw_all(w: Workload, names=("q", "k", "v", "qs", "ks", "dout"), seed_base=None) -> dict:
    return {n: draw(w, n, seed_base) for n in names}


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored tensor for the oracle."""
    return t.detach().to("cpu", torch.float64).numpy()


# ---------------------------------------------------------------------------
# Serving-shaped decode over a block-paged cache.  Sequence lengths are drawn
# log-uniformly between min_len and max_len (a mix of short and long
# contexts, as a decode batch of a serving engine holds), every sequence's
# blocks go to pages in a seeded random order, and the pools hold exactly
# the pages in use plus `spare` unused ones.  Extra tensor ids: lengths = 10,
# page order = 11; q, qs as above ([batch, hq, d] / [batch, hq, ds]), the K,
# V and ks pools with the ids of k, v and ks.

@dataclass(frozen=True)
class PagedWorkload:
    name: str
    wid: int
    batch: int
    hq: int
    hkv: int
    d: int
    ds: int
    min_len: int
    max_len: int
    topk: int
    dtype: str = "bf16"
    hks: int = 0
    spare: int = 3
    block: int = 64
    scales: dict = field(default_factory=lambda: dict(_HALF))

    @property
    def kheads(self) -> int:
        return self.hks if self.hks else self.hkv

    @property
    def max_blocks(self) -> int:
        return (self.max_len + self.block - 1) // self.block

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "PagedWorkload":
        return replace(self, **kw)


PAGED_WORKLOADS = {
    "decode_paged_mix": PagedWorkload("decode_paged_mix", 7, 32, 32, 8, 128, 32, 64, 65536, 8),
}


def _normals(seed: int, shape, scale: float, dtype: str) -> torch.Tensor:
    rng = np.random.Generator(np.random.PCG64(seed))
    n = math.prod(shape)
    out = torch.empty(n, dtype=torch.float32 if dtype == "f32" else torch.bfloat16)
    chunk = 1 << 26
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        a = rng.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            a *= np.float32(scale)
        out[s:s + m] = _round(a, dtype)
    return out.view(shape)


def draw_paged(pw: PagedWorkload, lens=None) -> dict:
    """CPU tensors of a paged decode batch: seq_len [batch] int32, block_table
    [batch, max_blocks] int32 (-1 past a sequence's last block), k_pool,
    v_pool [pages, hkv, 64, d], ks_pool [pages, hks, ds], q [batch, hq, d],
    qs [batch, hq, ds].  `lens` overrides the drawn lengths."""
    base = 1000 * pw.wid
    if lens is None:
        rng = np.random.Generator(np.random.PCG64(base + 10))
        u = rng.random(pw.batch)
        lo, hi = math.log(pw.min_len), math.log(pw.max_len)
        lens = np.minimum(pw.max_len, np.floor(np.exp(lo + u * (hi - lo)))).astype(np.int64)
        lens = np.maximum(lens, pw.min_len)
    lens = np.asarray(lens, dtype=np.int64)
    nblk = (lens + pw.block - 1) // pw.block
    pages = int(nblk.sum()) + pw.spare
    order = np.random.Generator(np.random.PCG64(base + 11)).permutation(pages)
    table = np.full((pw.batch, pw.max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(pw.batch):
        table[b, :nblk[b]] = order[off:off + nblk[b]]
        off += int(nblk[b])
    sc = pw.scales
    return {
        "seq_len": torch.from_numpy(lens.astype(np.int32)),
        "block_table": torch.from_numpy(table),
        "k_pool": _normals(base + 1, (pages, pw.hkv, pw.block, pw.d), sc.get("k", 1.0), pw.dtype),
        "v_pool": _normals(base + 2, (pages, pw.hkv, pw.block, pw.d), sc.get("v", 1.0), pw.dtype),
        "ks_pool": _normals(base + 4, (pages, pw.kheads, pw.ds), sc.get("ks", 1.0), pw.dtype),
        "q": _normals(base + 0, (pw.batch, pw.hq, pw.d), sc.get("q", 1.0), pw.dtype),
        "qs": _normals(base + 3, (pw.batch, pw.hq, pw.ds), sc.get("qs", 1.0), pw.dtype),
    }
