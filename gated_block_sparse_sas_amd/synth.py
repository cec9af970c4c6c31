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
