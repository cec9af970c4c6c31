"""ctypes marshalling for the C oracle (``sas_oracle.c``).

Test infrastructure only: see the package docstring.  Every function takes
numpy arrays (any float dtype; they are upcast exactly to float64) in the BHSD
layout described in ``sas_oracle.h`` and returns float64 results.
"""

from __future__ import annotations

import ctypes
from fractions import Fraction
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sas_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a separately built copy (the sanitizer run) may be named by the environment
_LIB_ENV = os.environ.get("SAS_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``sas_oracle.c`` into ``liboracle.so`` with gcc (fp64, OpenMP)."""
    global _lib
    if _LIB_ENV:
        return _LIB_ENV
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("hks", ctypes.c_int32), ("tq", ctypes.c_int32), ("tk", ctypes.c_int32),
        ("d", ctypes.c_int32), ("ds", ctypes.c_int32), ("block", ctypes.c_int32),
        ("sm_scale", ctypes.c_double), ("sel_scale", ctypes.c_double),
    ]


@dataclass
class OracleShape:
    batch: int
    hq: int
    hkv: int
    tq: int
    tk: int
    d: int
    ds: int
    block: int
    hks: int | None = None
    sm_scale: float | None = None
    sel_scale: float | None = None

    @property
    def nb(self) -> int:
        return (self.tk + self.block - 1) // self.block

    def c_struct(self) -> _Shape:
        return _Shape(
            self.batch, self.hq, self.hkv, self.hks if self.hks else self.hkv, self.tq, self.tk,
            self.d, self.ds, self.block,
            self.sm_scale if self.sm_scale else 1.0 / math.sqrt(self.d),
            self.sel_scale if self.sel_scale else 1.0 / math.sqrt(self.ds),
        )


def _load():
    global _lib
    if _lib is None:
        if _LIB_ENV:
            lib = ctypes.CDLL(_LIB_ENV)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_gate_scores.argtypes = [P, P, P, P, P, P]
        lib.oracle_attn_fwd.argtypes = [P, P, P, P, P, P, P, I64, P, P, P]
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, I64, P, P, P, P, I64, P, P, P,
                                        I64, P, P]
        lib.oracle_topk_blocks.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
        lib.oracle_topk_budget.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, P, P, P, P, P]
        lib.oracle_threshold_blocks.argtypes = [P, ctypes.c_float, ctypes.c_int32, P, P, P, P,
                                                P, P]
        lib.oracle_sparse_fwd.argtypes = [P, ctypes.c_int32, P, P, P, P, P, I64, P, P, P]
        for f in (lib.oracle_gate_scores, lib.oracle_attn_fwd, lib.oracle_attn_bwd,
                  lib.oracle_topk_blocks, lib.oracle_topk_budget, lib.oracle_threshold_blocks,
                  lib.oracle_sparse_fwd):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _idx(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed with code %d" % (what, rc))


def gate_scores(shape: OracleShape, qs, ks):
    """Returns (z, lam, beta): z, beta [B,Hq,Tq,NB]; lam [B,Hq,Tq]."""
    qs, ks = _f64(qs), _f64(ks)
    z = np.empty((shape.batch, shape.hq, shape.tq, shape.nb))
    beta = np.empty_like(z)
    lam = np.empty((shape.batch, shape.hq, shape.tq))
    st = shape.c_struct()
    _check(_load().oracle_gate_scores(ctypes.byref(st), _ptr(qs), _ptr(ks), _ptr(z), _ptr(lam),
                                      _ptr(beta)), "gate_scores")
    return z, lam, beta


def attn_fwd(shape: OracleShape, q, k, v, qs=None, ks=None, z=None, rows=None):
    """Dense-active gated forward.  Returns (o, lse); with ``rows`` (flat
    (b,h,i) indices) o is [n,d] and lse [n], else full [B,Hq,Tq,d] / [B,Hq,Tq]."""
    q, k, v, qs, ks, z = map(_f64, (q, k, v, qs, ks, z))
    rows = _idx(rows)
    n = shape.batch * shape.hq * shape.tq if rows is None else len(rows)
    o = np.empty((n, shape.d))
    lse = np.empty((n,))
    st = shape.c_struct()
    _check(_load().oracle_attn_fwd(ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(ks),
                                   _ptr(z), n, _ptr(rows), _ptr(o), _ptr(lse)), "attn_fwd")
    if rows is None:
        return (o.reshape(shape.batch, shape.hq, shape.tq, shape.d),
                lse.reshape(shape.batch, shape.hq, shape.tq))
    return o, lse


def attn_bwd(shape: OracleShape, q, k, v, dout, qs=None, ks=None, z=None,
             rows="all", keys="all", sblocks="all"):
    """Dense-active backward.  ``rows``/``keys``/``sblocks`` are flat index
    lists ((b,h,i), (b,g,u), (b,s,j)) or "all" (full tensors, reshaped) or
    None (skip).  Returns dict with dq, dz, dqs, dk, dv, dks."""
    q, k, v, dout, qs, ks, z = map(_f64, (q, k, v, dout, qs, ks, z))
    S = shape
    hks = S.hks if S.hks else S.hkv

    def sel(lst, total):
        if isinstance(lst, str):
            return -1, None, total, True
        if lst is None:
            return 0, None, 0, False
        a = _idx(lst)
        return len(a), a, len(a), False

    nr, ra, nr_o, r_all = sel(rows, S.batch * S.hq * S.tq)
    nk, ka, nk_o, k_all = sel(keys, S.batch * S.hkv * S.tk)
    ns, sa, ns_o, s_all = sel(sblocks, S.batch * hks * S.nb)
    if z is not None:
        ns, sa, ns_o = 0, None, 0
    dq = np.zeros((nr_o, S.d)); dz = np.zeros((nr_o, S.nb)); dqs = np.zeros((nr_o, S.ds))
    dk = np.zeros((nk_o, S.d)); dv = np.zeros((nk_o, S.d)); dks = np.zeros((ns_o, S.ds))
    st = S.c_struct()
    _check(_load().oracle_attn_bwd(
        ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(qs), _ptr(ks), _ptr(z),
        nr, _ptr(ra), _ptr(dq), _ptr(dz), _ptr(dqs),
        nk, _ptr(ka), _ptr(dk), _ptr(dv),
        ns, _ptr(sa), _ptr(dks)), "attn_bwd")
    out = dict(dq=dq, dz=dz, dqs=dqs, dk=dk, dv=dv, dks=dks)
    if r_all:
        out["dq"] = dq.reshape(S.batch, S.hq, S.tq, S.d)
        out["dz"] = dz.reshape(S.batch, S.hq, S.tq, S.nb)
        out["dqs"] = dqs.reshape(S.batch, S.hq, S.tq, S.ds)
    if k_all:
        out["dk"] = dk.reshape(S.batch, S.hkv, S.tk, S.d)
        out["dv"] = dv.reshape(S.batch, S.hkv, S.tk, S.d)
    if s_all and z is None:
        out["dks"] = dks.reshape(S.batch, hks, S.nb, S.ds)
    if z is not None:
        out["dqs"] = None
        out["dks"] = None
    return out


def topk_blocks(shape: OracleShape, topk: int, qs=None, ks=None, z=None, renorm: int = 0):
    """Returns (idx int32 [B,Hq,Tq,K], bias float64 same shape)."""
    qs, ks, z = map(_f64, (qs, ks, z))
    idx = np.empty((shape.batch, shape.hq, shape.tq, topk), dtype=np.int32)
    bias = np.empty((shape.batch, shape.hq, shape.tq, topk))
    st = shape.c_struct()
    _check(_load().oracle_topk_blocks(ctypes.byref(st), int(topk), int(renorm), _ptr(qs), _ptr(ks),
                                      _ptr(z), _ptr(idx), _ptr(bias)), "topk_blocks")
    return idx, bias


def budget_ratio(frac):
    """The budget fraction as an exact (numerator, denominator): a float is
    read as the decimal it prints as (0.3 -> 3/10), a Fraction or an int as
    is, a (num, den) pair as given; frac <= 0 -> (0, 1), no fraction."""
    if isinstance(frac, tuple):
        num, den = int(frac[0]), int(frac[1])
    else:
        f = Fraction(repr(frac)) if isinstance(frac, float) else Fraction(frac)
        num, den = f.numerator, f.denominator
    if num <= 0:
        return 0, 1
    if den < 1 or num >= 2 ** 31 or den >= 2 ** 31:
        raise ValueError("budget fraction %r does not fit int32" % (frac,))
    return num, den


def topk_budget(shape: OracleShape, kmax: int, frac, qs=None, ks=None, z=None,
                renorm: int = 0):
    """Top-K with n_t = min(kmax, ceil(num * c(t) / den)) blocks per row, the
    fraction num / den taken exactly (see budget_ratio; frac <= 0: the fixed
    budget).  Returns (idx int32 [B,Hq,Tq,kmax], bias float64)."""
    qs, ks, z = map(_f64, (qs, ks, z))
    num, den = budget_ratio(frac)
    idx = np.empty((shape.batch, shape.hq, shape.tq, kmax), dtype=np.int32)
    bias = np.empty((shape.batch, shape.hq, shape.tq, kmax))
    st = shape.c_struct()
    _check(_load().oracle_topk_budget(ctypes.byref(st), int(kmax), num, den,
                                      int(renorm), _ptr(qs), _ptr(ks), _ptr(z), _ptr(idx),
                                      _ptr(bias)), "topk_budget")
    return idx, bias


def threshold_blocks(shape: OracleShape, theta: float, qs=None, ks=None, z=None,
                     renorm: int = 0):
    """Blocks whose normalised gate is >= theta, ascending.  Returns (count int32
    [B,Hq,Tq], idx int32 [B,Hq,Tq,NB] padded -1, bias float64 padded -inf)."""
    qs, ks, z = map(_f64, (qs, ks, z))
    count = np.empty((shape.batch, shape.hq, shape.tq), dtype=np.int32)
    idx = np.empty((shape.batch, shape.hq, shape.tq, shape.nb), dtype=np.int32)
    bias = np.empty((shape.batch, shape.hq, shape.tq, shape.nb))
    st = shape.c_struct()
    _check(_load().oracle_threshold_blocks(ctypes.byref(st), ctypes.c_float(theta), int(renorm),
                                           _ptr(qs), _ptr(ks), _ptr(z), _ptr(count), _ptr(idx),
                                           _ptr(bias)), "threshold_blocks")
    return count, idx, bias


def sparse_fwd(shape: OracleShape, topk: int, q, k, v, idx, bias, rows=None):
    """Sparse forward over the listed blocks + current block.  Returns (o, lse)
    like :func:`attn_fwd`."""
    q, k, v, bias = map(_f64, (q, k, v, bias))
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32))
    rows = _idx(rows)
    n = shape.batch * shape.hq * shape.tq if rows is None else len(rows)
    o = np.empty((n, shape.d))
    lse = np.empty((n,))
    st = shape.c_struct()
    _check(_load().oracle_sparse_fwd(ctypes.byref(st), int(topk), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(idx), _ptr(bias), n, _ptr(rows), _ptr(o), _ptr(lse)),
           "sparse_fwd")
    if rows is None:
        return (o.reshape(shape.batch, shape.hq, shape.tq, shape.d),
                lse.reshape(shape.batch, shape.hq, shape.tq))
    return o, lse
