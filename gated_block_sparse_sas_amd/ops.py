"""Python binding of libsas.so: argument marshalling only.

Each function takes torch tensors on the GPU (PyTorch provides device memory
and the current stream), allocates the outputs, and calls the C entry point of
the same name declared in ``include/sas.h``.  No step of the computation runs
here.  If ``libsas.so`` is missing or a call returns an error status, the call
raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from fractions import Fraction

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SAS_LIBRARY names another build of the same library (the sanitizer run)
LIB_PATH = os.environ.get("SAS_LIBRARY") or os.path.join(_HERE, "libsas.so")
_lib = None

SAS_F32, SAS_BF16 = 0, 1
_STATUS = {0: "SAS_OK", 1: "SAS_ERR_NULL", 2: "SAS_ERR_SHAPE", 3: "SAS_ERR_DTYPE",
           4: "SAS_ERR_ALIGN", 5: "SAS_ERR_UNSUPPORTED", 6: "SAS_ERR_WORKSPACE",
           7: "SAS_ERR_HIP"}
EXPORTS = ("sas_gate_scores", "sas_attn_fwd", "sas_attn_bwd", "sas_attn_bwd_ev",
           "sas_topk_blocks", "sas_topk_blocks_budget", "sas_sparse_fwd", "sas_sparse_fwd_ev",
           "sas_paged_append", "sas_paged_topk", "sas_paged_decode",
           "sas_threshold_count", "sas_threshold_fill", "sas_sparse_fwd_csr",
           "sas_sparse_fwd_csr_ev", "sas_sparse_fwd_noalloc", "sas_noalloc_scratch_bytes",
           "sas_topk_decode", "sas_paged_topk_decode", "sas_status_string",
           "sas_last_hip_error")


class SasError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s failed: %s (%s)" % (fn, _STATUS.get(code, code), msg))
        self.code = code


class Shape(ctypes.Structure):
    """Mirror of ``sas_shape``."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("hks", ctypes.c_int32), ("tq", ctypes.c_int32), ("tk", ctypes.c_int32),
        ("d", ctypes.c_int32), ("ds", ctypes.c_int32), ("block", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("sel_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("sel_dtype", ctypes.c_int32),
    ]


class PagedShape(ctypes.Structure):
    """Mirror of ``sas_paged_shape``."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
        ("hks", ctypes.c_int32), ("d", ctypes.c_int32), ("ds", ctypes.c_int32),
        ("block", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("pages", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("sel_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("sel_dtype", ctypes.c_int32),
    ]


def load():
    """Load libsas.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsas.so not built: run gated_block_sparse_sas_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        P, SZ = ctypes.c_void_p, ctypes.c_void_p
        I32 = ctypes.c_int32
        lib.sas_gate_scores.argtypes = [P, P, P, P, P, P]
        lib.sas_attn_fwd.argtypes = [P, P, P, P, P, P, P, P, P, P]
        lib.sas_attn_bwd.argtypes = [P] * 17 + [SZ, P]
        lib.sas_topk_blocks.argtypes = [P, I32, I32, P, P, P, P, P]
        lib.sas_topk_blocks_budget.argtypes = [P, I32, I32, I32, I32, P, P, P, P, P]
        lib.sas_sparse_fwd.argtypes = [P, I32, P, P, P, P, P, P, P, P, SZ, P]
        lib.sas_attn_bwd_ev.argtypes = [P] * 17 + [SZ, P, I32, P]
        lib.sas_sparse_fwd_ev.argtypes = [P, I32, P, P, P, P, P, P, P, P, SZ, P, I32, P]
        I64 = ctypes.c_int64
        lib.sas_threshold_count.argtypes = [P, ctypes.c_float, P, P, P, P, SZ, P]
        lib.sas_threshold_fill.argtypes = [P, ctypes.c_float, I32, P, P, P, I64, P, P, P]
        lib.sas_sparse_fwd_csr.argtypes = [P, I64] + [P] * 9 + [SZ, P]
        lib.sas_sparse_fwd_csr_ev.argtypes = [P, I64] + [P] * 9 + [SZ, P, I32, P]
        lib.sas_paged_append.argtypes = [P] * 10
        lib.sas_paged_topk.argtypes = [P, I32, I32, P, P, P, P, P, P, P]
        lib.sas_paged_decode.argtypes = [P, I32] + [P] * 10 + [SZ, P]
        lib.sas_sparse_fwd_noalloc.argtypes = [P, I32] + [P] * 8
        lib.sas_topk_decode.argtypes = [P, I32, I32] + [P] * 10
        lib.sas_paged_topk_decode.argtypes = [P, I32, I32] + [P] * 12
        lib.sas_noalloc_scratch_bytes.argtypes = []
        lib.sas_noalloc_scratch_bytes.restype = ctypes.c_size_t
        for n in ("sas_gate_scores", "sas_attn_fwd", "sas_attn_bwd", "sas_topk_blocks",
                  "sas_topk_blocks_budget", "sas_sparse_fwd", "sas_attn_bwd_ev",
                  "sas_sparse_fwd_ev", "sas_paged_append", "sas_paged_topk",
                  "sas_paged_decode", "sas_threshold_count", "sas_threshold_fill",
                  "sas_sparse_fwd_csr", "sas_sparse_fwd_csr_ev", "sas_sparse_fwd_noalloc",
                  "sas_topk_decode", "sas_paged_topk_decode"):
            getattr(lib, n).restype = ctypes.c_int
        lib.sas_status_string.argtypes = [ctypes.c_int]
        lib.sas_status_string.restype = ctypes.c_char_p
        lib.sas_last_hip_error.restype = ctypes.c_int32
        _lib = lib
    return _lib


def _check(fn, code):
    if code != 0:
        lib = load()
        msg = lib.sas_status_string(code).decode()
        if code == 7:
            msg += ", hipError %d" % lib.sas_last_hip_error()
        raise SasError(fn, code, msg)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SAS_BF16
    if t.dtype == torch.float32:
        return SAS_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _p(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (BHSD)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def make_shape(batch, hq, hkv, tq, tk, d, ds, block=64, hks=0, sm_scale=0.0, sel_scale=0.0,
               dtype=SAS_BF16, sel_dtype=None) -> Shape:
    return Shape(batch, hq, hkv, hks, tq, tk, d, ds, block, float(sm_scale or 0.0),
                 float(sel_scale or 0.0), dtype, dtype if sel_dtype is None else sel_dtype)


def shape_of(q, k, qs, ks, block=64, sm_scale=None, sel_scale=None) -> Shape:
    b, hq, tq, d = q.shape
    _, hkv, tk, _ = k.shape
    ds = qs.shape[-1]
    hks = ks.shape[1]
    return make_shape(b, hq, hkv, tq, tk, d, ds, block, hks, sm_scale, sel_scale, _dt(q),
                      _dt(qs))


def gate_scores(qs, ks, tk, block=64, sel_scale=None, with_bias=False):
    """Gate normaliser lam [B,Hq,Tq] (and the log-gate matrix if asked)."""
    b, hq, tq, ds = qs.shape
    hks = ks.shape[1]
    sh = make_shape(b, hq, hks, tq, tk, 64, ds, block, hks, 0.0, sel_scale, _dt(qs), _dt(qs))
    lam = torch.empty((b, hq, tq), dtype=torch.float32, device=qs.device)
    beta = (torch.empty((b, hq, tq, tk // block), dtype=torch.float32, device=qs.device)
            if with_bias else None)
    _check("sas_gate_scores", load().sas_gate_scores(ctypes.byref(sh), _p(qs), _p(ks), _p(lam),
                                                     _p(beta), _stream(qs)))
    return (lam, beta) if with_bias else lam


def attn_fwd(q, k, v, qs, ks, gate_lse, block=64, sm_scale=None, sel_scale=None):
    """Dense-active gated forward.  Returns (o, lse)."""
    sh = shape_of(q, k, qs, ks, block, sm_scale, sel_scale)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check("sas_attn_fwd", load().sas_attn_fwd(ctypes.byref(sh), _p(q), _p(k), _p(v), _p(qs),
                                               _p(ks), _p(gate_lse), _p(o), _p(lse), _stream(q)))
    return o, lse


def bwd_workspace_bytes(sh: Shape, with_dz=True) -> int:
    n = ctypes.c_size_t(0)
    dz_dummy = ctypes.c_void_p(16) if with_dz else None
    _check("sas_attn_bwd", load().sas_attn_bwd(ctypes.byref(sh), *([None] * 14), dz_dummy, None,
                                               ctypes.byref(n), None))
    return n.value


def _events(events):
    if not events:
        return None, 0
    for e in events:
        if e is not None and not e.cuda_event:
            e.record()  # torch creates the hipEvent on first record; the library re-records it
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) if e is not None
                                            else None for e in events])
    return arr, len(events)


def attn_bwd(q, k, v, o, dout, lse, qs, ks, gate_lse, block=64, sm_scale=None, sel_scale=None,
             with_dz=True, ws=None, events=None):
    """Backward of :func:`attn_fwd`.  Returns dict dq, dk, dv, dqs, dks, dz.
    ``events``: optional torch.cuda.Event list recorded between the kernels
    (see ``sas_attn_bwd_ev``)."""
    sh = shape_of(q, k, qs, ks, block, sm_scale, sel_scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dqs = torch.empty_like(qs)
    dks = torch.empty_like(ks)
    dz = (torch.empty(q.shape[:3] + (k.shape[2] // block,), dtype=torch.float32,
                      device=q.device) if with_dz else None)
    need = bwd_workspace_bytes(sh, with_dz)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(ws.numel())
    ev, nev = _events(events)
    _check("sas_attn_bwd", load().sas_attn_bwd_ev(
        ctypes.byref(sh), _p(q), _p(k), _p(v), _p(o), _p(dout), _p(lse), _p(qs), _p(ks),
        _p(gate_lse), _p(dq), _p(dk), _p(dv), _p(dqs), _p(dks), _p(dz), _p(ws), ctypes.byref(n),
        ev, nev, _stream(q)))
    return dict(dq=dq, dk=dk, dv=dv, dqs=dqs, dks=dks, dz=dz)


def topk_blocks(qs, ks, topk, tk, block=64, renorm=0, sel_scale=None):
    """Top-K historical blocks per row.  Returns (idx int32, bias float32)."""
    b, hq, tq, ds = qs.shape
    hks = ks.shape[1]
    sh = make_shape(b, hq, hks, tq, tk, 64, ds, block, hks, 0.0, sel_scale, _dt(qs), _dt(qs))
    idx = torch.empty((b, hq, tq, topk), dtype=torch.int32, device=qs.device)
    bias = torch.empty((b, hq, tq, topk), dtype=torch.float32, device=qs.device)
    _check("sas_topk_blocks", load().sas_topk_blocks(ctypes.byref(sh), int(topk), int(renorm),
                                                     _p(qs), _p(ks), _p(idx), _p(bias),
                                                     _stream(qs)))
    return idx, bias


def _ratio(frac):
    """(numerator, denominator) of a budget fraction: a float is taken as the
    decimal it prints as (0.25 -> 1/4), a Fraction or int as is, a pair as given."""
    if isinstance(frac, tuple):
        num, den = int(frac[0]), int(frac[1])
    else:
        f = Fraction(repr(frac)) if isinstance(frac, float) else Fraction(frac)
        num, den = f.numerator, f.denominator
    return (0, 1) if num <= 0 else (num, den)


def topk_blocks_budget(qs, ks, kmax, frac, tk, block=64, renorm=0, sel_scale=None):
    """Top-K with n_t = min(kmax, c(t), ceil(num c(t) / den)) blocks per row for
    the exact fraction num / den of ``frac`` (<= 0: the fixed budget).  Returns
    (idx int32, bias float32), kmax slots per row."""
    b, hq, tq, ds = qs.shape
    hks = ks.shape[1]
    sh = make_shape(b, hq, hks, tq, tk, 64, ds, block, hks, 0.0, sel_scale, _dt(qs), _dt(qs))
    idx = torch.empty((b, hq, tq, kmax), dtype=torch.int32, device=qs.device)
    bias = torch.empty((b, hq, tq, kmax), dtype=torch.float32, device=qs.device)
    _check("sas_topk_blocks_budget",
           load().sas_topk_blocks_budget(ctypes.byref(sh), int(kmax), *_ratio(frac),
                                         int(renorm), _p(qs), _p(ks), _p(idx), _p(bias),
                                         _stream(qs)))
    return idx, bias


def sparse_workspace_bytes(sh: Shape, topk: int) -> int:
    n = ctypes.c_size_t(0)
    _check("sas_sparse_fwd", load().sas_sparse_fwd(ctypes.byref(sh), int(topk), *([None] * 7),
                                                   None, ctypes.byref(n), None))
    return n.value


def sparse_fwd(q, k, v, idx, bias, block=64, sm_scale=None, ws=None, with_lse=True,
               events=None):
    """Top-K sparse forward (prefill or decode).  Returns (o, lse)."""
    b, hq, tq, d = q.shape
    _, hkv, tk, _ = k.shape
    topk = idx.shape[-1]
    sh = make_shape(b, hq, hkv, tq, tk, d, 32, block, hkv, sm_scale, 0.0, _dt(q), _dt(q))
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, tq), dtype=torch.float32, device=q.device) if with_lse else None
    need = sparse_workspace_bytes(sh, topk)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(ws.numel())
    ev, nev = _events(events)
    _check("sas_sparse_fwd", load().sas_sparse_fwd_ev(
        ctypes.byref(sh), int(topk), _p(q), _p(k), _p(v), _p(idx), _p(bias), _p(o), _p(lse),
        _p(ws), ctypes.byref(n), ev, nev, _stream(q)))
    return o, lse


def topk_decode(q, k, v, qs, ks, topk, block=64, renorm=0, sm_scale=None, sel_scale=None,
                with_sel=True, with_lse=True):
    """Top-K selection and sparse forward in one call (``sas_topk_decode``):
    the results of :func:`topk_blocks` then :func:`sparse_fwd`.  Returns (o,
    lse, idx, bias); idx / bias None when ``with_sel`` is False."""
    b, hq, tq, d = q.shape
    _, hkv, tk, _ = k.shape
    ds, hks = qs.shape[-1], ks.shape[1]
    sh = make_shape(b, hq, hkv, tq, tk, d, ds, block, hks, sm_scale, sel_scale, _dt(q), _dt(qs))
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, tq), dtype=torch.float32, device=q.device) if with_lse else None
    idx = (torch.empty((b, hq, tq, topk), dtype=torch.int32, device=q.device) if with_sel
           else None)
    bias = (torch.empty((b, hq, tq, topk), dtype=torch.float32, device=q.device) if with_sel
            else None)
    _check("sas_topk_decode", load().sas_topk_decode(
        ctypes.byref(sh), int(topk), int(renorm), _p(q), _p(k), _p(v), _p(qs), _p(ks), _p(idx),
        _p(bias), _p(o), _p(lse), _stream(q)))
    return o, lse, idx, bias


def sparse_fwd_noalloc(q, k, v, idx, bias, block=64, sm_scale=None, with_lse=True):
    """:func:`sparse_fwd` through ``sas_sparse_fwd_noalloc``: the library's fixed
    scratch array instead of a workspace.  Returns (o, lse)."""
    b, hq, tq, d = q.shape
    _, hkv, tk, _ = k.shape
    topk = idx.shape[-1]
    sh = make_shape(b, hq, hkv, tq, tk, d, 32, block, hkv, sm_scale, 0.0, _dt(q), _dt(q))
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, tq), dtype=torch.float32, device=q.device) if with_lse else None
    _check("sas_sparse_fwd_noalloc", load().sas_sparse_fwd_noalloc(
        ctypes.byref(sh), int(topk), _p(q), _p(k), _p(v), _p(idx), _p(bias), _p(o), _p(lse),
        _stream(q)))
    return o, lse


# ---------------------------------------------------------------------------
# Paged decode cache: pools [pages, hkv, 64, d] (K, V) and [pages, hks, ds]
# (selector keys), block_table [batch, max_blocks] int32, seq_len [batch] int32.

def make_paged_shape(batch, hq, hkv, d, ds, max_blocks, pages, hks=0, block=64, sm_scale=0.0,
                     sel_scale=0.0, dtype=SAS_BF16) -> PagedShape:
    return PagedShape(batch, hq, hkv, hks, d, ds, block, max_blocks, pages,
                      float(sm_scale or 0.0), float(sel_scale or 0.0), dtype, dtype)


def paged_append(pos, block_table, k_new, v_new, k_pool, v_pool, ks_new=None, ks_pool=None):
    """Write one token per sequence (k_new, v_new [batch, hkv, d]) at position pos[b];
    with ks_new [batch, hks, ds], store the selector key of every block completed."""
    pages, hkv, _, d = k_pool.shape
    batch, max_blocks = block_table.shape
    hks, ds = (ks_pool.shape[1], ks_pool.shape[2]) if ks_pool is not None else (hkv, 16)
    sh = make_paged_shape(batch, hkv, hkv, d, ds, max_blocks, pages, hks, dtype=_dt(k_pool))
    _check("sas_paged_append", load().sas_paged_append(
        ctypes.byref(sh), _p(pos), _p(block_table), _p(k_new), _p(v_new), _p(ks_new),
        _p(k_pool), _p(v_pool), _p(ks_pool), _stream(k_pool)))


def paged_topk(qs, ks_pool, block_table, seq_len, topk, renorm=0, sel_scale=None):
    """Top-K historical blocks of each sequence's query: qs [batch, hq, ds].
    Returns (idx [batch, hq, topk] int32, bias float32)."""
    batch, hq, ds = qs.shape
    pages, hks, _ = ks_pool.shape
    max_blocks = block_table.shape[1]
    sh = make_paged_shape(batch, hq, hks, 64, ds, max_blocks, pages, hks, sel_scale=sel_scale,
                          dtype=_dt(qs))
    idx = torch.empty((batch, hq, topk), dtype=torch.int32, device=qs.device)
    bias = torch.empty((batch, hq, topk), dtype=torch.float32, device=qs.device)
    _check("sas_paged_topk", load().sas_paged_topk(
        ctypes.byref(sh), int(topk), int(renorm), _p(seq_len), _p(block_table), _p(qs),
        _p(ks_pool), _p(idx), _p(bias), _stream(qs)))
    return idx, bias


def paged_topk_decode(q, k_pool, v_pool, qs, ks_pool, block_table, seq_len, topk, renorm=0,
                      sm_scale=None, sel_scale=None, with_sel=True, with_lse=True):
    """:func:`paged_topk` then :func:`paged_decode` in one call
    (``sas_paged_topk_decode``).  Returns (o, lse, idx, bias)."""
    batch, hq, d = q.shape
    pages, hkv, _, _ = k_pool.shape
    ds, hks = qs.shape[-1], ks_pool.shape[1]
    max_blocks = block_table.shape[1]
    sh = make_paged_shape(batch, hq, hkv, d, ds, max_blocks, pages, hks, sm_scale=sm_scale,
                          sel_scale=sel_scale, dtype=_dt(q))
    o = torch.empty_like(q)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if with_lse else None
    idx = (torch.empty((batch, hq, topk), dtype=torch.int32, device=q.device) if with_sel
           else None)
    bias = (torch.empty((batch, hq, topk), dtype=torch.float32, device=q.device) if with_sel
            else None)
    _check("sas_paged_topk_decode", load().sas_paged_topk_decode(
        ctypes.byref(sh), int(topk), int(renorm), _p(seq_len), _p(block_table), _p(q),
        _p(k_pool), _p(v_pool), _p(qs), _p(ks_pool), _p(idx), _p(bias), _p(o), _p(lse),
        _stream(q)))
    return o, lse, idx, bias


def paged_workspace_bytes(sh: PagedShape, topk: int) -> int:
    n = ctypes.c_size_t(0)
    _check("sas_paged_decode", load().sas_paged_decode(ctypes.byref(sh), int(topk), *([None] * 10),
                                                       ctypes.byref(n), None))
    return n.value


def paged_decode(q, k_pool, v_pool, block_table, seq_len, idx, bias, sm_scale=None, ws=None,
                 with_lse=True):
    """Top-K sparse decode over the pools: q [batch, hq, d].  Returns (o, lse)."""
    batch, hq, d = q.shape
    pages, hkv, _, _ = k_pool.shape
    max_blocks = block_table.shape[1]
    topk = idx.shape[-1]
    sh = make_paged_shape(batch, hq, hkv, d, 16, max_blocks, pages, sm_scale=sm_scale,
                          dtype=_dt(q))
    o = torch.empty_like(q)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device) if with_lse else None
    need = paged_workspace_bytes(sh, topk)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(ws.numel())
    _check("sas_paged_decode", load().sas_paged_decode(
        ctypes.byref(sh), int(topk), _p(seq_len), _p(block_table), _p(q), _p(k_pool), _p(v_pool),
        _p(idx), _p(bias), _p(o), _p(lse), _p(ws), ctypes.byref(n), _stream(q)))
    return o, lse


# ---------------------------------------------------------------------------
# Dynamic-threshold selection (CSR) and the sparse forward over it.

def _thr_shape(qs, ks, tk, block, sel_scale):
    b, hq, tq, ds = qs.shape
    hks = ks.shape[1]
    return make_shape(b, hq, hks, tq, tk, 64, ds, block, hks, 0.0, sel_scale, _dt(qs), _dt(qs))


def threshold_count(qs, ks, theta, tk, block=64, sel_scale=None, ws=None):
    """Pass 1 of the threshold selection: row_ptr int64 [rows+1] (device), rows in
    BHSD order; nnz = row_ptr[-1] once the stream reaches it."""
    b, hq, tq, _ = qs.shape
    sh = _thr_shape(qs, ks, tk, block, sel_scale)
    lib = load()
    n = ctypes.c_size_t(0)
    _check("sas_threshold_count", lib.sas_threshold_count(
        ctypes.byref(sh), ctypes.c_float(theta), None, None, None, None, ctypes.byref(n), None))
    if ws is None or ws.numel() < n.value:
        ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=qs.device)
    row_ptr = torch.empty(b * hq * tq + 1, dtype=torch.int64, device=qs.device)
    n = ctypes.c_size_t(ws.numel())
    _check("sas_threshold_count", lib.sas_threshold_count(
        ctypes.byref(sh), ctypes.c_float(theta), _p(qs), _p(ks), _p(row_ptr), _p(ws),
        ctypes.byref(n), _stream(qs)))
    return row_ptr


def threshold_fill(qs, ks, theta, tk, row_ptr, nnz, block=64, renorm=0, sel_scale=None):
    """Pass 2: (col int32 [nnz], bias float32 [nnz]) for the row_ptr of pass 1."""
    sh = _thr_shape(qs, ks, tk, block, sel_scale)
    col = torch.empty(max(nnz, 1), dtype=torch.int32, device=qs.device)
    bias = torch.empty(max(nnz, 1), dtype=torch.float32, device=qs.device)
    _check("sas_threshold_fill", load().sas_threshold_fill(
        ctypes.byref(sh), ctypes.c_float(theta), int(renorm), _p(qs), _p(ks), _p(row_ptr),
        ctypes.c_int64(nnz), _p(col), _p(bias), _stream(qs)))
    return col[:nnz], bias[:nnz]


def threshold_blocks(qs, ks, theta, tk, block=64, renorm=0, sel_scale=None, capacity=None):
    """Blocks whose normalised gate is >= theta.  Returns (row_ptr int64 [rows+1],
    col int32 [n], bias float32 [n]); rows = batch*hq*tq in BHSD order.

    capacity None: reads nnz = row_ptr[-1] back to the host between the two
    passes (one stream synchronisation) and n = nnz.  capacity = n: nothing is
    read back; the fill writes the entries below n and the arrays have n
    entries, those past row_ptr[-1] belonging to no row (sparse_fwd_csr skips
    them).  The selection is complete iff row_ptr[-1] <= n, which the caller
    checks whenever it next synchronises."""
    row_ptr = threshold_count(qs, ks, theta, tk, block, sel_scale)
    nnz = int(row_ptr[-1].item()) if capacity is None else int(capacity)
    col, bias = threshold_fill(qs, ks, theta, tk, row_ptr, nnz, block, renorm, sel_scale)
    return row_ptr, col, bias


def sparse_csr_workspace_bytes(sh: Shape, nnz: int) -> int:
    n = ctypes.c_size_t(0)
    _check("sas_sparse_fwd_csr", load().sas_sparse_fwd_csr(
        ctypes.byref(sh), ctypes.c_int64(nnz), *([None] * 9), ctypes.byref(n), None))
    return n.value


def sparse_fwd_csr(q, k, v, row_ptr, col, bias, block=64, sm_scale=None, ws=None, with_lse=True,
                   events=None):
    """Sparse forward over a CSR selection (rows in BHSD order).  Returns (o, lse)."""
    b, hq, tq, d = q.shape
    _, hkv, tk, _ = k.shape
    nnz = int(col.numel())
    sh = make_shape(b, hq, hkv, tq, tk, d, 32, block, hkv, sm_scale, 0.0, _dt(q), _dt(q))
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, tq), dtype=torch.float32, device=q.device) if with_lse else None
    need = sparse_csr_workspace_bytes(sh, nnz)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(ws.numel())
    ev, nev = _events(events)
    colp = _p(col) if nnz else None
    biasp = _p(bias) if nnz else None
    _check("sas_sparse_fwd_csr", load().sas_sparse_fwd_csr_ev(
        ctypes.byref(sh), ctypes.c_int64(nnz), _p(row_ptr), colp, biasp, _p(q), _p(k), _p(v),
        _p(o), _p(lse), _p(ws), ctypes.byref(n), ev, nev, _stream(q)))
    return o, lse
