"""Host-side checks of libsas.so (no GPU needed, no kernel is launched).

* the library loads and exports every function ``include/sas.h`` declares;
* every argument check returns its documented status before any launch;
* the workspace size queries answer without launching anything.
"""

import ctypes
import os
import re

import pytest

from gated_block_sparse_sas_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from gated_block_sparse_sas_amd import build
        build.build()
    return ops.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"sas_gate_scores", "sas_attn_fwd", "sas_attn_bwd", "sas_topk_blocks",
                          "sas_sparse_fwd", "sas_status_string"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(ops.EXPORTS) == set(names)


def test_oracle_exports(oracle_mod):
    lib = ctypes.CDLL(oracle_mod.build(force=False))
    text = open(os.path.join(ROOT, "oracle", "sas_oracle.h")).read()
    for n in set(re.findall(r"\b(oracle_[a-z_]+)\s*\(", text)):
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(8):
        s = lib.sas_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.sas_status_string(99).decode() == "unknown status"


# Fake, 16-byte aligned device addresses: every call below fails a host check
# (or is a size query / empty call) before any pointer is dereferenced.
A = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10004)
STREAM = None


def shape(**kw):
    base = dict(batch=1, hq=4, hkv=2, tq=256, tk=256, d=128, ds=32, block=64, hks=0, sm_scale=0.0,
                sel_scale=0.0, dtype=ops.SAS_BF16)
    base.update(kw)
    return ops.make_shape(**base)


def fwd(lib, sh, **ptrs):
    p = dict(q=A, k=A, v=A, qs=A, ks=A, lam=A, o=A, lse=A)
    p.update(ptrs)
    return lib.sas_attn_fwd(ctypes.byref(sh) if sh is not None else None, p["q"], p["k"], p["v"],
                            p["qs"], p["ks"], p["lam"], p["o"], p["lse"], STREAM)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=3), 2),                 # hq % hkv
    (dict(hks=3), 2),                # hq % hks
    (dict(tq=300), 2),               # tq > tk
    (dict(tq=0), 2),
    (dict(batch=-1), 2),
    (dict(dtype=7), 3),
    (dict(sel_dtype=ops.SAS_F32), 3),  # mixed dtypes
    (dict(block=128), 5),              # units of at most 64 tokens
    (dict(block=24), 5),               # units: powers of two
    (dict(tk=250, tq=250), 5),       # tk % 64
    (dict(d=96), 5),
    (dict(ds=24), 5),
    (dict(dtype=ops.SAS_F32, sel_dtype=ops.SAS_F32, d=128), 5),  # fp32 path is d=64 only
])
def test_fwd_shape_checks(lib, kw, code):
    assert fwd(lib, shape(**kw)) == code


def test_fwd_pointer_checks(lib):
    assert fwd(lib, None) == 1
    for n in ("q", "k", "v", "qs", "ks", "lam", "o", "lse"):
        assert fwd(lib, shape(), **{n: None}) == 1, n
        assert fwd(lib, shape(), **{n: MIS}) == 4, n


def test_empty_batch_is_noop(lib):
    assert fwd(lib, shape(batch=0)) == 0
    assert lib.sas_gate_scores(ctypes.byref(shape(batch=0)), A, A, A, None, STREAM) == 0


def test_gate_checks(lib):
    assert lib.sas_gate_scores(ctypes.byref(shape()), None, A, A, None, STREAM) == 1
    assert lib.sas_gate_scores(ctypes.byref(shape()), A, A, A, MIS, STREAM) == 4


def test_topk_checks(lib):
    sh = shape()
    assert lib.sas_topk_blocks(ctypes.byref(sh), 0, 0, A, A, A, A, STREAM) == 2
    assert lib.sas_topk_blocks(ctypes.byref(sh), 4, 2, A, A, A, A, STREAM) == 2
    assert lib.sas_topk_blocks(ctypes.byref(sh), 4, 0, A, A, None, A, STREAM) == 1
    assert lib.sas_topk_blocks(ctypes.byref(sh), 4, 0, A, A, A, MIS, STREAM) == 4
    # topk > 16 with few rows keeps nb + 256 + 2 next_pow2(K) floats of LDS per
    # row: past 64 KiB unsupported; topk <= 16 takes the kernel without LDS
    big = shape(tk=1 << 20, tq=64)
    assert lib.sas_topk_blocks(ctypes.byref(big), 40, 0, A, A, A, A, STREAM) == 5
    assert lib.sas_topk_blocks(ctypes.byref(shape(tk=1 << 20, tq=64, batch=0)), 4, 0, A, A, A,
                               A, STREAM) == 0


def test_topk_budget_checks(lib):
    sh = shape()
    i32 = ctypes.c_int32
    lib.sas_topk_blocks_budget.argtypes = [ctypes.c_void_p, i32, i32, i32,
                                           i32] + [ctypes.c_void_p] * 5
    fn = lib.sas_topk_blocks_budget
    assert fn(ctypes.byref(sh), 0, 1, 4, 0, A, A, A, A, STREAM) == 2       # kmax < 1
    assert fn(ctypes.byref(sh), 8, 1, 4, 2, A, A, A, A, STREAM) == 2       # renorm
    assert fn(ctypes.byref(sh), 8, 1, 0, 0, A, A, A, A, STREAM) == 2       # denominator 0
    assert fn(ctypes.byref(sh), 8, 1, -4, 0, A, A, A, A, STREAM) == 2      # negative denominator
    assert fn(ctypes.byref(sh), 8, 1, 4, 0, None, A, A, A, STREAM) == 1
    assert fn(ctypes.byref(sh), 8, 1, 4, 0, A, A, A, MIS, STREAM) == 4
    assert fn(ctypes.byref(sh), 2048, 1, 4, 0, A, A, A, A, STREAM) == 5
    big = shape(tk=1 << 20, tq=64)  # the row's scores no longer fit the kernel's LDS
    assert fn(ctypes.byref(big), 8, 1, 4, 0, A, A, A, A, STREAM) == 5
    assert fn(ctypes.byref(shape(batch=0)), 8, 1, 4, 0, A, A, A, A, STREAM) == 0
    # no fraction (numerator <= 0) and fractions above one are valid
    assert fn(ctypes.byref(shape(batch=0)), 8, 0, 1, 0, A, A, A, A, STREAM) == 0
    assert fn(ctypes.byref(shape(batch=0)), 8, 5, 2, 0, A, A, A, A, STREAM) == 0


def bwd(lib, sh, ws, n, **ptrs):
    names = ("q", "k", "v", "o", "dout", "lse", "qs", "ks", "lam", "dq", "dk", "dv", "dqs", "dks")
    p = {k: A for k in names}
    p.update(ptrs)
    dz = ptrs.get("dz", A)
    return lib.sas_attn_bwd(ctypes.byref(sh), *[p[k] for k in names], dz, ws,
                            ctypes.byref(n) if n is not None else None, STREAM)


def test_bwd_workspace_query_and_checks(lib):
    sh = shape()
    n = ctypes.c_size_t(0)
    assert bwd(lib, sh, None, n) == 0
    rows = 1 * 4 * 256
    need_min = rows * 4 + 1 * 2 * 4 * 32 * 4  # delta + dks accumulator
    assert n.value >= need_min
    n2 = ctypes.c_size_t(0)
    assert bwd(lib, sh, None, n2, dz=None) == 0
    assert n2.value >= n.value + rows * 4 * 4  # dz kept in the workspace
    small = ctypes.c_size_t(n.value - 1)
    assert bwd(lib, sh, A, small) == 6
    assert bwd(lib, sh, A, None) == 1
    ok = ctypes.c_size_t(n.value)
    assert bwd(lib, sh, A, ok, dq=None) == 1
    assert bwd(lib, sh, A, ok, dks=MIS) == 4


def test_sparse_workspace_query_and_checks(lib):
    sh = shape()
    n = ctypes.c_size_t(0)
    assert lib.sas_sparse_fwd(ctypes.byref(sh), 4, *([None] * 7), None, ctypes.byref(n),
                              STREAM) == 0
    # 4 of the 2 historical blocks on average: the dense-kernel path, whose
    # workspace is the per-(block, row) bias matrix (batch * hq * nb * tq floats)
    assert n.value >= 1 * 4 * 4 * 256 * 4
    sparse = shape(tq=4096, tk=4096)  # 2 of 32 blocks on average: partials per (row, slot)
    m = ctypes.c_size_t(0)
    assert lib.sas_sparse_fwd(ctypes.byref(sparse), 2, *([None] * 7), None, ctypes.byref(m),
                              STREAM) == 0
    assert m.value >= 1 * 4 * 4096 * 2 * (2 * 128 + 4)
    small = ctypes.c_size_t(n.value - 1)
    assert lib.sas_sparse_fwd(ctypes.byref(sh), 4, A, A, A, A, A, A, None, A,
                              ctypes.byref(small), STREAM) == 6
    assert lib.sas_sparse_fwd(ctypes.byref(sh), 0, A, A, A, A, A, A, None, A,
                              ctypes.byref(n), STREAM) == 2
    assert lib.sas_sparse_fwd(ctypes.byref(sh), 4, A, A, A, None, A, A, None, A,
                              ctypes.byref(n), STREAM) == 1


def pshape(**kw):
    a = dict(batch=2, hq=4, hkv=2, d=128, ds=32, max_blocks=8, pages=20)
    a.update(kw)
    return ops.make_paged_shape(a["batch"], a["hq"], a["hkv"], a["d"], a["ds"], a["max_blocks"],
                                a["pages"], hks=a.get("hks", 0), block=a.get("block", 64))


@pytest.mark.parametrize("kw,code", [
    (dict(block=32), 5), (dict(d=96), 5), (dict(ds=48), 5), (dict(hq=3), 2),
    (dict(max_blocks=0), 2), (dict(pages=0), 2), (dict(batch=-1), 2), (dict(hks=3), 2),
])
def test_paged_shape_checks(lib, kw, code):
    sh = pshape(**kw)
    n = ctypes.c_size_t(0)
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *([None] * 10), ctypes.byref(n),
                                STREAM) == code
    assert lib.sas_paged_topk(ctypes.byref(sh), 4, 0, A, A, A, A, A, A, STREAM) == code
    assert lib.sas_paged_append(ctypes.byref(sh), A, A, A, A, None, A, A, None, STREAM) == code


def test_paged_checks(lib):
    sh = pshape()
    n = ctypes.c_size_t(0)
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *([None] * 10), ctypes.byref(n),
                                STREAM) == 0
    assert n.value > 0
    small = ctypes.c_size_t(n.value - 1)
    args = [A] * 8 + [None, A]  # lse NULL is allowed
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *args, ctypes.byref(small), STREAM) == 6
    assert lib.sas_paged_decode(ctypes.byref(sh), 0, *args, ctypes.byref(n), STREAM) == 2
    bad = list(args)
    bad[2] = None  # q
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *bad, ctypes.byref(n), STREAM) == 1
    bad[2] = MIS
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *bad, ctypes.byref(n), STREAM) == 4
    assert lib.sas_paged_decode(ctypes.byref(sh), 4, *args, None, STREAM) == 1
    # top-K: budget, renorm, pointers, LDS limit
    assert lib.sas_paged_topk(ctypes.byref(sh), 0, 0, A, A, A, A, A, A, STREAM) == 2
    assert lib.sas_paged_topk(ctypes.byref(sh), 4, 2, A, A, A, A, A, A, STREAM) == 2
    assert lib.sas_paged_topk(ctypes.byref(sh), 4, 0, A, None, A, A, A, A, STREAM) == 1
    big = pshape(max_blocks=20000)  # topk > 16: LDS per row past 64 KiB
    assert lib.sas_paged_topk(ctypes.byref(big), 40, 0, A, A, A, A, A, A, STREAM) == 5
    # append: ks_new without ks_pool, misaligned pool
    assert lib.sas_paged_append(ctypes.byref(sh), A, A, A, A, A, A, A, None, STREAM) == 1
    assert lib.sas_paged_append(ctypes.byref(sh), A, A, A, A, None, MIS, A, None, STREAM) == 4
    # dtype mismatch
    sh2 = pshape()
    sh2.sel_dtype = ops.SAS_F32
    assert lib.sas_paged_topk(ctypes.byref(sh2), 4, 0, A, A, A, A, A, A, STREAM) == 3
    # empty batch: nothing launched
    e = pshape(batch=0)
    assert lib.sas_paged_append(ctypes.byref(e), A, A, A, A, None, A, A, None, STREAM) == 0
    assert lib.sas_paged_topk(ctypes.byref(e), 4, 0, A, A, A, A, A, A, STREAM) == 0


def test_threshold_and_csr_checks(lib):
    sh = shape()
    n = ctypes.c_size_t(0)
    F = ctypes.c_float
    # size queries
    assert lib.sas_threshold_count(ctypes.byref(sh), F(0.1), None, None, None, None,
                                   ctypes.byref(n), STREAM) == 0
    assert n.value >= 8
    small = ctypes.c_size_t(n.value - 1)
    assert lib.sas_threshold_count(ctypes.byref(sh), F(0.1), A, A, A, A, ctypes.byref(small),
                                   STREAM) == 6
    assert lib.sas_threshold_count(ctypes.byref(sh), F(float("nan")), A, A, A, A,
                                   ctypes.byref(n), STREAM) == 2
    assert lib.sas_threshold_count(ctypes.byref(sh), F(0.1), A, None, A, A, ctypes.byref(n),
                                   STREAM) == 1
    assert lib.sas_threshold_count(ctypes.byref(sh), F(0.1), A, A, MIS, A, ctypes.byref(n),
                                   STREAM) == 4
    # fill: nnz < 0, renorm, NULL col with nnz > 0; nnz == 0 launches nothing
    assert lib.sas_threshold_fill(ctypes.byref(sh), F(0.1), 0, A, A, A, -1, A, A, STREAM) == 2
    assert lib.sas_threshold_fill(ctypes.byref(sh), F(0.1), 3, A, A, A, 5, A, A, STREAM) == 2
    assert lib.sas_threshold_fill(ctypes.byref(sh), F(0.1), 0, A, A, A, 5, None, A, STREAM) == 1
    assert lib.sas_threshold_fill(ctypes.byref(sh), F(0.1), 0, A, A, A, 0, None, None,
                                  STREAM) == 0
    # CSR sparse forward: size query grows with nnz, checks
    n0, n1 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), 0, *([None] * 9), ctypes.byref(n0),
                                  STREAM) == 0
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), 1000, *([None] * 9), ctypes.byref(n1),
                                  STREAM) == 0
    assert n1.value > n0.value
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), -1, *([None] * 9), ctypes.byref(n0),
                                  STREAM) == 2
    args = [A, A, A, A, A, A, A, None, A]  # row_ptr col bias q k v o lse ws
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), 1000, *args, ctypes.byref(n0), STREAM) == 6
    bad = list(args)
    bad[0] = None
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), 1000, *bad, ctypes.byref(n1), STREAM) == 1
    f32 = shape(dtype=ops.SAS_F32, d=64)
    assert lib.sas_sparse_fwd_csr(ctypes.byref(f32), 10, *args, ctypes.byref(n1), STREAM) == 5


def test_block_size_support(lib):
    # gate blocks of 1 .. 64 tokens (powers of two), in the gate and the forward
    for blk, ok in ((1, True), (2, True), (8, True), (16, True), (32, True), (64, True),
                    (48, False), (128, False)):
        for dt, d in ((ops.SAS_F32, 64), (ops.SAS_BF16, 128), (ops.SAS_BF16, 64)):
            sh = shape(batch=0, block=blk, dtype=dt, d=d)
            r_gate = lib.sas_gate_scores(ctypes.byref(sh), A, A, A, None, STREAM)
            r_fwd = fwd(lib, sh)
            assert r_gate == (0 if ok else 5), (blk, dt)
            assert r_fwd == (0 if ok else 5), (blk, dt, r_fwd)
    # bf16 backward: units of 16, 32, 64 tokens at d = 128 (and 1 .. 8 with
    # ds = 32), 64 tokens at d = 64
    n = ctypes.c_size_t(1 << 30)
    for blk, d, ds, want in ((32, 128, 32, 0), (16, 128, 32, 0), (8, 128, 32, 0),
                             (1, 128, 32, 0), (4, 128, 16, 5), (2, 128, 64, 5), (32, 64, 32, 5),
                             (64, 64, 32, 0)):
        bw = shape(batch=0, block=blk, d=d, ds=ds)
        assert lib.sas_attn_bwd(ctypes.byref(bw), *([A] * 15), A, ctypes.byref(n),
                                STREAM) == want, (blk, d, ds)
    # CSR and fixed-budget sparse forwards: any supported unit size
    n = ctypes.c_size_t(0)
    sh = shape(block=16)
    assert lib.sas_sparse_fwd_csr(ctypes.byref(sh), 10, *([None] * 9), ctypes.byref(n),
                                  STREAM) == 0
    assert lib.sas_sparse_fwd(ctypes.byref(sh), 4, *([None] * 7), None, ctypes.byref(n),
                              STREAM) == 0


def test_fused_decode_checks(lib):
    # sas_topk_decode: q k v qs ks idx bias o lse; idx, bias, lse optional
    sh = shape(tq=1)
    f = lib.sas_topk_decode
    assert f(ctypes.byref(sh), 0, 0, *([A] * 10), STREAM) == 2       # topk < 1
    assert f(ctypes.byref(sh), 4, 2, *([A] * 10), STREAM) == 2       # renorm
    assert f(ctypes.byref(sh), 17, 0, *([A] * 10), STREAM) == 5      # topk > 16
    assert f(ctypes.byref(sh), 4, 0, None, *([A] * 9), STREAM) == 1  # q NULL
    args = [A] * 5 + [None, None, A, None]                          # no idx / bias / lse
    assert f(ctypes.byref(shape(tq=1, batch=0)), 4, 0, *args, STREAM) == 0
    assert f(ctypes.byref(sh), 4, 0, *([A] * 5), MIS, A, A, A, STREAM) == 4
    assert f(None, 4, 0, *([A] * 10), STREAM) == 1
    # sas_paged_topk_decode: seq_len table q k_pool v_pool qs ks_pool idx bias o lse
    g = lib.sas_paged_topk_decode
    ps = pshape()
    assert g(ctypes.byref(ps), 0, 0, *([A] * 12), STREAM) == 2
    assert g(ctypes.byref(ps), 17, 0, *([A] * 12), STREAM) == 5
    assert g(ctypes.byref(ps), 4, 0, A, None, *([A] * 10), STREAM) == 1   # table NULL
    assert g(ctypes.byref(pshape(batch=0)), 4, 0, *([A] * 7), None, None, A, None, STREAM) == 0
