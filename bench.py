#!/usr/bin/env python
"""Benchmark of the SAS gated block-sparse attention hot path on one MI355X.

One step is one pass of the whole hot path on resident synthetic inputs:
  train_32k          gate normaliser -> gated forward -> backward (dq, dk, dv,
                     dz, dqs, dks): batch 1, 32 query / 8 kv heads, d 128,
                     T 32768, 64-token blocks, selector dim 32, bf16
  prefill_32k_top16  top-K block selection -> top-K sparse forward (K = 16)
  decode_64k_top8    top-K selection -> sparse decode, 16 sequences x 64k keys
  prefill_32k_top25pct  budgeted top-K selection (a quarter of each query's
                     history, at most 128 blocks) -> top-K sparse forward
  decode_paged_mix   decode over a block-paged cache: 32 sequences of mixed
                     lengths (64 .. 65536 tokens), top-K selection -> decode
  (both decodes also once more as one fused selection + decode launch)
  decode_64k_b16_top32  16-token context units: top-K (K = 32) -> sparse decode
  prefill_32k_b16_top64 16-token context units: top-K (K = 64) -> sparse prefill
  prefill_32k_theta  dynamic-threshold selection (normalised gate >= 0.01, CSR:
                     count, fill into a capacity of 9/8 of the set-up count, no
                     host read in between) -> sparse forward over CSR
  train_32k_b1       train_32k with token-level context units (one selector
                     key per token): gate -> forward -> backward (no dense dz)
The headline value is the training fwd+bwd rate at 32k in TFLOP/s counting
attended (row, key) pairs only (forward 4*d flop per pair, backward 10*d).
Times come from HIP events recorded on the stream the kernels run on.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
from fractions import Fraction
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "gated-attn fwd+bwd TFLOP/s @32k bf16 (% MFMA peak); top-K sparse fwd TFLOP/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(tq, tk):
    """Attended (row, key) pairs of one head of dense causal attention."""
    qoff = tk - tq
    return sum(qoff + i + 1 for i in range(tq))


def sparse_pairs(w):
    """Attended pairs of one head under a top-K block budget (current block
    causal + n(t) full historical blocks, n(t) = min(K, c), further capped at
    ceil(num c / den) for a budget that is the fraction num / den of the history)."""
    tot = 0
    fr = Fraction(repr(w.frac)) if w.frac > 0 else None
    for i in range(w.tq):
        t = w.tk - w.tq + i
        c = t // w.block
        n = min(w.topk, c)
        if fr is not None:
            n = min(n, -(-fr.numerator * c // fr.denominator))
        tot += n * w.block + (t - c * w.block + 1)
    return tot


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(T: int):
    """The fp64 oracle, timed on a bounded sample of the 32k training job."""
    import numpy as np
    import oracle
    from gated_block_sparse_sas_amd import synth
    oracle.build(force=False)
    w = synth.WORKLOADS["train_32k"]
    cpu = synth.draw_all(w)
    # causal prefix of T tokens of kv group 0 (query heads 0..3)
    hpg = w.hq // w.hkv
    x = {
        "q": synth.to_f64(cpu["q"][:, :hpg, :T]),
        "k": synth.to_f64(cpu["k"][:, :1, :T]),
        "v": synth.to_f64(cpu["v"][:, :1, :T]),
        "qs": synth.to_f64(cpu["qs"][:, :hpg, :T]),
        "ks": synth.to_f64(cpu["ks"][:, :1, :T // w.block]),
        "dout": synth.to_f64(cpu["dout"][:, :hpg, :T]),
    }
    S = oracle.OracleShape(1, hpg, 1, T, T, w.d, w.ds, w.block)
    t0 = time.perf_counter()
    oracle.attn_fwd(S, x["q"], x["k"], x["v"], x["qs"], x["ks"])
    oracle.attn_bwd(S, x["q"], x["k"], x["v"], x["dout"], x["qs"], x["ks"])
    dt = time.perf_counter() - t0
    flop = 14.0 * w.d * hpg * causal_pairs(T, T)
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": ("fp64 oracle forward+backward (dq, dk, dv, dz, dqs, dks) on the causal "
                   "prefix of %d tokens of kv group 0 (4 query heads) of train_32k; %.1f s; "
                   "attended flop counted as on the GPU" % (T, dt)),
        "seconds": dt,
        "cpu": cpu_model(),
    }


# Kernel symbol of each timed part, as a profiler lists it, and the sources it
# is built from (a change to any of them voids stored HBM-traffic counters).
KERNELS = {
    "bwd_dkdv": ("bwd_dkdv16_kernel<32, 1>", ("attn_bwd.hip", "sas_device.h", "sas_internal.h")),
    "bwd_dq": ("bwd_dq32_kernel<32, 1>", ("attn_bwd.hip", "sas_device.h", "sas_internal.h")),
    "fwd": ("attn_fwd_kernel<128, 32, 1, false>", ("attn_fwd.hip", "sas_device.h", "sas_internal.h")),
}


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gated_block_sparse_sas_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(part):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by the factor a plain copy
    of known size gave).  None when no summary exists or the kernel's sources
    changed after the counters were taken."""
    name, files = KERNELS[part]
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s_train_32k.md" % part)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("record: "):
                rec = json.loads(line[len("record: "):])
    if rec is None or rec.get("kernel") != name or rec.get("src") != source_digest(files):
        return None
    return round(rec["fetch_kib"] * rec["fetch_factor"] * 1024 +
                 rec["write_kib"] * rec["write_factor"] * 1024)


def stored_mfma(part):
    """Matrix-core busy share and shader clock of a training kernel from the
    committed rocprofv3 counter summary (SQ_VALU_MFMA_BUSY_CYCLES over
    GRBM_GUI_ACTIVE); None when absent or the kernel's sources changed."""
    name, files = KERNELS[part]
    path = os.path.join(ROOT, "profiles", "mfma_util_train_32k.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("record: "):
                rec = json.loads(line[len("record: "):])
                if rec.get("part") == part:
                    if rec.get("kernel") != name or rec.get("src") != source_digest(files):
                        return None
                    return {"mfma_busy": rec["busy"], "clock_ghz": rec["clock_ghz"]}
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-sample-t", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (heads and batch "
              "shard with no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_block_sparse_sas_amd import ops, synth
    ops.load()  # raises if libsas.so is missing: there is no fallback
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = synth.WORKLOADS
    wt, wp, wd = W["train_32k"], W["prefill_32k_top16"], W["decode_64k_top8"]
    wq = W["prefill_32k_top25pct"]

    t0 = time.time()
    tr = {n: t.to(dev) for n, t in synth.draw_all(wt).items()}
    pf = {n: t.to(dev) for n, t in synth.draw_all(wp, ("q", "k", "v", "qs", "ks")).items()}
    dc = {n: t.to(dev) for n, t in synth.draw_all(wd, ("q", "k", "v", "qs", "ks")).items()}
    pq = {n: t.to(dev) for n, t in synth.draw_all(wq, ("q", "k", "v", "qs", "ks")).items()}
    wg = synth.PAGED_WORKLOADS["decode_paged_mix"]
    pg = {n: t.to(dev) for n, t in synth.draw_paged(wg).items()}
    wu = W["decode_64k_b16_top32"]
    du = {n: t.to(dev) for n, t in synth.draw_all(wu, ("q", "k", "v", "qs", "ks")).items()}
    wv = W["prefill_32k_b16_top64"]
    pv = {n: t.to(dev) for n, t in synth.draw_all(wv, ("q", "k", "v", "qs", "ks")).items()}
    wh = W["prefill_32k_theta"]
    ph = {n: t.to(dev) for n, t in synth.draw_all(wh, ("q", "k", "v", "qs", "ks")).items()}
    # training with token-level context units: the train_32k tensors with one
    # selector key per token
    w1 = wt.with_(name="train_32k_b1", block=1)
    ks1 = synth.draw_all(w1, ("ks",))["ks"].to(dev)
    torch.cuda.synchronize()
    log("inputs resident in HBM (%.1f s)" % (time.time() - t0))

    sh_t = ops.shape_of(tr["q"], tr["k"], tr["qs"], tr["ks"])
    ws_t = torch.empty(ops.bwd_workspace_bytes(sh_t), dtype=torch.uint8, device=dev)
    sh_p = ops.make_shape(1, wp.hq, wp.hkv, wp.tq, wp.tk, wp.d, wp.ds, 64, wp.hkv)
    ws_p = torch.empty(ops.sparse_workspace_bytes(sh_p, wp.topk), dtype=torch.uint8, device=dev)
    sh_d = ops.make_shape(wd.batch, wd.hq, wd.hkv, wd.tq, wd.tk, wd.d, wd.ds, 64, wd.hkv)
    ws_d = torch.empty(ops.sparse_workspace_bytes(sh_d, wd.topk), dtype=torch.uint8, device=dev)
    sh_q = ops.make_shape(1, wq.hq, wq.hkv, wq.tq, wq.tk, wq.d, wq.ds, 64, wq.hkv)
    ws_q = torch.empty(ops.sparse_workspace_bytes(sh_q, wq.topk), dtype=torch.uint8, device=dev)
    sh_g = ops.make_paged_shape(wg.batch, wg.hq, wg.hkv, wg.d, wg.ds, wg.max_blocks,
                                pg["k_pool"].shape[0])
    ws_g = torch.empty(ops.paged_workspace_bytes(sh_g, wg.topk), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    nnz_h = int(ops.threshold_count(ph["qs"], ph["ks"], wh.theta, wh.tk, ws=ws_h)[-1].item())
    # the step enqueues count, fill and forward with a capacity bound instead
    # of reading each count back; every step's count is checked afterwards
    cap_h = nnz_h + nnz_h // 8
    sh_h = ops.make_shape(1, wh.hq, wh.hkv, wh.tq, wh.tk, wh.d, wh.ds, 64, wh.hkv)
    ws_hs = torch.empty(ops.sparse_csr_workspace_bytes(sh_h, cap_h), dtype=torch.uint8,
                        device=dev)
    nnz_seen = []
    sh_u = ops.make_shape(wu.batch, wu.hq, wu.hkv, wu.tq, wu.tk, wu.d, wu.ds, wu.block, wu.hkv)
    ws_u = torch.empty(ops.sparse_workspace_bytes(sh_u, wu.topk), dtype=torch.uint8, device=dev)
    sh_v = ops.make_shape(wv.batch, wv.hq, wv.hkv, wv.tq, wv.tk, wv.d, wv.ds, wv.block, wv.hkv)
    ws_v = torch.empty(ops.sparse_workspace_bytes(sh_v, wv.topk), dtype=torch.uint8, device=dev)
    sh_1 = ops.shape_of(tr["q"], tr["k"], tr["qs"], ks1, block=1)
    ws_1 = torch.empty(ops.bwd_workspace_bytes(sh_1, False), dtype=torch.uint8, device=dev)

    names = ["start", "gate", "fwd", "bwd_dq", "bwd_dkdv", "bwd_dks", "bwd", "pf_topk",
             "pf_partial", "pf_sparse", "dc_topk", "dc_partial", "dc_sparse", "pq_topk",
             "pq_partial", "pq_sparse", "pg_topk", "pg_decode", "dc_fused", "pg_fused",
             "th_start", "th_count",
             "th_fill0", "th_fill", "th_partial", "th_sparse", "u_topk", "u_sparse",
             "v_topk", "v_sparse", "t1_gate", "t1_fwd", "t1_bwd"]

    def step(ev):
        E = {n: ev[n] for n in names}
        E["start"].record()
        lam = ops.gate_scores(tr["qs"], tr["ks"], wt.tk)
        E["gate"].record()
        o, lse = ops.attn_fwd(tr["q"], tr["k"], tr["v"], tr["qs"], tr["ks"], lam)
        E["fwd"].record()
        ops.attn_bwd(tr["q"], tr["k"], tr["v"], o, tr["dout"], lse, tr["qs"], tr["ks"], lam,
                     ws=ws_t, events=[E["bwd_dq"], E["bwd_dkdv"], E["bwd_dks"]])
        E["bwd"].record()
        idx, bias = ops.topk_blocks(pf["qs"], pf["ks"], wp.topk, wp.tk)
        E["pf_topk"].record()
        ops.sparse_fwd(pf["q"], pf["k"], pf["v"], idx, bias, ws=ws_p, events=[E["pf_partial"]])
        E["pf_sparse"].record()
        idx, bias = ops.topk_blocks(dc["qs"], dc["ks"], wd.topk, wd.tk)
        E["dc_topk"].record()
        ops.sparse_fwd(dc["q"], dc["k"], dc["v"], idx, bias, ws=ws_d, events=[E["dc_partial"]])
        E["dc_sparse"].record()
        # the gate renormalised over the kept blocks (renorm = 1); the other
        # sparse workloads use the training gate (renorm = 0)
        idx, bias = ops.topk_blocks_budget(pq["qs"], pq["ks"], wq.topk, wq.frac, wq.tk, renorm=1)
        E["pq_topk"].record()
        ops.sparse_fwd(pq["q"], pq["k"], pq["v"], idx, bias, ws=ws_q, events=[E["pq_partial"]])
        E["pq_sparse"].record()
        idx, bias = ops.paged_topk(pg["qs"], pg["ks_pool"], pg["block_table"], pg["seq_len"],
                                   wg.topk)
        E["pg_topk"].record()
        ops.paged_decode(pg["q"], pg["k_pool"], pg["v_pool"], pg["block_table"], pg["seq_len"],
                         idx, bias, ws=ws_g)
        E["pg_decode"].record()
        # the same two decodes with selection and attention in one launch
        ops.topk_decode(dc["q"], dc["k"], dc["v"], dc["qs"], dc["ks"], wd.topk)
        E["dc_fused"].record()
        ops.paged_topk_decode(pg["q"], pg["k_pool"], pg["v_pool"], pg["qs"], pg["ks_pool"],
                              pg["block_table"], pg["seq_len"], wg.topk)
        E["pg_fused"].record()
        E["th_start"].record()
        row_ptr = ops.threshold_count(ph["qs"], ph["ks"], wh.theta, wh.tk, ws=ws_h)
        E["th_count"].record()
        E["th_fill0"].record()
        col, bias = ops.threshold_fill(ph["qs"], ph["ks"], wh.theta, wh.tk, row_ptr, cap_h)
        E["th_fill"].record()
        ops.sparse_fwd_csr(ph["q"], ph["k"], ph["v"], row_ptr, col, bias, ws=ws_hs,
                           events=[E["th_partial"]])
        E["th_sparse"].record()
        nnz_seen.append(row_ptr[-1:])
        idx, bias = ops.topk_blocks(du["qs"], du["ks"], wu.topk, wu.tk, block=wu.block)
        E["u_topk"].record()
        ops.sparse_fwd(du["q"], du["k"], du["v"], idx, bias, block=wu.block, ws=ws_u)
        E["u_sparse"].record()
        idx, bias = ops.topk_blocks(pv["qs"], pv["ks"], wv.topk, wv.tk, block=wv.block)
        E["v_topk"].record()
        ops.sparse_fwd(pv["q"], pv["k"], pv["v"], idx, bias, block=wv.block, ws=ws_v)
        E["v_sparse"].record()
        lam = ops.gate_scores(tr["qs"], ks1, wt.tk, block=1)
        E["t1_gate"].record()
        o, lse = ops.attn_fwd(tr["q"], tr["k"], tr["v"], tr["qs"], ks1, lam, block=1)
        E["t1_fwd"].record()
        ops.attn_bwd(tr["q"], tr["k"], tr["v"], o, tr["dout"], lse, tr["qs"], ks1, lam, block=1,
                     with_dz=False, ws=ws_1)
        E["t1_bwd"].record()

    def new_events():
        return {n: torch.cuda.Event(enable_timing=True) for n in names}

    for i in range(args.warmup):
        step(new_events())
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    evs = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    log("timed %d steps in %.3f s" % (args.steps, wall))

    def dur(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs)  # ms

    part = {
        "gate": dur("start", "gate"), "fwd": dur("gate", "fwd"),
        "bwd_dq": dur("fwd", "bwd_dq"), "bwd_dkdv": dur("bwd_dq", "bwd_dkdv"),
        "bwd_dks": dur("bwd_dkdv", "bwd_dks"), "bwd": dur("fwd", "bwd"),
        "prefill_topk": dur("bwd", "pf_topk"), "prefill_partial": dur("pf_topk", "pf_partial"),
        "prefill_sparse": dur("pf_topk", "pf_sparse"), "decode_topk": dur("pf_sparse", "dc_topk"),
        "decode_partial": dur("dc_topk", "dc_partial"),
        "decode_sparse": dur("dc_topk", "dc_sparse"),
        "quarter_topk": dur("dc_sparse", "pq_topk"),
        "quarter_partial": dur("pq_topk", "pq_partial"),
        "quarter_sparse": dur("pq_topk", "pq_sparse"),
        "paged_topk": dur("pq_sparse", "pg_topk"),
        "paged_decode": dur("pg_topk", "pg_decode"),
        "decode_fused": dur("pg_decode", "dc_fused"),
        "paged_fused": dur("dc_fused", "pg_fused"),
        "theta_count": dur("th_start", "th_count"),
        "theta_fill": dur("th_fill0", "th_fill"),
        "theta_partial": dur("th_fill", "th_partial"),
        "theta_sparse": dur("th_fill", "th_sparse"),
        "units_topk": dur("th_sparse", "u_topk"),
        "units_decode": dur("u_topk", "u_sparse"),
        "units_prefill_topk": dur("u_sparse", "v_topk"),
        "units_prefill": dur("v_topk", "v_sparse"),
        "units1_gate": dur("v_sparse", "t1_gate"),
        "units1_fwd": dur("t1_gate", "t1_fwd"),
        "units1_bwd": dur("t1_fwd", "t1_bwd"),
    }
    step_ms = dur("start", "t1_bwd")

    pairs_t = wt.batch * wt.hq * causal_pairs(wt.tq, wt.tk)
    fl_fwd = 4.0 * wt.d * pairs_t
    fl_bwd = 10.0 * wt.d * pairs_t
    t_train = part["gate"] + part["fwd"] + part["bwd"]
    value = (fl_fwd + fl_bwd) / (t_train * 1e-3) / 1e12
    pairs_p = wp.batch * wp.hq * sparse_pairs(wp)
    fl_sp = 4.0 * wp.d * pairs_p
    sp_tflops = fl_sp / (part["prefill_sparse"] * 1e-3) / 1e12
    pairs_q = wq.batch * wq.hq * sparse_pairs(wq)
    fl_q = 4.0 * wq.d * pairs_q
    q_tflops = fl_q / (part["quarter_sparse"] * 1e-3) / 1e12
    dec_blocks = wd.batch * wd.hq * (min(wd.topk, (wd.tk - 1) // 64) + 1)
    dec_bytes = dec_blocks * 2 * 64 * wd.d * 2  # K and V of every attended block, bf16
    dec_gbps = dec_bytes / (part["decode_sparse"] * 1e-3) / 1e9
    lens_g = pg["seq_len"].cpu().tolist()
    pg_blocks = wg.hq * sum(min(wg.topk, (n - 1) // 64) + 1 for n in lens_g)
    pg_bytes = pg_blocks * 2 * 64 * wg.d * 2  # K and V of every attended block, bf16
    pg_gbps = pg_bytes / (part["paged_decode"] * 1e-3) / 1e9
    assert all(int(n.item()) == nnz_h <= cap_h for n in nnz_seen)
    rows_h = wh.batch * wh.hq * wh.tq
    # attended pairs: 64 keys per selected block + the causal part of the current block
    pairs_h = nnz_h * 64 + wh.batch * wh.hq * sum(
        (wh.tk - wh.tq + i) % 64 + 1 for i in range(wh.tq))
    h_tflops = 4.0 * wh.d * pairs_h / (part["theta_sparse"] * 1e-3) / 1e12
    u_bytes = wu.batch * wu.hq * (min(wu.topk, (wu.tk - 1) // wu.block) + 1) * 2 * wu.block * wu.d * 2
    u_gbps = u_bytes / (part["units_decode"] * 1e-3) / 1e9
    t_units1 = part["units1_gate"] + part["units1_fwd"] + part["units1_bwd"]
    units1_tflops = (fl_fwd + fl_bwd) / (t_units1 * 1e-3) / 1e12
    pairs_v = wv.batch * wv.hq * sparse_pairs(wv)
    v_tflops = 4.0 * wv.d * pairs_v / (part["units_prefill"] * 1e-3) / 1e12

    # dominant kernel: the key-stationary backward kernel (dK, dV): S, dP, dV
    # and dK over every attended pair = 8*d flop per pair
    kern = {"bwd_dkdv": (8.0 * wt.d * pairs_t, part["bwd_dkdv"]),
            "fwd": (fl_fwd, part["fwd"]),
            "bwd_dq": (6.0 * wt.d * pairs_t, part["bwd_dq"])}
    dom = max(kern, key=lambda n: kern[n][1])
    kflop, kms = kern[dom]
    achieved = kflop / (kms * 1e-3) / 1e12
    roofline = {
        "kernel": KERNELS[dom][0],
        "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": stored_traffic(dom),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
        "avg_ms": round(kms, 4),
        "per_unit": {"bwd_dkdv": "8*d flop per attended pair (S, dP, dV, dK)",
                     "fwd": "4*d flop per attended pair (S, PV)",
                     "bwd_dq": "6*d flop per attended pair (S, dP, dQ)"}[dom],
        "units_per_launch": pairs_t,
        # the profiled launch's matrix-core busy share and clock (counters)
        "counters": stored_mfma(dom),
    }

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs shaped like the pages' 32k workloads)",
        "config": {"workload": "train_32k", "batch": wt.batch, "hq": wt.hq, "hkv": wt.hkv,
                   "seq_len": wt.tq, "d": wt.d, "block": wt.block, "ds": wt.ds,
                   "also_in_step": ["prefill_32k_top16", "decode_64k_top8",
                                    "prefill_32k_top25pct", "decode_paged_mix",
                                    "prefill_32k_theta", "decode_64k_b16_top32",
                                    "prefill_32k_b16_top64", "train_32k_b1"]},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "train_ms": round(t_train, 3),
        "parts_ms": {k: round(v, 4) for k, v in part.items()},
        "sparse_prefill": {"workload": "prefill_32k_top16", "tflops": round(sp_tflops, 2),
                           "ms": round(part["prefill_sparse"], 3),
                           "topk_ms": round(part["prefill_topk"], 3),
                           "attended_pairs": pairs_p},
        "sparse_prefill_quarter": {"workload": "prefill_32k_top25pct",
                                   "budget": "min(%d, ceil(%.2f c(t)))" % (wq.topk, wq.frac),
                                   "renorm": 1,
                                   "tflops": round(q_tflops, 2),
                                   "ms": round(part["quarter_sparse"], 3),
                                   "topk_ms": round(part["quarter_topk"], 3),
                                   "attended_pairs": pairs_q},
        "decode": {"workload": "decode_64k_top8", "ms": round(part["decode_sparse"], 4),
                   "topk_ms": round(part["decode_topk"], 4), "kv_bytes": dec_bytes,
                   "GBps": round(dec_gbps, 1),
                   "frac_hbm": round(dec_gbps / PEAK_HBM_GBPS, 4),
                   "fused_ms": round(part["decode_fused"], 4),
                   "fused_note": "selection + decode in one launch (sas_topk_decode)"},
        "paged_decode": {"workload": "decode_paged_mix", "sequences": wg.batch,
                         "len_min": min(lens_g), "len_max": max(lens_g),
                         "tokens": sum(lens_g), "ms": round(part["paged_decode"], 4),
                         "topk_ms": round(part["paged_topk"], 4), "kv_bytes": pg_bytes,
                         "GBps": round(pg_gbps, 1),
                         "frac_hbm": round(pg_gbps / PEAK_HBM_GBPS, 4),
                         "fused_ms": round(part["paged_fused"], 4)},
        "sparse_prefill_theta": {"workload": "prefill_32k_theta", "theta": wh.theta,
                                 "nnz": nnz_h, "capacity": cap_h, "host_read": False,
                                 "blocks_per_row": round(nnz_h / rows_h, 2),
                                 "count_ms": round(part["theta_count"], 3),
                                 "fill_ms": round(part["theta_fill"], 3),
                                 "ms": round(part["theta_sparse"], 3),
                                 "tflops": round(h_tflops, 2), "attended_pairs": pairs_h},
        "decode_units16": {"workload": "decode_64k_b16_top32", "block": wu.block,
                           "ms": round(part["units_decode"], 4),
                           "topk_ms": round(part["units_topk"], 4), "kv_bytes": u_bytes,
                           "GBps": round(u_gbps, 1), "frac_hbm": round(u_gbps / PEAK_HBM_GBPS, 4)},
        "prefill_units16": {"workload": "prefill_32k_b16_top64", "block": wv.block,
                            "ms": round(part["units_prefill"], 3),
                            "topk_ms": round(part["units_prefill_topk"], 3),
                            "tflops": round(v_tflops, 2), "attended_pairs": pairs_v},
        "train_units1": {"workload": "train_32k_b1", "block": 1, "ms": round(t_units1, 3),
                         "gate_ms": round(part["units1_gate"], 3),
                         "fwd_ms": round(part["units1_fwd"], 3),
                         "bwd_ms": round(part["units1_bwd"], 3),
                         "tflops": round(units1_tflops, 2),
                         "flop_count": "14*d per attended pair, as train_32k (selector "
                                       "products not counted)"},
        "roofline": roofline,
        "wall_s_timed": round(wall, 3),
    }
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy of %d MiB done" % args.calib_copy_mib)
        del src, dst
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a %d-token sample ..." % args.cpu_sample_t)
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_t)
        log("cpu baseline: %.1f s" % out["cpu_baseline"]["seconds"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
