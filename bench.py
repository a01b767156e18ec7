#!/usr/bin/env python3
"""Benchmark: one dense verify pass per step on one MI355X.

Workload (the dense verify-pass configuration): 64 layers x {qkv 7168x5120,
o 5120x6144, gate+up 34816x5120, down 5120x17408}, every matrix NVFP4
(21,474,836,480 weights, 12,079,595,520 weight bytes), BF16 activations,
N cycled over 2, 4, 8 from one pass to the next, all 256 matrices in one
persistent launch (wq_verify_launch of a prepared plan).  Inputs are
seeded synthetic arrays (fp8_weight_streaming_amd.inputs), resident in HBM
before the timed region.  The weights are streamed in the tiled NVFP4
layout (the same bytes, permuted once at load time by wq_nvfp4_tile,
outside the timed region); the plain row-major layout is timed too and
reported under "plain_layout".

Printed: ONE JSON line with the metric (achieved HBM GB/s over the timed
passes, algorithmic bytes per pass / pass time), the per-N breakdown, a
roofline object for the verify kernel (HIP events on the launch stream),
"single_products": the other four workloads (NVFP4 1024x1024 N=1,
17408x5120 N=1, 5120x17408 N=8, FP8-row 151936x5120 N=8) as single calls,
µs and GB/s per call for N = 1..8 (--no-single skips them), the chained MLP
pass (--no-chain skips it), and the cpu_baseline leg: the CPU oracle's rate
on a bounded sample, then the comparison of sampled GPU outputs of every
row with the oracle (parity fields; the oracle runs nowhere else, and
--no-cpu-baseline leaves them unchecked).

    python bench.py [--gpus 1] [--steps 90] [--warmup 9]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import mmap
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from fp8_weight_streaming_amd import inputs  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) and µs per verify pass, N=1..8 columns"
PEAK_GBPS = 8000.0
N_CYCLE = [2, 4, 8]
NMAX = 8
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "verify_pass_traffic.txt")
# the kernels and the planner that lays out their work (the counters belong to both)
KERNEL_SOURCES = ["fp8_weight_streaming_amd/csrc/wq_kernels.hip", "fp8_weight_streaming_amd/csrc/wq_internal.h",
                  "fp8_weight_streaming_amd/csrc/wq_api.cpp"]


# ---- input generation (before the GPU is touched) ---------------------------

_SHARED = {}


def _layout(wl):
    offs, tot = [], [0, 0, 0]
    for spec in wl.matrices:
        sizes = (spec.M * spec.K // 2, spec.M * spec.K // 16, NMAX * spec.K * 2)
        offs.append(tuple(tot))
        for j in range(3):
            tot[j] += sizes[j]
    return offs, tot


def _gen_worker(i):
    import torch
    torch.set_num_threads(1)
    wl, offs = _SHARED["wl"], _SHARED["offs"]
    spec = wl.matrices[i]
    d = inputs.nvfp4_inputs(spec.M, spec.K, NMAX, wl.seed(i), wl.g, wl.x_scale)
    oc, os_, ox = offs[i]
    np.frombuffer(_SHARED["codes"], np.uint8, d.codes.size, oc)[:] = d.codes.reshape(-1)
    np.frombuffer(_SHARED["scales"], np.uint8, d.scales.size, os_)[:] = d.scales.reshape(-1)
    np.frombuffer(_SHARED["x"], np.uint8, d.x.size * 2, ox)[:] = d.x.reshape(-1).view(np.uint8)
    return i


def generate(wl, workers):
    """Draw every matrix of the pass into shared anonymous memory, with a
    pool of forked workers (workers = 0: in this process, e.g. under a
    profiler that has already initialised the GPU)."""
    offs, tot = _layout(wl)
    _SHARED.update(wl=wl, offs=offs, codes=mmap.mmap(-1, tot[0]), scales=mmap.mmap(-1, tot[1]),
                   x=mmap.mmap(-1, tot[2]))
    if workers <= 0:
        for i in range(len(wl.matrices)):
            _gen_worker(i)
    else:
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            for _ in pool.imap_unordered(_gen_worker, range(len(wl.matrices)), chunksize=1):
                pass
    host = []
    for i, spec in enumerate(wl.matrices):
        oc, os_, ox = offs[i]
        codes = np.frombuffer(_SHARED["codes"], np.uint8, spec.M * spec.K // 2, oc).reshape(spec.M, spec.K // 2)
        scales = np.frombuffer(_SHARED["scales"], np.uint8, spec.M * spec.K // 16, os_).reshape(spec.M, spec.K // 16)
        x = np.frombuffer(_SHARED["x"], np.uint16, NMAX * spec.K, ox).reshape(NMAX, spec.K)
        host.append(inputs.NVFP4Inputs(codes=codes, scales=scales, g=wl.g, x=x))
    return host


# ---- byte accounting -----------------------------------------------------------

def algorithmic_bytes(wl, N):
    """Bytes the method must move for one pass at N columns: 0.5625 B per
    NVFP4 weight (codes + block scales), the BF16 activations (2NK per
    matrix), the FP32 outputs (4NM) and the 4-byte tensor scale."""
    tot = 0
    for s in wl.matrices:
        tot += s.M * s.K // 2 + s.M * s.K // 16 + 2 * N * s.K + 4 * N * s.M + 4
    return tot


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None, None
    kv = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, kv
    try:
        return float(kv["hbm_bytes_per_launch_mean"]), kv
    except (KeyError, ValueError):
        return None, kv


# ---- CPU baseline ----------------------------------------------------------------

def host_cpu():
    """The host's logical CPU count, the CPUs this process may run on, and
    the CPU model name as lscpu reports it (falling back to /proc/cpuinfo)."""
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    if model is None and os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = None
    return {"nproc": os.cpu_count(), "cpus_allowed": allowed, "model": model}


def cpu_baseline(wl, host, budget_s=12.0, max_layers=8, one_thread_stride=16):
    """The oracle, as it is, on the first layers of the same pass.

    All threads: every matrix of layer l at N = 2, 4 and 8, layer after layer
    until `budget_s` seconds have been spent (at most `max_layers` layers);
    the time per N, scaled to the pass's layers, is the oracle's time per
    pass at that N.  One thread: every `one_thread_stride`-th row of layer
    0's four matrices at N = 2, 4 and 8 (the oracle's cost is linear in the
    rows it computes)."""
    import oracle
    t_n = {N: 0.0 for N in N_CYCLE}
    b_n = {N: 0 for N in N_CYCLE}
    t0 = time.perf_counter()
    layers = 0
    while layers < max_layers:
        for j in range(4):
            i = 4 * layers + j
            d = host[i]
            s = wl.matrices[i]
            for N in N_CYCLE:
                ta = time.perf_counter()
                oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N])
                t_n[N] += time.perf_counter() - ta
                b_n[N] += s.M * s.K // 2 + s.M * s.K // 16 + 2 * N * s.K + 4 * N * s.M + 4
        layers += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = sum(t_n.values())
    nbytes = sum(b_n.values())
    threads = oracle.num_threads()
    pass_layers = len(wl.matrices) // 4
    per_n = {str(N): {"us_per_pass": t_n[N] / layers * pass_layers * 1e6, "gbps": b_n[N] / t_n[N] / 1e9}
             for N in N_CYCLE}
    # one thread, on a row sample of layer 0
    oracle.set_num_threads(1)
    try:
        t1, b1 = 0.0, 0
        for j in range(4):
            d, s = host[j], wl.matrices[j]
            rows = np.arange(0, s.M, one_thread_stride)
            for N in N_CYCLE:
                ta = time.perf_counter()
                oracle.gemm_nvfp4(d.codes, d.scales, d.g, d.x[:N], rows=rows)
                t1 += time.perf_counter() - ta
                b1 += rows.size * (s.K // 2 + s.K // 16 + 4 * N) + 2 * N * s.K + 4
        one = {"value": b1 / t1 / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
               "sample": "every %dth row of layer 0's 4 matrices at N=2,4,8: %.4f GB algorithmic in %.1f s"
                         % (one_thread_stride, b1 / 1e9, t1)}
    finally:
        oracle.set_num_threads(threads)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "FP64 oracle (C, OpenMP, %d threads) on all rows of layers 0..%d (%d matrices) at N=2,4,8: "
                      "%.3f GB algorithmic in %.1f s; us_per_pass scales the per-layer time to %d layers"
                      % (threads, layers - 1, 4 * layers, nbytes / 1e9, dt, pass_layers),
            "host": host_cpu(), "per_n": per_n, "one_thread": one,
            "speedup_one_to_all": (nbytes / dt) / (b1 / t1)}


# ---- the cpu_baseline leg's comparisons ------------------------------------------
# The rows below time the GPU and keep host copies of (samples of) its
# outputs; these functions, run only from the cpu_baseline leg, compare them
# with the oracle and fill in the rows' parity fields.

PENDING = []  # (check function, row dict to fill, payload)


def check_sampled_nvfp4(row, p):
    """Sampled NVFP4 products: |y - y_oracle| <= 1e-3 sum|w x| everywhere."""
    import oracle
    worst, ok = 0.0, True
    for codes, scales, g, x, y in p["samples"]:
        yr, ar = oracle.gemm_nvfp4(codes, scales, g, x)
        err = np.abs(y - yr)
        bound = 1e-3 * ar
        ok = ok and not (err > bound).any() and not np.isnan(y).any()
        worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    row["max_err_over_bound"] = worst
    if "ok" in row:
        row["ok"] = bool(ok)
    else:
        row["parity_ok"] = bool(ok)
    return ok


def check_product(row, p):
    """One single product's sampled rows; at the workload's own N the oracle
    call is also timed as the row's CPU figure."""
    import oracle
    d, rows, N, yg = p["d"], p["rows"], p["N"], p["y"]
    t0 = time.perf_counter()
    if p["fmt"] == "nvfp4":
        yr, ar = oracle.gemm_nvfp4(d.codes, d.scales, p["g"], d.x[:N], rows=rows)
    else:
        yr, ar = oracle.gemm_fp8row(d.w, d.row_scale, d.x[:N], rows=rows)
    t_or = time.perf_counter() - t0
    err = np.abs(yg - yr)
    bound = 1e-3 * ar
    row["max_err_over_bound"] = float((err / np.maximum(bound, 1e-300)).max())
    row["parity_ok"] = bool(not (err > bound).any() and np.array_equal(np.isnan(yg), np.isnan(yr)))
    if p["own"]:
        scale_rows = p["M"] / rows.size
        row["oracle_us"] = t_or * scale_rows * 1e6
        row["oracle_gbps"] = p["nbytes"] / (t_or * scale_rows) / 1e9
        row["oracle_cores"] = oracle.num_threads()
    return row["parity_ok"]


def check_accept(row, p):
    """Tokens = the greedy choice over the kernel's own logits, unchanged by
    the drafts; the accepted count = the oracle's rule (N - 3 by design)."""
    from oracle.accept import greedy_accept, greedy_token
    tk, lg, N = p["tokens"], p["logits"], p["N"]
    ok = (all(tk[n] == greedy_token(lg[n]) for n in range(N)) and np.array_equal(tk, p["first_tokens"])
          and p["accepted"] == greedy_accept(lg, p["drafts"])[1] == N - 3)
    row["parity_ok"] = bool(ok)
    return ok


def check_quantizer(row, p):
    """Sampled rows of a quantizer's output, bit for bit."""
    from oracle.quant import quantize_fp8row, quantize_nvfp4
    if p["name"] == "fp8row":
        qr, rr = quantize_fp8row(p["w"])
        ok = np.array_equal(p["q"], qr) and np.array_equal(p["r"].view(np.uint32), rr.view(np.uint32))
    else:
        cr, sr = quantize_nvfp4(p["w"], np.float32(p["g"]))
        ok = np.array_equal(p["codes"], cr) and np.array_equal(p["scales"], sr)
    row["bit_exact"] = bool(ok)
    return ok


def check_chain_layer0(row, p):
    """Layer 0 of the chain at N = 8, each stage from the GPU's own input to
    it: a within a BF16 step of the oracle's normalization; sampled s within
    the GEMM bound carried through silu and the BF16 rounding; sampled rows
    of h within the GEMM bound plus FP32 rounding of the sum."""
    import oracle
    from oracle import chain
    a_bits, s_bits, h0, F = p["a_bits"], p["s_bits"], p["h0"], p["F"]
    a_ref = chain.normalize(h0.astype(np.float64), p["gamma"], p["eps"])
    ok = bool(np.all(np.abs(chain.bf16_value(a_bits) - a_ref) <= 2.0 ** -7 * np.abs(a_ref)))
    g, ag = oracle.gemm_nvfp4(*p["gate"], a_bits)
    u, au = oracle.gemm_nvfp4(*p["up"], a_bits)
    s_ref = chain.bf16_round(chain.silu(g) * u)
    s_gpu = chain.bf16_value(s_bits[:, p["f"]])
    eg, eu = 1e-3 * ag, 1e-3 * au
    bound = 1.1 * np.abs(u) * eg + (np.abs(chain.silu(g)) + 1.1 * eg) * eu + 2.0 ** -7 * np.maximum(
        np.abs(s_ref), np.abs(s_gpu)) + 1e-37
    worst_s = float((np.abs(s_gpu - s_ref) / bound).max())
    m = p["m"]
    y, ay = oracle.gemm_nvfp4(*p["down"], s_bits)
    href = h0[:, m].astype(np.float64) + y
    bound = 1e-3 * ay + 2.0 ** -23 * (np.abs(h0[:, m]) + np.abs(y)) + 1e-37
    worst_h = float((np.abs(p["h1"][:, m].astype(np.float64) - href) / bound).max())
    ok = ok and worst_s <= 1.0 and worst_h <= 1.0
    row["parity_ok"] = bool(ok)
    row["layer0_max_err_over_bound"] = {"s": worst_s, "h": worst_h}
    return ok


def run_oracle_checks():
    ok = True
    for fn, row, payload in PENDING:
        ok = fn(row, payload) and ok
    PENDING.clear()
    return bool(ok)


# ---- the single-product configurations -------------------------------------------

def matrix_bytes(fmt, M, K, N):
    """Algorithmic bytes of one product: weights (NVFP4 0.5625 B, FP8 1 B
    per weight plus 4 B per row scale), BF16 X, FP32 Y, 4 B tensor scale."""
    if fmt == "nvfp4":
        return M * K // 2 + M * K // 16 + 2 * N * K + 4 * N * M + 4
    return M * K + 4 * M + 2 * N * K + 4 * N * M


def single_products(wq, torch, stream, probe_gbps, check_rows=2048):
    """Workloads 0, 1, 2 and 4 as single wq_gemm_* calls: for N = 1..8 on the
    tiled layout and at the workload's own N on the plain layout.  Calls
    run back to back over copies of the weights that together exceed 1 GiB
    (more than the 256 MB last-level cache), each call bracketed by HIP
    events on the launch stream; the median per-call time is reported.
    At the workload's own N the output is checked against the oracle (all
    rows, or check_rows sampled rows when M is larger), and that oracle call
    is timed as the CPU figure of the row; at other N, 64 sampled rows
    (the comparison runs in the cpu_baseline leg)."""
    dev = torch.device("cuda:0")
    GiB = 1 << 30
    out = []
    for ci in (0, 1, 2, 4):
        wl = inputs.workload(ci)
        spec = wl.matrices[0]
        M, K = spec.M, spec.K
        # eight X columns for every workload (column 0 is the workload's own
        # draw: X is drawn last, row-major)
        if wl.fmt == "nvfp4":
            d = inputs.nvfp4_inputs(M, K, NMAX, wl.seed(0), wl.g, wl.x_scale)
        else:
            d = inputs.fp8row_inputs(M, K, NMAX, wl.seed(0))
        x8 = torch.from_numpy(d.x.view(np.int16)).to(dev)
        if wl.fmt == "nvfp4":
            codes, scales = torch.from_numpy(d.codes).to(dev), torch.from_numpy(d.scales).to(dev)
            tb = wq.wq_nvfp4_tiled_bytes(M, K)
            nt = max(2, -(-GiB // tb))
            tiled = torch.empty((nt, tb), dtype=torch.uint8, device=dev)
            wq.wq_nvfp4_tile(codes, scales, tiled[0], stream)
            np_ = max(2, -(-GiB // (codes.numel() + scales.numel())))
            pc = codes.view(1, -1).repeat(np_, 1)
            ps = scales.view(1, -1).repeat(np_, 1)
            fmt_t, fmt_p = wq.WQ_FMT_NVFP4_TILED, wq.WQ_FMT_NVFP4

            def call_t(i, xN, y, ws):
                wq.wq_gemm_nvfp4_tiled(tiled[i % nt], wl.g, xN, y, M, K, ws, stream)

            def call_p(i, xN, y, ws):
                wq.wq_gemm_nvfp4(pc[i % np_], ps[i % np_], wl.g, xN, y, ws, stream, M=M, K=K)
        else:
            w, rs = torch.from_numpy(d.w).to(dev), torch.from_numpy(d.row_scale).to(dev)
            tb = wq.wq_fp8_tiled_bytes(M, K)
            nt = max(2, -(-GiB // tb))
            tiled = torch.empty((nt, tb), dtype=torch.uint8, device=dev)
            wq.wq_fp8_tile(w, tiled[0], stream)
            np_ = max(2, -(-GiB // w.numel()))
            pw = w.view(1, -1).repeat(np_, 1)
            fmt_t, fmt_p = wq.WQ_FMT_FP8ROW_TILED, wq.WQ_FMT_FP8ROW

            def call_t(i, xN, y, ws):
                wq.wq_gemm_fp8row_tiled(tiled[i % nt], rs, xN, y, M, K, ws, stream)

            def call_p(i, xN, y, ws):
                wq.wq_gemm_fp8row(pw[i % np_], rs, xN, y, ws, stream, M=M, K=K)
        for i in range(1, nt):
            tiled[i].copy_(tiled[0])
        torch.cuda.synchronize()
        rng = np.random.default_rng(777 + ci)
        runs = [("tiled", fmt_t, call_t, nt, N) for N in range(1, NMAX + 1)] + [("plain", fmt_p, call_p, np_, wl.N)]
        for layout, fmt, call, copies, N in runs:
            xN = x8[:N]
            y = torch.full((N, M), float("nan"), dtype=torch.float32, device=dev)
            wsb = wq.wq_gemm_workspace_bytes(fmt, M, K, N)
            ws = torch.zeros(wsb, dtype=torch.uint8, device=dev) if wsb else None
            for i in range(3):
                call(i, xN, y, ws)
            reps = max(20, min(copies, 2000))
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            torch.cuda.synchronize()
            for i in range(reps):
                ev[i][0].record(stream)
                call(3 + i, xN, y, ws)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
            nbytes = matrix_bytes(wl.fmt, M, K, N)
            row = {"workload": ci, "name": wl.name, "N": N, "layout": layout, "split": list(wq.wq_gemm_split(fmt, M, K)),
                   "calls": 3 + reps, "us": us, "gbps": nbytes / us / 1e3, "pct_of_8TBps": 100 * nbytes / us / 1e3 / PEAK_GBPS,
                   "pct_of_probe": 100 * nbytes / us / 1e3 / probe_gbps, "copies": copies}
            own = N == wl.N
            rows = np.arange(M) if (own and M <= check_rows) else np.unique(
                np.concatenate([rng.integers(0, M, check_rows if own else 64), [0, M - 1]]))
            yg = y.cpu().numpy()[:, rows].astype(np.float64)
            row["rows_checked"] = int(rows.size)
            row["parity_ok"] = None
            PENDING.append((check_product, row, {"fmt": wl.fmt, "d": d, "g": wl.g, "rows": rows, "N": N, "y": yg,
                                                 "own": own, "nbytes": nbytes, "M": M}))
            out.append(row)
            del y, ws
        if wl.fmt == "fp8row":
            out += head_accept_rows(wq, torch, stream, wl, d, tiled, nt, rs, x8, probe_gbps)
        del tiled
    return out


def head_accept_rows(wq, torch, stream, wl, d, tiled, nt, rs, x8, probe_gbps):
    """Greedy acceptance fused onto the FP8 head (workload 4, N = 8), with
    and without writing the logits, timed like the products; the tokens are
    checked against the greedy choice over the kernel's own logits and the
    accepted count against the oracle's rule (in the cpu_baseline leg)."""
    dev = torch.device("cuda:0")
    spec = wl.matrices[0]
    M, K, N = spec.M, spec.K, NMAX
    fmt = wq.WQ_FMT_FP8ROW_TILED
    ws = torch.zeros(wq.wq_head_accept_workspace_bytes(fmt, M, K, N), dtype=torch.uint8, device=dev)
    tokens = torch.zeros(N, dtype=torch.int32, device=dev)
    acc = torch.zeros(1, dtype=torch.int32, device=dev)
    logits = torch.empty((N, M), dtype=torch.float32, device=dev)
    drafts = torch.zeros(N - 1, dtype=torch.int32, device=dev)
    wq.wq_head_accept(fmt, tiled[0], rs, 1.0, x8, M, K, drafts, tokens, acc, logits=logits, workspace=ws,
                      stream=stream)
    torch.cuda.synchronize()
    t0 = tokens.cpu().numpy()
    dr = list(t0[:N - 1])
    dr[N - 3] = (dr[N - 3] + 1) % M  # drafts 1..N-3 accepted, draft N-2 rejected
    drafts.copy_(torch.tensor(dr, dtype=torch.int32))
    rows = []
    for with_logits in (False, True):
        lg = logits if with_logits else None
        for i in range(3):
            wq.wq_head_accept(fmt, tiled[i % nt], rs, 1.0, x8, M, K, drafts, tokens, acc, logits=lg, workspace=ws,
                              stream=stream)
        reps = 20
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            ev[i][0].record(stream)
            wq.wq_head_accept(fmt, tiled[i % nt], rs, 1.0, x8, M, K, drafts, tokens, acc, logits=lg, workspace=ws,
                              stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        nbytes = matrix_bytes("fp8row", M, K, N) - (0 if with_logits else 4 * N * M)
        tk, a = tokens.cpu().numpy(), int(acc.cpu().numpy()[0])
        lgn = logits.cpu().numpy()
        row = {"workload": 4, "name": "greedy acceptance fused on the fp8-row head 151936x5120",
               "N": N, "layout": "accept+logits" if with_logits else "accept", "logits_written": with_logits,
               "calls": 3 + reps + (0 if with_logits else 1), "us": us,
               "gbps": nbytes / us / 1e3, "pct_of_8TBps": 100 * nbytes / us / 1e3 / PEAK_GBPS,
               "pct_of_probe": 100 * nbytes / us / 1e3 / probe_gbps, "accepted": a, "parity_ok": None,
               "max_err_over_bound": 0.0, "rows_checked": 0}
        PENDING.append((check_accept, row, {"tokens": tk, "first_tokens": t0, "accepted": a, "logits": lgn,
                                            "drafts": dr, "N": N}))
        rows.append(row)
    return rows


def quantizer_rows(wq, torch, stream, probe_gbps, check_rows=64):
    """The load-time quantizers on BF16 weights of the FP8 head's shape
    (151936x5120 -> row-scaled FP8) and of the up-projection's shape
    (17408x5120 -> NVFP4), HIP-event medians over 10 calls; sampled rows are
    checked bit for bit against the oracle's quantizers (in the cpu_baseline
    leg)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    rows = []
    for name, M, K in (("fp8row", 151936, 5120), ("nvfp4", 17408, 5120)):
        w = (torch.randn((M, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
        if name == "fp8row":
            q = torch.empty((M, K), dtype=torch.uint8, device=dev)
            r = torch.empty(M, dtype=torch.float32, device=dev)
            call = lambda: wq.wq_quantize_fp8row(w, q, r, stream)  # noqa: E731
            nbytes = 2 * M * K + M * K + 4 * M
            g = None
        else:
            g = float(np.float32(float(w.view(torch.bfloat16).abs().max()) / (6 * 448)))
            c = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            sc = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
            call = lambda: wq.wq_quantize_nvfp4(w, g, c, sc, stream)  # noqa: E731
            nbytes = 2 * M * K + M * K // 2 + M * K // 16
        for _ in range(2):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        sel = np.unique(np.random.default_rng(7).integers(0, M, check_rows))
        idx = torch.from_numpy(sel).to(dev)
        wh = w[idx].cpu().numpy().view(np.uint16)
        if name == "fp8row":
            got = {"q": q[idx].cpu().numpy(), "r": r.cpu().numpy()[sel]}
        else:
            got = {"codes": c[idx].cpu().numpy(), "scales": sc[idx].cpu().numpy()}
        row = {"quantizer": name, "M": M, "K": K, "us": us, "gbps": nbytes / us / 1e3,
               "pct_of_8TBps": 100 * nbytes / us / 1e3 / PEAK_GBPS, "rows_checked": int(sel.size),
               "bit_exact": None}
        PENDING.append((check_quantizer, row, {"name": name, "w": wh, "g": g, **got}))
        rows.append(row)
        del w
    return rows


def draft_step_row(wq, torch, stream, wl, host, mats_dev, probe_gbps, check_rows=32):
    """An N = 1 draft step on NVFP4 weights: one dense layer (layer 0 of the
    pass, tiled) and an NVFP4 output head 151936x5120, re-encoded on the GPU
    from BF16 by wq_quantize_nvfp4 and tiled, in one verify launch (the
    crit README's case study drafts from NVFP4 copies of the draft layer
    and head).  Sampled rows are checked against the oracle (in the
    cpu_baseline leg)."""
    dev = torch.device("cuda:0")
    M, K = 151936, 5120
    gen = torch.Generator(device=dev)
    gen.manual_seed(4343)
    wb = (torch.randn((M, K), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    g = float(np.float32(float(wb.abs().max()) / (6 * 448)))
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    wq.wq_quantize_nvfp4(wb.view(torch.int16), g, codes, scales, stream)
    del wb
    head_t = torch.empty(wq.wq_nvfp4_tiled_bytes(M, K), dtype=torch.uint8, device=dev)
    wq.wq_nvfp4_tile(codes, scales, head_t, stream)
    xh = torch.from_numpy(inputs.to_bf16(np.random.default_rng(11).standard_normal((1, K)).astype(np.float32))
                          .view(np.int16)).to(dev)
    yh = torch.zeros((1, M), dtype=torch.float32, device=dev)
    mats = [wq.Matrix(wq.WQ_FMT_NVFP4_TILED, s.M, s.K, t, None, x[:1], y[:1], wl.g)
            for s, (c, sc, x, y, t) in zip(wl.matrices[:4], mats_dev[:4])]
    mats.append(wq.Matrix(wq.WQ_FMT_NVFP4_TILED, M, K, head_t, None, xh, yh, g))
    ws = torch.zeros(wq.wq_verify_workspace_bytes(mats, 1), dtype=torch.uint8, device=dev)
    plan = wq.wq_verify_prepare(mats, 1, ws, stream)
    for _ in range(3):
        wq.wq_verify_launch(plan, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in ev:
        a.record(stream)
        wq.wq_verify_launch(plan, stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
    nbytes = sum(matrix_bytes("nvfp4", m.M, m.K, 1) for m in mats)
    rng = np.random.default_rng(99)
    samples = []
    for i, m in enumerate(mats):
        rows = np.unique(np.concatenate([rng.integers(0, m.M, check_rows), [0, m.M - 1]]))
        yg = m.y.cpu().numpy()[:, rows].astype(np.float64)
        if i < 4:
            d = host[i]
            samples.append((d.codes[rows], d.scales[rows], d.g, d.x[:1], yg))
        else:
            idx = torch.from_numpy(rows).to(dev)
            samples.append((codes[idx].cpu().numpy(), scales[idx].cpu().numpy(), g, xh.cpu().numpy().view(np.uint16),
                            yg))
    row = {"name": "N=1 draft step: one dense layer + NVFP4 head 151936x5120 (GPU-quantized), one launch",
           "matrices": len(mats), "us": us, "algorithmic_bytes": nbytes, "gbps": nbytes / us / 1e3,
           "pct_of_8TBps": 100 * nbytes / us / 1e3 / PEAK_GBPS, "pct_of_probe": 100 * nbytes / us / 1e3 / probe_gbps,
           "parity_ok": None, "max_err_over_bound": None}
    PENDING.append((check_sampled_nvfp4, row, {"samples": samples}))
    return row


def device_n_rows(wq, torch, stream, wl, mats_dev, bytes_n, reps=10, warm=3):
    """The pass launched with its column count in device memory
    (wq_verify_launch_n on one plan prepared for N = 8), timed as the main
    loop is: N cycled 2, 4, 8 launch after launch (the count written to
    device memory before each, outside the events), `warm` untimed cycles
    first, then `reps` timed cycles; the mean per N."""
    dev = torch.device("cuda:0")
    mats = [wq.Matrix(wq.WQ_FMT_NVFP4_TILED, s.M, s.K, t, None, x, y, wl.g)
            for s, (c, sc, x, y, t) in zip(wl.matrices, mats_dev)]
    ws = torch.zeros(wq.wq_verify_workspace_bytes(mats, 8), dtype=torch.uint8, device=dev)
    plan = wq.wq_verify_prepare(mats, 8, ws, stream)
    n_dev = torch.zeros(1, dtype=torch.int32, device=dev)
    times = {N: [] for N in N_CYCLE}
    for cycle in range(warm + reps):
        for N in N_CYCLE:
            n_dev.fill_(N)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            wq.wq_verify_launch_n(plan, n_dev, stream)
            b.record(stream)
            if cycle >= warm:
                times[N].append((a, b))
    torch.cuda.synchronize()
    out = {}
    for N in N_CYCLE:
        us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in times[N]]))
        out[str(N)] = {"us_per_pass_mean": us, "gbps": bytes_n[N] / us / 1e3,
                       "pct_of_8TBps": 100 * bytes_n[N] / us / 1e3 / PEAK_GBPS}
    return out


def valu_rows(wq, torch, stream, wl, host, mats_dev, plans, bytes_n, reps=5, check_rows=16):
    """The MFMA/VALU comparison: the same prepared plans launched with the
    NVFP4 steps on the matrix cores (wq_verify_launch) and on the vector
    ALUs (wq_verify_launch_valu), alternating, HIP events per launch: the
    dense pass at N = 2, 4, 8, and the 17408x5120 up-projection as a
    one-matrix pass at N = 1, 2, 8.  The VALU outputs are checked against
    the oracle on sampled rows (in the cpu_baseline leg)."""
    dev = torch.device("cuda:0")
    out = {"dense_pass": {}, "up_proj_17408x5120": {}}

    def ab(plan, nbytes):
        for _ in range(2):
            wq.wq_verify_launch(plan, stream)
            wq.wq_verify_launch_valu(plan, stream)
        ev = {"mfma": [], "valu": []}
        for _ in range(reps):
            for kind, fn in (("mfma", wq.wq_verify_launch), ("valu", wq.wq_verify_launch_valu)):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(plan, stream)
                b.record(stream)
                ev[kind].append((a, b))
        torch.cuda.synchronize()
        r = {}
        for kind in ("mfma", "valu"):
            us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in ev[kind]]))
            r[kind + "_us"] = us
            r[kind + "_pct_of_8TBps"] = 100 * nbytes / us / 1e3 / PEAK_GBPS
        r["valu_over_mfma"] = r["valu_us"] / r["mfma_us"]
        return r

    rng = np.random.default_rng(4545)
    samples = []
    for N in N_CYCLE:
        out["dense_pass"][str(N)] = ab(plans[N], bytes_n[N])
        # the last launch was the VALU one: sample its outputs of layer 0
        for i in range(4):
            spec, d = wl.matrices[i], host[i]
            rows = np.unique(np.concatenate([rng.integers(0, spec.M, check_rows), [0, spec.M - 1]]))
            y = mats_dev[i][3][:N].cpu().numpy()[:, rows].astype(np.float64)
            samples.append((d.codes[rows], d.scales[rows], d.g, d.x[:N], y))
    w1 = inputs.workload(1)
    M, K = w1.matrices[0].M, w1.matrices[0].K
    d = inputs.nvfp4_inputs(M, K, NMAX, w1.seed(0), w1.g, w1.x_scale)
    t = torch.empty(wq.wq_nvfp4_tiled_bytes(M, K), dtype=torch.uint8, device=dev)
    wq.wq_nvfp4_tile(torch.from_numpy(d.codes).to(dev), torch.from_numpy(d.scales).to(dev), t, stream)
    x = torch.from_numpy(d.x.view(np.int16)).to(dev)
    for N in (1, 2, 8):
        y = torch.full((N, M), float("nan"), dtype=torch.float32, device=dev)
        mats = [wq.Matrix(wq.WQ_FMT_NVFP4_TILED, M, K, t, None, x[:N], y, w1.g)]
        ws = torch.zeros(wq.wq_verify_workspace_bytes(mats, N), dtype=torch.uint8, device=dev)
        plan = wq.wq_verify_prepare(mats, N, ws, stream)
        out["up_proj_17408x5120"][str(N)] = ab(plan, matrix_bytes("nvfp4", M, K, N))
        rows = np.unique(np.concatenate([rng.integers(0, M, 4 * check_rows), [0, M - 1]]))
        samples.append((d.codes[rows], d.scales[rows], w1.g, d.x[:N], y.cpu().numpy()[:, rows].astype(np.float64)))
    out["parity_ok"] = None
    out["max_err_over_bound"] = None
    out["note"] = ("the verify-pass kernel with its NVFP4 step on the vector ALUs (stream_kernel<N, 8>) against the "
                   "matrix cores (stream_kernel<N, 4>), same plans; valu_over_mfma > 1 means the matrix cores win")
    PENDING.append((check_sampled_nvfp4, out, {"samples": samples}))
    return out


def chain_bytes(D, F, N, layers):
    """Bytes a chained MLP pass must move: per layer the NVFP4 gate, up and
    down weights (0.5625 B each), gamma (2D), the residual read and written
    (4ND each), the normalized input written (2ND), the gated product
    written and read (2NF each) and three tensor scales."""
    per = 3 * D * F // 2 + 3 * D * F // 16 + 2 * D + 8 * N * D + 2 * N * D + 4 * N * F + 12
    return per * layers


def chain_rows(wq, torch, stream, wl, host, mats_dev, probe_gbps, check_rows=48, reps=5, single_launch=True):
    """The verify pass as chained MLP layers (wq_mlp_chain_*): each of the
    pass's layers applies RMSNorm, gate/up (rows 0..F-1 and F..2F-1 of its
    gate_up matrix), SwiGLU and down to the residual stream of the N verify
    columns, three kernels per layer, eager and replayed as one HIP graph.
    Layer 0 is checked against the oracle on sampled outputs (in the
    cpu_baseline leg)."""
    dev = torch.device("cuda:0")
    layers = len(wl.matrices) // 4
    D, F = wl.matrices[3].M, wl.matrices[3].K
    rng = np.random.default_rng(2024)
    descs, keep = [], []
    for l in range(layers):
        c, sc = mats_dev[4 * l + 2][0], mats_dev[4 * l + 2][1]
        gu = torch.empty(wq.wq_nvfp4_tiled_bytes(2 * F, D), dtype=torch.uint8, device=dev)
        wq.wq_nvfp4_tile_glu(c[:F], sc[:F], c[F:], sc[F:], gu, stream)
        gamma = torch.from_numpy(inputs.to_bf16((1 + 0.2 * rng.standard_normal(D)).astype(np.float32))
                                 .view(np.int16)).to(dev)
        keep.append((gu, gamma))
        descs.append(wq.MlpLayer(gu, mats_dev[4 * l + 3][4], gamma, wl.g, wl.g, wl.g))
    torch.cuda.synchronize()
    eps = 1e-6
    h0_host = inputs.residual_inputs(NMAX, D, seed=2025)
    rows = {}
    for N in (1, 2, 4, 8):
        h0 = torch.from_numpy(h0_host[:N].copy()).to(dev)
        h = h0.clone()
        a = torch.zeros((N, D), dtype=torch.int16, device=dev)
        sb = torch.zeros((N, F), dtype=torch.int16, device=dev)
        ws = torch.empty(wq.wq_mlp_chain_workspace_bytes(layers, D, F, N), dtype=torch.uint8, device=dev)
        plan = wq.wq_mlp_chain_prepare(descs, D, F, N, eps, h, a, sb, ws, stream)
        for _ in range(2):
            wq.wq_mlp_chain_launch(plan, stream)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            h.copy_(h0)
            e0.record(stream)
            wq.wq_mlp_chain_launch(plan, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        eager_us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(graph, stream=side):
            wq.wq_mlp_chain_launch(plan, side)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e0, e1 in ev:
            h.copy_(h0)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        single_us = None
        if single_launch and plan.grid_chain > 0:
            wq.wq_mlp_chain_launch_persistent(plan, stream)
            for e0, e1 in ev:
                h.copy_(h0)
                e0.record(stream)
                wq.wq_mlp_chain_launch_persistent(plan, stream)
                e1.record(stream)
            torch.cuda.synchronize()
            single_us = float(np.median([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]))
        nb = chain_bytes(D, F, N, layers)
        kc, nc = wq.wq_mlp_chain_split(D, F)
        rows[str(N)] = {"eager_us": eager_us, "graph_us": graph_us, "us_per_layer_graph": graph_us / layers,
                        "algorithmic_bytes": nb, "gbps_graph": nb / graph_us / 1e3,
                        "pct_of_8TBps_graph": 100 * nb / graph_us / 1e3 / PEAK_GBPS,
                        "pct_of_8TBps_eager": 100 * nb / eager_us / 1e3 / PEAK_GBPS,
                        "single_launch_us": single_us,
                        "pct_of_8TBps_single_launch": (100 * nb / single_us / 1e3 / PEAK_GBPS) if single_us else None,
                        "launches": 3 * layers + 1, "down_k_chunks": nc}
        # the graph and its capture stream are released (and the device idle)
        # before the next N's buffers are made
        torch.cuda.synchronize()
        del graph, side, ws, plan

    # layer 0 at N = 8 against the oracle (sampled rows of s and h)
    N = 8
    h0 = torch.from_numpy(h0_host.copy()).to(dev)
    h = h0.clone()
    a = torch.zeros((N, D), dtype=torch.int16, device=dev)
    sb = torch.zeros((N, F), dtype=torch.int16, device=dev)
    ws = torch.empty(wq.wq_mlp_chain_workspace_bytes(1, D, F, N), dtype=torch.uint8, device=dev)
    plan = wq.wq_mlp_chain_prepare(descs[:1], D, F, N, eps, h, a, sb, ws, stream)
    wq.wq_mlp_chain_launch(plan, stream)
    torch.cuda.synchronize()
    gu, dn = host[2], host[3]
    f = np.unique(np.concatenate([rng.integers(0, F, check_rows), [0, F - 1]]))
    m = np.unique(np.concatenate([rng.integers(0, D, check_rows), [0, D - 1]]))
    s_bits = sb.cpu().numpy().view(np.uint16)
    payload = {"a_bits": a.cpu().numpy().view(np.uint16), "s_bits": s_bits, "h1": h.cpu().numpy(), "h0": h0_host,
               "gamma": keep[0][1].cpu().numpy().view(np.uint16), "eps": eps, "F": F, "f": f, "m": m,
               "gate": (gu.codes[f], gu.scales[f], gu.g), "up": (gu.codes[F + f], gu.scales[F + f], gu.g),
               "down": (dn.codes[m], dn.scales[m], dn.g)}
    row = {"name": "chained MLP verify pass: %d layers x (RMSNorm, gate+up %dx%d, SwiGLU, down %dx%d, residual)"
                   % (layers, 2 * F, D, D, F),
           "per_n": rows, "parity_ok": None, "layer0_max_err_over_bound": None, "probe_read_gbps": probe_gbps}
    PENDING.append((check_chain_layer0, row, payload))
    return row


# ---- rocprofv3 summaries (profiles/) ----------------------------------------------
# `bench.py --summarize-rocprof KIND --rocprof-dir DIR [--rocprof-dir DIR2] [--bench-log LOG] --out FILE`
# turns the CSV output of a profiled bench.py run into the text committed
# under profiles/.  The profiled commands are written into each summary.

PROF_CMD = {
    "dense": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/kt -o kt -- python3 bench.py "
             "--steps 30 --warmup 3 --no-cpu-baseline --no-single --no-chain --check-rows 2 --workers 0",
    "single": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/kts -o kts -- python3 bench.py "
              "--only-single --no-cpu-baseline",
    "chain": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktc -o ktc -- python3 bench.py "
             "--steps 3 --warmup 1 --no-cpu-baseline --no-single --no-chain-single --no-valu --check-rows 1 --workers 0",
    "traffic_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o fetch -- python3 "
                     "bench.py --steps 6 --warmup 0 --no-cpu-baseline --no-single --no-chain --no-valu --check-rows 1 "
                     "--workers 0",
    "traffic_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o write -- python3 "
                     "bench.py --steps 6 --warmup 0 --no-cpu-baseline --no-single --no-chain --no-valu --check-rows 1 "
                     "--workers 0",
    "single_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmcs_fetch -o fetch -- python3 "
                    "bench.py --only-single --no-cpu-baseline",
    "single_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmcs_write -o write -- python3 "
                    "bench.py --only-single --no-cpu-baseline",
}


def _kernel_name(raw):
    import re
    n = re.sub(r"^void ", "", raw)
    n = re.sub(r"\(anonymous namespace\)::", "", n)
    n = re.sub(r"\((?:[^()]|\([^()]*\))*\)$", "", n).strip()
    return n


def _rocprof_csv(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no %s files under %s" % (suffix, d))
    return rows


def _trace(d):
    """Kernel dispatches of a --kernel-trace run: (start ns, end ns, name), in start order."""
    out = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _kernel_name(r["Kernel_Name"]))
           for r in _rocprof_csv(d, "kernel_trace.csv")]
    return sorted(out)


def _counters(d):
    """Per-dispatch counter values of a --pmc run, in dispatch order: [(name, value)]."""
    rows = _rocprof_csv(d, "counter_collection.csv")
    key = "Dispatch_Id" if "Dispatch_Id" in rows[0] else None
    rows.sort(key=lambda r: int(r[key]) if key else 0)
    return [(_kernel_name(r["Kernel_Name"]), float(r["Counter_Value"])) for r in rows]


def _stats(v):
    import statistics
    return len(v), statistics.mean(v), statistics.median(v), min(v), max(v)


def _bench_json(path):
    with open(path) as f:
        lines = [l for l in f if l.startswith("{")]
    if not lines:
        raise SystemExit("no JSON line in %s" % path)
    return json.loads(lines[-1])


def _summary_cmd(kind, args):
    extra = "".join(" --rocprof-dir %s" % d for d in args.rocprof_dir)
    if args.bench_log:
        extra += " --bench-log %s" % args.bench_log
    return "python3 bench.py --summarize-rocprof %s%s --out %s" % (kind, extra, args.out or "-")


def summarize_dense(args):
    """Kernel trace of the dense pass: the timed region's launches per N
    (the launches longer than 1 ms after the warm-up ones), and every
    dispatch of the run."""
    rows = _trace(args.rocprof_dir[0])
    bl = _bench_json(args.bench_log)
    dense = [(s, e, n) for s, e, n in rows if n.startswith("wq::stream_kernel<") and n.endswith(", 4>")
             and (e - s) > 1e6]
    steps, warm = bl["steps"], bl["warmup"]
    timed = dense[warm:warm + steps]
    L = ["# Kernel trace of the dense verify pass (64 layers, NVFP4, N cycled 2/4/8), MI355X", "#",
         "# commands (from the repository root, after `export TMPDIR=/tmp`):",
         "#   " + PROF_CMD["dense"] + " > gpurun_out/prof_kt.log",
         "#   " + _summary_cmd("dense", args), "#",
         "# stream_kernel<N, 4> is the tiled verify pass (the timed path of bench.py; one launch per pass, the",
         "# 64 down projections computed in LDS blocks, no reduction launch); stream_kernel<N, 0> the plain",
         "# row-major pass (reported as plain_layout) with its split-K reduce_kernel; stream_kernel_dyn the pass",
         "# with N read on the device (per_n_device_count); stream_kernel<N, 8> the same plans with the NVFP4",
         "# steps on the vector ALUs (mfma_vs_valu); probe_read_kernel<false> / <true> the read probe and the",
         "# read-with-writes probe.  Durations in microseconds.", "",
         "timed region of bench.py (the %d steps between its two synchronizations, %d per N):" % (steps, steps // 3),
         "%-36s %7s %12s %12s %12s %12s %9s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us",
                                               "%8TB_avg")]
    wl = inputs.workload(3)
    for N in N_CYCLE:
        v = [(e - s) / 1e3 for s, e, n in timed if n == "wq::stream_kernel<%d, 4>" % N]
        st = _stats(v)
        L.append("%-36s %7d %12.1f %12.1f %12.1f %12.1f %9.1f" % (("wq::stream_kernel<%d, 4>" % N,) + st + (
            100 * algorithmic_bytes(wl, N) / (st[1] * 1e3) / PEAK_GBPS,)))
    v = [(e - s) / 1e3 for s, e, n in timed]
    tot = sum(algorithmic_bytes(wl, int(n.split("<")[1].split(",")[0])) for s, e, n in timed)
    L.append("%-36s %7d %12.1f %12.1f %12.1f %12.1f %9.1f" % (("all timed launches",) + _stats(v) + (
        100 * tot / (sum(v) * 1e3) / PEAK_GBPS,)))
    # the MFMA/VALU comparison rows (mfma_vs_valu): the same plans with the
    # NVFP4 steps on the vector ALUs (stream_kernel<N, 8>) and on the matrix
    # cores (stream_kernel<N, 4>); passes longer than 1 ms are the dense
    # pass, shorter ones the 17408x5120 one-matrix pass
    if any(n.endswith(", 8>") for s_, e_, n in rows):
        import statistics
        L += ["", "matrix cores against vector ALUs (the mfma_vs_valu rows; median kernel durations, us):",
              "%-28s %4s %12s %12s %10s" % ("pass", "N", "mfma_us", "valu_us", "valu/mfma")]
        for label, big in (("dense 64-layer pass", True), ("17408x5120, one matrix", False)):
            for N in range(1, 9):
                mf = [(e - s_) / 1e3 for s_, e, n in rows if n == "wq::stream_kernel<%d, 4>" % N and ((e - s_) > 1e6) == big]
                va = [(e - s_) / 1e3 for s_, e, n in rows if n == "wq::stream_kernel<%d, 8>" % N and ((e - s_) > 1e6) == big]
                if mf and va:
                    m, v = statistics.median(mf), statistics.median(va)
                    L.append("%-28s %4d %12.1f %12.1f %10.2f" % (label, N, m, v, v / m))
    L += ["", "bench.py's own figures for the same run (HIP events on the launch stream):",
          "  roofline.avg_launch_us = %.1f; per_n us_per_pass_mean = %s" % (
              bl["roofline"]["avg_launch_us"],
              ", ".join("N=%s %.1f" % (k, x["us_per_pass_mean"]) for k, x in bl["per_n"].items())), "",
          "every dispatch of the run:",
          "%-36s %7s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us")]
    keep, order = {}, []
    for s, e, n in rows:
        if not n.startswith("wq::"):
            continue
        if n not in keep:
            order.append(n)
        keep.setdefault(n, []).append((e - s) / 1e3)
    for n in order:
        L.append("%-36s %7d %12.1f %12.1f %12.1f %12.1f" % ((n[:36],) + _stats(keep[n])))
    return "\n".join(L) + "\n"


def _is_main_single(n):
    """The first kernel of a single-product call: the stream kernel, or the
    split-tile kernel of the tiled products with few tiles per CU."""
    return n.startswith("wq::stream_kernel<") or n.startswith("wq::split_kernel<")


def _single_groups(rows, bl):
    """Assign the single products' dispatches to bench rows: each row made
    `calls` calls, back to back, in the order of the JSON; a call is one
    stream kernel or split kernel, then (chunked products) a reduce_kernel or
    (acceptance) an accept_kernel."""
    main = []
    for s, e, n in rows:
        if _is_main_single(n):
            main.append([n, (e - s) / 1e3, 0.0])
        elif n in ("wq::reduce_kernel", "wq::accept_kernel") and main:
            main[-1][2] += (e - s) / 1e3
    out, i = [], 0
    for r in bl["single_products"]:
        grp = main[i:i + r["calls"]]
        i += r["calls"]
        names = {g[0] for g in grp}
        if len(grp) != r["calls"] or len(names) != 1:
            raise SystemExit("dispatches do not match the bench rows at %s N=%d %s" % (r["name"], r["N"], r["layout"]))
        out.append((r, names.pop(), [g[1] for g in grp], [g[2] for g in grp]))
    if i != len(main):
        raise SystemExit("%d stream- or split-kernel dispatches left over" % (len(main) - i))
    return out


def _row_bytes(r):
    wl = inputs.workload(r["workload"])
    M, K = wl.matrices[0].M, wl.matrices[0].K
    nb = matrix_bytes(wl.fmt, M, K, r["N"])
    if r["layout"] == "accept":
        nb -= 4 * r["N"] * M
    return nb


def summarize_single(args):
    """Kernel trace of the single products (--only-single run)."""
    import statistics
    rows = _trace(args.rocprof_dir[0])
    bl = _bench_json(args.bench_log)
    L = ["# Kernel trace of the single products (workloads 0, 1, 2, 4), MI355X", "#",
         "# commands (from the repository root, after `export TMPDIR=/tmp`):",
         "#   " + PROF_CMD["single"] + " > gpurun_out/prof_kts.log",
         "#   " + _summary_cmd("single", args), "#",
         "# Each row: one (workload, layout, N) run of back-to-back calls over rotated weight copies (> 1 GiB);",
         "# layout accept: greedy acceptance fused on the tiled FP8 head (wq_head_accept), without / with logits;",
         "# kernel: split_kernel<N, fp8> for tiled products with fewer than 8 row tiles per CU (no second kernel),",
         "# stream_kernel<N, mode> otherwise; us = median duration of that kernel plus median second kernel",
         "# (reduce or accept) duration;",
         "# GB/s = algorithmic bytes / us; events_us = bench.py's HIP-event median per call (launch included).", "",
         "%-44s %-14s %2s %-27s %6s %9s %8s %9s %8s %6s" % ("workload", "layout", "N", "kernel", "calls", "kernel_us",
                                                         "2nd_us", "events_us", "GB/s", "%8TB")]
    for r, name, d, d2 in _single_groups(rows, bl):
        sd, s2 = statistics.median(d), statistics.median(d2)
        us, nb = sd + s2, _row_bytes(r)
        L.append("%-44s %-14s %2d %-27s %6d %9.2f %8.2f %9.2f %8.0f %6.1f" % (
            r["name"][:44], r["layout"], r["N"], name[:27], len(d), sd, s2, r["us"], nb / us / 1e3,
            100 * nb / us / 1e3 / PEAK_GBPS))
    return "\n".join(L) + "\n"


def _copy_scale(c):
    v = [x for n, x in c if n == "wq::probe_copy_kernel"]
    if not v:
        raise SystemExit("no probe_copy_kernel dispatch in the counter run")
    return (1 << 30) / (v[0] * 1024)


def summarize_traffic(args):
    """FETCH_SIZE and WRITE_SIZE of the dense pass's kernels, scaled by the
    same counters on a 1 GiB copy."""
    import statistics
    fe, wr = _counters(args.rocprof_dir[0]), _counters(args.rocprof_dir[1])
    fs, ws = _copy_scale(fe), _copy_scale(wr)
    wl = inputs.workload(3)
    by = lambda c, k: [x for n, x in c if n == k]  # noqa: E731
    L = ["# HBM traffic of the tiled-NVFP4 verify pass kernel, from rocprofv3 counters on MI355X", "#",
         "# commands (one counter per run, from the repository root, after `export TMPDIR=/tmp`):",
         "#   " + PROF_CMD["traffic_fetch"], "#   " + PROF_CMD["traffic_write"], "#   " + _summary_cmd("traffic", args),
         "#", "# Scale: the same counters on wq_probe_copy of exactly 1 GiB (reads 1 GiB, writes 1 GiB):",
         "#   FETCH_SIZE read %.1f KiB -> factor %.4f;  WRITE_SIZE read %.1f KiB -> factor %.4f" % (
             (1 << 30) / fs / 1024, fs, (1 << 30) / ws / 1024, ws),
         "# Per-dispatch values below are KiB as counted (mean over the run's dispatches), then bytes after scaling.",
         ""]
    tot = []
    for N in N_CYCLE:
        k = "wq::stream_kernel<%d, 4>" % N
        f, w = statistics.mean(by(fe, k)), statistics.mean(by(wr, k))
        b = f * 1024 * fs + w * 1024 * ws
        a = algorithmic_bytes(wl, N)
        tot.append(b)
        L.append("N=%d: FETCH_SIZE %.0f KiB (x%.3f) + WRITE_SIZE %.0f KiB (x%.3f) = %.0f bytes; algorithmic %d bytes; "
                 "ratio %.4f" % (N, f, fs, w, ws, b, a, b / a))
        kp = "wq::stream_kernel<%d, 0>" % N
        if by(fe, kp) and by(wr, kp):
            bp = statistics.mean(by(fe, kp)) * 1024 * fs + statistics.mean(by(wr, kp)) * 1024 * ws
            L.append("     plain layout stream_kernel<%d, 0>: %.0f bytes (ratio %.4f; its reduce_kernel launches "
                     "are extra)" % (N, bp, bp / a))
    L += ["", "kernel_source_sha256_16 = %s" % kernel_source_hash(), "fetch_scale = %.6f" % fs,
          "write_scale = %.6f" % ws, "hbm_bytes_per_launch_mean = %.0f" % statistics.mean(tot)]
    return "\n".join(L) + "\n"


def summarize_single_traffic(args):
    """FETCH_SIZE and WRITE_SIZE of every single-product call (--only-single
    runs), per bench row: the median bytes per call against the algorithmic
    bytes.  A ratio under 0.98 means some weight bytes came from a cache."""
    import statistics
    bl = _bench_json(args.bench_log)
    fe, wr = _counters(args.rocprof_dir[0]), _counters(args.rocprof_dir[1])
    fs, ws = _copy_scale(fe), _copy_scale(wr)

    def per_row(c):
        seq = []
        for n, x in c:
            if _is_main_single(n):
                seq.append([n, x])
            elif n in ("wq::reduce_kernel", "wq::accept_kernel") and seq:
                seq[-1][1] += x
        out, i = [], 0
        for r in bl["single_products"]:
            out.append([x for _, x in seq[i:i + r["calls"]]])
            i += r["calls"]
        if i != len(seq):
            raise SystemExit("%d stream- or split-kernel dispatches left over" % (len(seq) - i))
        return out

    pf, pw = per_row(fe), per_row(wr)
    L = ["# HBM traffic of the single products (workloads 0, 1, 2, 4), from rocprofv3 counters on MI355X", "#",
         "# commands (one counter per run, from the repository root, after `export TMPDIR=/tmp`):",
         "#   " + PROF_CMD["single_fetch"], "#   " + PROF_CMD["single_write"],
         "#   " + _summary_cmd("single-traffic", args), "#",
         "# Scale: FETCH_SIZE x%.4f, WRITE_SIZE x%.4f (the counters on wq_probe_copy of exactly 1 GiB)." % (fs, ws),
         "# Per call (stream or split kernel plus its reduce or accept kernel, median over the row's calls): bytes after",
         "# scaling.  ratio = (fetch + write) / algorithmic bytes; a ratio under 0.98 is flagged (weights served",
         "# from a cache: the rotation over copies did not defeat the 256 MB last-level cache).", "",
         "%-44s %-14s %2s %12s %12s %14s %7s %s" % ("workload", "layout", "N", "fetch_B", "write_B", "algorithmic_B",
                                                   "ratio", "flag")]
    for r, f, w in zip(bl["single_products"], pf, pw):
        fb, wb = statistics.median(f) * 1024 * fs, statistics.median(w) * 1024 * ws
        nb = _row_bytes(r)
        ratio = (fb + wb) / nb
        L.append("%-44s %-14s %2d %12.0f %12.0f %14d %7.4f %s" % (r["name"][:44], r["layout"], r["N"], fb, wb, nb,
                                                                 ratio, "CACHED" if ratio < 0.98 else ""))
    return "\n".join(L) + "\n"


def summarize_chain(args):
    """Kernel trace of the chained MLP rows."""
    rows = _trace(args.rocprof_dir[0])
    L = ["# Kernel trace of the chained MLP pass (64 layers: RMSNorm + gate/up 34816x5120 + SwiGLU, down 5120x17408,",
         "# residual) in bench.py's chained_mlp rows, MI355X", "#",
         "# commands (from the repository root, after `export TMPDIR=/tmp`):",
         "#   " + PROF_CMD["chain"] + " > gpurun_out/prof_ktc.log", "#   " + _summary_cmd("chain", args), "#",
         "# stream_kernel<N, 6>: gate/up with RMSNorm staging and SwiGLU epilogue (100.3 MB of weights per layer);",
         "# stream_kernel<N, 7>: down, K split in chunks (50.1 MB per layer); chain_reduce_kernel: residual update",
         "# and sums of squares (once more per launch for the first layer's norm).  The rows include the warm-up,",
         "# eager, graph-replay runs and the layer-0 check.  The single cooperative launch (chain_kernel<N>) is",
         "# left out of profiled runs (--no-chain-single); bench.py times it with HIP events.  Microseconds.", "",
         "%-40s %7s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "median_us", "min_us", "max_us")]
    keep, order = {}, []
    for s, e, n in rows:
        if not (n.startswith("wq::stream_kernel<") and (n.endswith(", 6>") or n.endswith(", 7>"))
                or n.startswith("wq::chain")):
            continue
        if n not in keep:
            order.append(n)
        keep.setdefault(n, []).append((e - s) / 1e3)
    for n in order:
        L.append("%-40s %7d %12.1f %12.1f %12.1f %12.1f" % ((n[:40],) + _stats(keep[n])))
    return "\n".join(L) + "\n"


SUMMARIES = {"dense": summarize_dense, "single": summarize_single, "traffic": summarize_traffic,
             "single-traffic": summarize_single_traffic, "chain": summarize_chain}


# ---- main ------------------------------------------------------------------------

def run_probes(wq, torch, stream):
    """The read probe (attainable read rate), the read-with-writes probe (the
    price of an output byte) and one copy of exactly 1 GiB (the scale of the
    byte counters in profiled runs)."""
    dev = torch.device("cuda:0")
    probe_buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    probe_buf.fill_(1)
    sink = torch.empty(wq.wq_probe_sink_words(), dtype=torch.int32, device=dev)
    for _ in range(2):
        wq.wq_probe_read(probe_buf, sink, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        wq.wq_probe_read(probe_buf, sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    probe_gbps = 5 * probe_buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # the same read stream with about 1% of its bytes written as scattered
    # 256-byte write-through stores (the verify pass's outputs at N = 8 are
    # 0.9% of its bytes): what an output byte costs in read time
    every_kb = 96
    wdst = torch.empty(wq.wq_probe_read_write_bytes(probe_buf.numel(), every_kb), dtype=torch.uint8, device=dev)
    wq.wq_probe_read_write(probe_buf, wdst, every_kb, sink, stream)
    e0.record(stream)
    for _ in range(5):
        wq.wq_probe_read_write(probe_buf, wdst, every_kb, sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t_rw = e0.elapsed_time(e1) * 1e-3 / 5
    t_r = probe_buf.numel() / (probe_gbps * 1e9)
    write_probe = {"every_kb_read": every_kb, "bytes_read": probe_buf.numel(), "bytes_written": wdst.numel(),
                   "read_only_gbps": probe_gbps, "with_writes_read_gbps": probe_buf.numel() / t_rw / 1e9,
                   "us_per_mb_written": (t_rw - t_r) * 1e6 / (wdst.numel() / 1e6),
                   "read_bytes_lost_per_byte_written": (t_rw - t_r) * probe_gbps * 1e9 / wdst.numel()}
    del wdst
    copy_dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    wq.wq_probe_copy(probe_buf[: 1 << 30], copy_dst, stream)
    torch.cuda.synchronize()
    # the buffers go back to torch's cache, not to the driver: after a
    # hipFree of these 5 GiB the dense pass ran 3% slower until the device
    # next sat idle (measured: 1768 -> 1825 us at N = 2, for 60 passes)
    del probe_buf, copy_dst
    return probe_gbps, write_probe


def only_single(args):
    """--only-single: the probes and the single products, nothing else (the
    run profiled for the single products' kernel trace and byte counters)."""
    import torch
    from fp8_weight_streaming_amd import wq
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    probe_gbps, write_probe = run_probes(wq, torch, stream)
    singles = single_products(wq, torch, stream, probe_gbps)
    ok = None
    if not args.no_cpu_baseline:
        ok = run_oracle_checks()
    print(json.dumps({"single_products": singles, "probe_read_gbps": probe_gbps, "probe_write_cost": write_probe,
                      "parity_ok": ok}))
    if ok is False:
        print("[bench] PARITY FAILED", file=sys.stderr)
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=90)
    ap.add_argument("--warmup", type=int, default=9)
    ap.add_argument("--layers", type=int, default=64, help="layers of the pass (64 is the measured workload)")
    ap.add_argument("--check-rows", type=int, default=32, help="sampled rows per matrix checked against the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-single", action="store_true", help="skip the single-product workloads 0, 1, 2, 4")
    ap.add_argument("--only-single", action="store_true",
                    help="run only the probes and the single products (profiled runs of the single products)")
    ap.add_argument("--no-chain", action="store_true", help="skip the chained MLP pass")
    ap.add_argument("--no-valu", action="store_true", help="skip the MFMA/VALU comparison rows")
    ap.add_argument("--no-chain-single", action="store_true",
                    help="skip the chain's single cooperative launch (kept out of rocprofv3 runs)")
    ap.add_argument("--workers", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--summarize-rocprof", metavar="KIND", choices=sorted(SUMMARIES),
                    help="write a profiles/ summary from rocprofv3 CSV output instead of benchmarking: " +
                         ", ".join(sorted(SUMMARIES)))
    ap.add_argument("--rocprof-dir", action="append", default=[],
                    help="rocprofv3 output directory (twice for the traffic summaries: FETCH_SIZE, then WRITE_SIZE)")
    ap.add_argument("--bench-log", help="stdout of the profiled bench.py run (its JSON line)")
    ap.add_argument("--out", help="summary file to write")
    args = ap.parse_args()

    if args.summarize_rocprof:
        text = SUMMARIES[args.summarize_rocprof](args)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text, end="")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the matrices of a verify pass are "
              "independent and would shard by rows or by matrix with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.only_single:
        only_single(args)
        return

    wl = inputs.workload(3, layers=args.layers)
    t_gen = time.perf_counter()
    print("[bench] generating %d matrices with %d workers" % (len(wl.matrices), args.workers), file=sys.stderr,
          flush=True)
    host = generate(wl, args.workers)
    t_gen = time.perf_counter() - t_gen
    print("[bench] generated in %.1f s" % t_gen, file=sys.stderr, flush=True)

    import torch
    from fp8_weight_streaming_amd import wq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # upload: inputs resident in HBM before anything is timed
    mats_dev = []
    for i, (spec, d) in enumerate(zip(wl.matrices, host)):
        codes = torch.from_numpy(d.codes).to(dev)
        scales = torch.from_numpy(d.scales).to(dev)
        x = torch.from_numpy(d.x.view(np.int16)).to(dev)
        y = torch.zeros((NMAX, spec.M), dtype=torch.float32, device=dev)
        tiled = torch.empty(wq.wq_nvfp4_tiled_bytes(spec.M, spec.K), dtype=torch.uint8, device=dev)
        wq.wq_nvfp4_tile(codes, scales, tiled, stream)
        mats_dev.append((codes, scales, x, y, tiled))
    torch.cuda.synchronize()
    print("[bench] uploaded %.2f GB and tiled it" % (sum(c.numel() + s.numel() for c, s, _, _, _ in mats_dev) / 1e9),
          file=sys.stderr, flush=True)

    def make_plans(fmt):
        plans = {}
        for N in N_CYCLE:
            if fmt == wq.WQ_FMT_NVFP4_TILED:
                mats = [wq.Matrix(fmt, s.M, s.K, t, None, x[:N], y[:N], wl.g)
                        for s, (c, sc, x, y, t) in zip(wl.matrices, mats_dev)]
            else:
                mats = [wq.Matrix(fmt, s.M, s.K, c, sc, x[:N], y[:N], wl.g)
                        for s, (c, sc, x, y, t) in zip(wl.matrices, mats_dev)]
            ws = torch.zeros(wq.wq_verify_workspace_bytes(mats, N), dtype=torch.uint8, device=dev)
            plans[N] = (wq.wq_verify_prepare(mats, N, ws, stream), ws)
        return plans

    plans_t = make_plans(wq.WQ_FMT_NVFP4_TILED)
    plans_p = make_plans(wq.WQ_FMT_NVFP4)
    plans = {N: p for N, (p, _) in plans_t.items()}
    torch.cuda.synchronize()

    bytes_n = {N: algorithmic_bytes(wl, N) for N in N_CYCLE}

    # The reported-only rows that stream the same 12 GB run first: on a
    # device that has been idle (generation, upload), the first ~10 passes
    # run up to 25% slower while its clocks come up (measured: 2500, 2144,
    # 2032, ... 1966 us at N = 8), more than a few warm-up steps cover;
    # these rows put ~180 ms of streaming ahead of the warm-up.

    # the plain row-major layout (reported only)
    plain = {}
    for N in N_CYCLE:
        p = plans_p[N][0]
        for _ in range(2):
            wq.wq_verify_launch(p, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(9):
            wq.wq_verify_launch(p, stream)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / 9 * 1e3
        plain[str(N)] = {"us_per_pass": us, "gbps": bytes_n[N] / us / 1e3}

    device_n = device_n_rows(wq, torch, stream, wl, mats_dev, bytes_n)

    probe_gbps, write_probe = run_probes(wq, torch, stream)

    # warmup
    for i in range(args.warmup):
        wq.wq_verify_launch(plans[N_CYCLE[i % 3]], stream)
    torch.cuda.synchronize()

    # timed region
    steps = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    ns = [N_CYCLE[i % 3] for i in range(steps)]
    launch = wq.lib().wq_verify_launch
    import ctypes
    plan_refs = {N: ctypes.byref(plans[N]) for N in N_CYCLE}
    sptr = stream.cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        st = launch(plan_refs[ns[i]], sptr)
        ev[i][1].record(stream)
        if st != 0:
            raise RuntimeError("wq_verify_launch failed: %d" % st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    wall_s = t1 - t0
    durs = np.array([a.elapsed_time(b) * 1e-3 for a, b in ev])  # seconds per launch
    total_bytes = sum(bytes_n[N] for N in ns)
    value = total_bytes / wall_s / 1e9
    per_n = {}
    for N in N_CYCLE:
        d = durs[[j for j in range(steps) if ns[j] == N]]
        per_n[str(N)] = {"us_per_pass_mean": float(d.mean() * 1e6), "us_per_pass_min": float(d.min() * 1e6),
                         "algorithmic_bytes": bytes_n[N],
                         "gbps": float(bytes_n[N] / d.mean() / 1e9),
                         "pct_of_8TBps": float(100 * bytes_n[N] / d.mean() / 1e9 / PEAK_GBPS)}
    kernel_s = float(durs.sum())
    achieved = total_bytes / kernel_s / 1e9
    traffic, traffic_kv = read_traffic()
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / PEAK_GBPS, "traffic": traffic,
                "kernel": "wq::stream_kernel<N, 4> (the tiled verify pass: one launch per pass; its split "
                          "matrices are computed in LDS blocks, so no reduction launch follows)",
                "avg_launch_us": kernel_s / steps * 1e6,
                "algorithmic_bytes_per_launch_mean": total_bytes / steps,
                "traffic_gbps": (traffic / (kernel_s / steps) / 1e9) if traffic else None,
                "probe_read_gbps": probe_gbps, "frac_of_probe": achieved / probe_gbps,
                "probe_write_cost": write_probe}

    # parity: sampled rows of every matrix at every N (compared with the
    # oracle in the cpu_baseline leg)
    rng = np.random.default_rng(12345)
    samples = []
    for N in N_CYCLE:
        wq.wq_verify_launch(plans[N], stream)
        torch.cuda.synchronize()
        for i, (spec, d) in enumerate(zip(wl.matrices, host)):
            rows = np.unique(np.concatenate([rng.integers(0, spec.M, args.check_rows), [0, spec.M - 1]]))
            y = mats_dev[i][3][:N].cpu().numpy()[:, rows].astype(np.float64)
            samples.append((d.codes[rows], d.scales[rows], d.g, d.x[:N], y))
    parity = {"ok": None, "elements_checked": int(sum(smp[4].size for smp in samples)), "max_err_over_bound": None,
              "bound": "|y - y_oracle| <= 1e-3 * sum|w*x|"}
    PENDING.append((check_sampled_nvfp4, parity, {"samples": samples}))
    ok = True

    valu = None
    if not args.no_valu:
        valu = valu_rows(wq, torch, stream, wl, host, mats_dev, plans, bytes_n)
    chained = None
    if not args.no_chain:
        chained = chain_rows(wq, torch, stream, wl, host, mats_dev, probe_gbps,
                             single_launch=not args.no_chain_single)
    draft = None
    singles = quant = None
    if not args.no_single:
        draft = draft_step_row(wq, torch, stream, wl, host, mats_dev, probe_gbps)
        del plans_p
        singles = single_products(wq, torch, stream, probe_gbps)
        quant = quantizer_rows(wq, torch, stream, probe_gbps)

    # the cpu_baseline leg: the oracle timed on a bounded sample, then every
    # comparison of GPU outputs with it (without this leg nothing is checked)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, host)
        ok = run_oracle_checks()
    else:
        parity["note"] = "not checked: the oracle runs only in the cpu_baseline leg (--no-cpu-baseline)"

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": wall_s / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": args.layers, "matrices": len(wl.matrices),
                   "weight_format": "nvfp4 (e2m1 codes, e4m3 scale per 16 k, fp32 tensor scale)",
                   "activations": "bf16", "outputs": "fp32", "n_cycle": N_CYCLE,
                   "weight_bytes_per_pass": sum(s.M * s.K // 2 + s.M * s.K // 16 for s in wl.matrices),
                   "pct_of_8TBps": 100 * value / PEAK_GBPS,
                   "us_per_pass": wall_s / steps * 1e6},
        # the long secondary rows first; the per-N figures, the parity
        # check, the CPU baseline and the roofline close the line
        "plain_layout": plain,
        "per_n_device_count": device_n,
        "mfma_vs_valu": valu,
        "draft_step": draft,
        "chained_mlp": chained,
        "single_products": singles,
        "quantizers": quant,
        "per_n": per_n,
        "parity": parity,
        "cpu_baseline": cpu,
        "roofline": roofline,
    }
    print(json.dumps(out))
    if not ok:
        print("[bench] PARITY FAILED", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
