#!/usr/bin/env python3
"""Benchmark: Vertical-Slash sparse attention (index estimate + forward + backward) on one MI355X.

Workload (default, --workload 3): one Qwen2.5-3B-shaped attention layer at
N = 131072, bf16, 16 Q / 2 KV heads, head_dim 128, causal, 64-token blocks,
vertical budget 2048 and slash budget 8192 tokens, seeded synthetic
Q/K/V/dO with RoPE and 0.1% outlier keys.  One step = vs_estimate_index +
vs_sparse_attn_fwd + vs_sparse_attn_bwd over inputs already resident in HBM.
Workloads 1, 2 and 5 time the same step on their shapes; workload 4 times one
striped worker's ring share: 32 forward calls (one per KV chunk, the merge
fused into each), delta, and 32 backward calls accumulating dQ, against an
index estimated once on the whole 524288-token sequence (untimed).

Prints one JSON line.  value = executed TFLOP/s = 14 * d * H_q * |M| / t_step
(|M| = valid entries of the index per head; 4d forward + 10d backward per
entry); also dense-equivalent TFLOP/s over the causal area and the fraction
of the bf16 matrix-core peak.  `roofline` is for the kernel with the largest
time per step; its `achieved` credits the kernel only its own share of the
method's work (forward 4d per entry: S and O; dQ kernel 6d: S, dP, dQ; each
dK/dV kernel 4d: dV and dK); the matrix-core work it actually issues,
recomputation included, is reported beside it as `executed_mfma`.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd sparse attn TFLOP/s (executed & dense-equiv), % bf16 MFMA peak, N=128K"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense matrix-core peaks (published)

# Matrix-core FLOPs per valid entry per head dimension, per kernel: the share
# of the method's work each kernel owns (the forward's S and O products; the
# backward's S recompute, dP and dQ in the dQ kernel; dV and dK in the dK/dV
# kernels), and what each kernel issues (the dK/dV kernels recompute S and dP).
OWN_PER_ENTRY = {"vs_fwd": 4, "vs_bwd_dq": 6, "vs_bwd_dkdv_slash": 4, "vs_bwd_dkdv_cols": 4}
ISSUED_PER_ENTRY = {"vs_fwd": 4, "vs_bwd_dq": 6, "vs_bwd_dkdv_slash": 8, "vs_bwd_dkdv_cols": 8}
# which entries a kernel processes: all, the slash-block ones or the vertical-column ones
ENTRY_KIND = {"vs_fwd": "all", "vs_bwd_dq": "all", "vs_bwd_dkdv_slash": "slash",
              "vs_bwd_dkdv_cols": "vertical"}

# HBM peak of MI355X (published), for the bandwidth-bound kernels.
HBM_PEAK_GBS = 8000.0


def hbm_alg_bytes(name, c):
    """Algorithmic bytes per launch of the bandwidth-bound kernels: what each
    must read and write once.  c: batch, n, h_q, h_kv, d, el (input element
    bytes), n_lists, tiles (256-key estimator tiles), nb (64-blocks), v_ent /
    s_ent (vertical / block-diagonal list entries, padding included)."""
    K = c["batch"] * c["n"] * c["h_kv"] * c["d"] * c["el"]
    Qw = c["n_lists"] * 64 * c["d"] * c["el"]                 # the window rows of every list
    part = c["batch"] * c["h_q"] * c["tiles"] * 64 * 8         # (max, sum) per window row and key tile
    lse = c["n_lists"] * 64 * 4
    vsc = c["batch"] * c["h_q"] * c["n"] * 4                   # column scores v[m]
    ssc = c["batch"] * c["h_q"] * c["nb"] * 4                  # block-diagonal scores
    lists = 4 * (c["v_ent"] + c["s_ent"])
    table = {
        "vs_est_pass1": K + Qw + part,
        "vs_est_combine": part + lse,
        "vs_est_pass2": K + Qw + lse + vsc + ssc,
        # the two-stage top-k: the chunks read the column scores, the last
        # stage the block-diagonal scores (and the chunks' candidates) and
        # writes the lists
        "vs_est_topk_chunk": vsc,
        "vs_est_topk": ssc + lists,
        "vs_prep_vertical": 2 * 4 * c["v_ent"],
        "vs_moba_means": K,
        "vs_moba_select": c["batch"] * c["n"] * c["h_q"] * (c["d"] * c["el"] + 4),
    }
    return table.get(name)


# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, each scaled by what the same counter reads for a plain copy of
# known size) are kept per workload in profiles/hbm_traffic_<workload>.json,
# each kernel's figure with a digest of its sources: it is reported only while
# they are unchanged.

# Host cores the CPU baseline may use on the GPU machine (its CPU share).
CPU_SHARE = 16


# The translation unit of each traced kernel (bf16 path); the rest are in
# vs_estimate.hip (vs_est_*) or vs_misc.hip.
KERNEL_SOURCE = {"vs_fwd": "vs_fwd.hip", "vs_bwd_dq": "vs_bwd_dq.hip", "vs_bwd_dkdv_slash": "vs_bwd_kv.hip",
                 "vs_bwd_dkdv_cols": "vs_bwd_kv.hip", "vs_xa_cells": "vs_xattn.hip",
                 "vs_xa_select": "vs_xattn.hip", "vs_moba_means": "vs_moba.hip", "vs_moba_select": "vs_moba.hip",
                 "vs_moba_union": "vs_moba.hip"}


def kernel_digest(kernel):
    """SHA-256 of a kernel's translation unit and the local headers it
    includes (recursively), so that a counter figure stays valid exactly as
    long as the code it was taken from."""
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_amd", "csrc")
    tu = KERNEL_SOURCE.get(kernel, "vs_estimate.hip" if kernel.startswith("vs_est_") else "vs_misc.hip")
    seen, stack = set(), [tu]
    while stack:
        f = stack.pop()
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            continue
        seen.add(f)
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            for line in fh:
                line = line.strip()
                if line.startswith("#include \""):
                    stack.append(line.split("\"")[1])
    h = hashlib.sha256()
    for f in sorted(seen):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    try:
        with open(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel)
    if data.get("workload") != workload or ent is None or ent.get("source_sha256") != kernel_digest(kernel):
        return None
    return int(ent["hbm_bytes_per_launch"])


# rocprofv3 kernel names -> traced names
_PROF_NAMES = (("vs_fwd_rows_kernel", "vs_fwd"), ("vs_bwd_dq_rows_kernel", "vs_bwd_dq"),
               ("vs_bwd_kv_slash_bf16_kernel", "vs_bwd_dkdv_slash"), ("vs_bwd_kv_pair_bf16_kernel", "vs_bwd_dkdv_slash"),
               ("vs_bwd_kv_cols_bf16_kernel", "vs_bwd_dkdv_cols"),
               ("vs_delta_kernel", "vs_delta"), ("vs_est_pass1", "vs_est_pass1"), ("vs_est_pass2", "vs_est_pass2"),
               ("vs_est_topk_chunk_kernel", "vs_est_topk_chunk"), ("vs_est_topk_kernel", "vs_est_topk"),
               ("vs_est_combine", "vs_est_combine"), ("vs_lse_log2", "vs_lse_log2"),
               ("vs_prep_vertical", "vs_prep_vertical"), ("vs_group_share", "vs_group_share"),
               ("vs_xa_cells_kernel", "vs_xa_cells"), ("vs_xa_select_kernel", "vs_xa_select"),
               ("vs_moba_means_kernel", "vs_moba_means"), ("vs_moba_select_kernel", "vs_moba_select"),
               ("vs_moba_union_kernel", "vs_moba_union"))


def write_traffic(run_dir, workload):
    """profiles/hbm_traffic_<workload>.json from four rocprofv3 counter runs
    under run_dir (fetch, write: the benchmark; copy_fetch, copy_write: the
    copy probe): per kernel the mean FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the bytes the copy moves per KiB the same
    counter reads for it, and the kernel's source digest."""
    import collections
    import csv

    def load(sub):
        agg = collections.defaultdict(list)
        with open(os.path.join(run_dir, sub, "run_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return agg

    def mean(xs):
        return sum(xs) / len(xs)

    fetch, write = load("fetch"), load("write")
    copy = "__amd_rocclr_copyBuffer"
    cf = [v for k, v in load("copy_fetch").items() if copy in k][0]
    cw = [v for k, v in load("copy_write").items() if copy in k][0]
    f_fetch = (1 << 30) / (mean(cf) * 1024)
    f_write = (1 << 30) / (mean(cw) * 1024)
    kern = {}
    for k in fetch:
        name = next((b for a, b in _PROF_NAMES if a in k), None)
        if name is None or k not in write:
            continue
        fk, wk = mean(fetch[k]), mean(write[k])
        kern[name] = {"fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                      "hbm_bytes_per_launch": int(fk * 1024 * f_fetch + wk * 1024 * f_write),
                      "source_sha256": kernel_digest(name)}
    out = {"workload": workload, "copy_factor_fetch": round(f_fetch, 4), "copy_factor_write": round(f_write, 4),
           "kernels": kern}
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def ring_graph(step, stream, args, acc_o, acc_l, dq, dkv, ent, d):
    """The worker's 32-call ring (forward with the merge fused, delta, backward
    accumulating dQ) captured once as a HIP graph and replayed: the step's
    ~290 kernel launches reach the GPU without a host round trip each.  The
    replayed results must equal the eager ring's (O, LSE and dQ exactly; dK
    and dV, which take fp32 atomics, within 1e-5 of their largest value)."""
    import torch
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (acc_o, acc_l, dq)]
    ref_kv = [(a.clone(), b.clone()) for a, b in dkv]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    for a, b in zip(ref, (acc_o, acc_l, dq)):
        if not torch.equal(a, b):
            raise RuntimeError("the graph replay of the ring differs from the eager ring")
    for (a, b), (c, e) in zip(ref_kv, dkv):
        for x, y in ((a, c), (b, e)):
            if float((x - y).abs().max()) > 1e-5 * max(float(x.abs().max()), 1.0):
                raise RuntimeError("the graph replay's dK / dV differ from the eager ring's")
    del g
    return {"ms_per_step": round(ms, 4), "exec_tflops": round(14 * d * ent / (ms * 1e-3) / 1e12, 3),
            "replays_checked": True}


def copy_probe(dev):
    """A plain device copy of known size, for calibrating the HBM byte counters."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": {"bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                                     "launches": 10}}), flush=True)


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def trace_read(vs):
    buf = ctypes.create_string_buffer(1 << 16)
    vs._abi.check(vs._abi.lib().vs_trace_collect(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, tot = line.split()
        out[name] = (int(cnt), float(tot))
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, over a pool of single-threaded
# worker processes.  The pool is forked before the GPU is first touched, so
# the workers share the fp64 inputs copy-on-write and hold no GPU state.
_SHARED = {}


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _oracle_estimate(h):
    import oracle
    s = _SHARED
    g = h * s["h_kv"] // s["h_q"]
    t0 = time.perf_counter()
    if s["topp"] is None:
        oracle.estimate_index(s["q"][:, h:h + 1], s["k"][:, g:g + 1], s["cu"], [s["vb"][h]], [s["sb"][h]])
    else:
        oracle.estimate_index_topp(s["q"][:, h:h + 1], s["k"][:, g:g + 1], s["cu"], [s["vb"][h]],
                                   [s["sb"][h]], [s["topp"][0]], [s["topp"][1]])
    return time.perf_counter() - t0


def _oracle_fwd_bwd(h, row_pos, index_h):
    """Support-form forward + backward of the given rows of Q head h."""
    import numpy as np
    import oracle
    s = _SHARED
    g = h * s["h_kv"] // s["h_q"]
    rows = np.asarray(row_pos)
    t0 = time.perf_counter()
    qh, doh = s["q"][rows, h:h + 1], s["do"][rows, h:h + 1]
    kg, vg = s["k"][:, g:g + 1], s["v"][:, g:g + 1]
    pos = np.arange(s["k"].shape[0]) if s["key_pos"] is None else s["key_pos"]
    O, L = oracle.attn_fwd_support(qh, kg, vg, rows, pos, s["cu"], index_h)
    D = oracle.bwd_delta(O, doh)
    oracle.attn_bwd_support(qh, kg, vg, doh, L, D, rows, pos, s["cu"], index_h)
    return time.perf_counter() - t0


class OraclePool:
    """Worker processes for the CPU baseline, forked while the process holds no GPU state."""

    def __init__(self, prob, topp, procs):
        import numpy as np
        import torch
        f64 = lambda t: t[0].to(torch.float64).numpy()
        _SHARED.update(q=f64(prob.q), k=f64(prob.k), v=f64(prob.v), do=f64(prob.do), cu=prob.cu_seqlens,
                       vb=prob.v_budget, sb=prob.s_budget, h_q=prob.h_q, h_kv=prob.h_kv, topp=topp,
                       key_pos=None)
        self.procs = procs
        self.pool = mp.get_context("fork").Pool(procs, initializer=_worker_init)
        self.np = np

    def close(self):
        self.pool.terminate()
        self.pool.join()


def _blocks_entries(acc, lists_h, cu, blocks):
    """Valid entries of the given global query blocks of one head (any segments)."""
    import numpy as np
    cu = list(cu)
    n_seg = len(cu) - 1
    tot = 0
    blocks = np.asarray(blocks)
    for s in range(n_seg):
        a, e = cu[s], cu[s + 1]
        sel = blocks[(blocks * 64 >= a) & (blocks * 64 < e)] - a // 64
        if sel.size == 0:
            continue
        iv, is_ = lists_h[s]
        iv = np.asarray(iv)
        tot += int(acc.executed_area([(iv[iv >= 0] - a, is_)], [0, e - a], 1, row_blocks=sel)[0])
    return tot


def cpu_baseline(pool, prob, lists, total_entries, target_s, row_blocks=None):
    """The oracle, as it stands, on a bounded sample of the same workload.

    Sample: the estimator for every Q head, then support-form forward +
    backward of query blocks spread evenly over the sequence and the heads
    (4 blocks per task), submitted while less than target_s seconds have
    passed.  Job time = estimator time + (sample time / sample entries) x |M|.
    """
    import numpy as np
    from dynamic_sparse_attention_amd import accounting as acc
    n_seg = len(prob.cu_seqlens) - 1
    hq = prob.h_q
    t0 = time.perf_counter()
    pool.pool.map(_oracle_estimate, range(hq))
    t_est = time.perf_counter() - t0
    blocks_all = np.arange(prob.n // 64) if row_blocks is None else np.asarray(row_blocks)
    nb = blocks_all.size
    spread = np.concatenate([blocks_all[s::64] for s in range(min(64, nb))])
    tasks = []
    for i in range(0, nb, 4):
        for h in range(hq):
            tasks.append((h, spread[(i + 4 * h) % nb: (i + 4 * h) % nb + 4]))
    index = [{(0, s): (np.asarray(lists[h * n_seg + s][0]), np.asarray(lists[h * n_seg + s][1]))
              for s in range(n_seg)} for h in range(hq)]
    t1 = time.perf_counter()
    pending, done = [], []
    it = iter(tasks)
    while True:
        while len(pending) < 2 * pool.procs and time.perf_counter() - t1 < target_s:
            nxt = next(it, None)
            if nxt is None:
                break
            h, blks = nxt
            rows = (blks[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)
            pending.append((h, blks, pool.pool.apply_async(_oracle_fwd_bwd, (h, rows, index[h]))))
        if not pending:
            break
        h, blks, r = pending.pop(0)
        r.get()
        done.append((h, blks))
    t_fb = time.perf_counter() - t1
    lists_h = lambda h: [(lists[h * n_seg + s][0], lists[h * n_seg + s][1]) for s in range(n_seg)]
    ent = sum(_blocks_entries(acc, lists_h(h), prob.cu_seqlens, blks) for h, blks in done)
    job_s = t_est + t_fb / max(ent, 1) * total_entries
    flops = 14 * prob.d * total_entries
    return {"value": round(flops / job_s / 1e12, 6), "unit": "TFLOP/s", "cores": pool.procs,
            "kind": "oracle", "host_cpus": os.cpu_count(),
            "sample": (f"fp64 numpy oracle on {pool.procs} single-threaded worker processes "
                       f"(host reports {os.cpu_count()} CPUs): estimator for all {hq} heads "
                       f"({t_est:.2f} s wall) and support-form fwd+bwd of {len(done)} tasks of 4 "
                       f"query blocks spread over the sequence and the heads ({ent} of "
                       f"{total_entries} entries, {t_fb:.2f} s wall); job time extrapolated "
                       f"to {job_s:.1f} s")}


# ---------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3,
                    help="workload id: 3 = N=131072 (default); 1, 2, 5 contiguous; 4 = striped worker")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--topp", default=None, metavar="P_V,P_S",
                    help="estimate with top-p budgets (vs_estimate_index_topp) at these mass "
                         "fractions, the workload's budgets as caps")
    ap.add_argument("--estimator", choices=("vs", "xattn", "moba"), default="vs",
                    help="vs: the Vertical-Slash index (default); xattn: XAttention block "
                         "selection (vs_estimate_index_xattn, block 128, stride 16); moba: the MoBA "
                         "block gate (vs_estimate_index_moba)")
    ap.add_argument("--threshold", type=float, default=0.9, help="XAttention selection threshold")
    ap.add_argument("--moba-block", type=int, default=4096, help="MoBA key block (tokens)")
    ap.add_argument("--moba-topk", type=int, default=12, help="MoBA blocks per query")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--write-traffic", metavar="RUN_DIR", default=None,
                    help="no GPU: write profiles/hbm_traffic_<workload>.json from rocprofv3 counter runs "
                         "RUN_DIR/{fetch,write,copy_fetch,copy_write}")
    args = ap.parse_args()
    if args.write_traffic:
        import workloads
        write_traffic(args.write_traffic, workloads.WORKLOADS[args.workload]["name"])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import workloads

    topp = None
    if args.topp:
        topp = tuple(float(x) for x in args.topp.split(","))
        if len(topp) != 2:
            raise SystemExit("--topp takes P_V,P_S")
    if topp is not None and args.workload == 4:
        raise SystemExit("--topp is for the contiguous workloads")
    if args.estimator != "vs" and (topp is not None or args.workload in (4, 5)):
        raise SystemExit("--estimator xattn / moba take one contiguous segment (workloads 1-3), no --topp")

    pool = None
    if args.copy_probe:
        prob = None
    else:
        t0 = time.time()
        prob = workloads.make_problem(args.workload)
        log(f"inputs {prob.name}: n={prob.n} in {time.time() - t0:.1f} s")
        if not args.no_cpu_baseline and args.estimator == "vs":
            pool = OraclePool(prob, topp, min(CPU_SHARE, os.cpu_count() or 1))

    import torch
    import dynamic_sparse_attention_amd as vs
    from dynamic_sparse_attention_amd import accounting

    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(dev)
        return
    try:
        out, lists, total_entries, row_blocks = run(args, prob, topp, dev, torch, vs, accounting, np)
        if pool is not None:
            if row_blocks is not None:
                _SHARED["key_pos"] = None
            t1 = time.time()
            out["cpu_baseline"] = cpu_baseline(pool, prob, lists, total_entries, args.cpu_seconds, row_blocks)
            log(f"cpu baseline {out['cpu_baseline']['value']} TFLOP/s in {time.time() - t1:.1f} s")
    finally:
        if pool is not None:
            pool.close()
    print(json.dumps(out), flush=True)


def run(args, prob, topp, dev, torch, vs, accounting, np):
    cu = prob.cu_seqlens
    Hq, d = prob.h_q, prob.d
    stream = torch.cuda.current_stream(dev)
    worker = args.workload == 4
    xattn = args.estimator == "xattn"
    moba = args.estimator == "moba"
    if not worker:
        q, k, v, do = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
        o = torch.empty_like(q)
        lse = torch.empty((1, Hq, prob.n), dtype=torch.float32, device=dev)
        dq = torch.empty((1, prob.n, Hq, d), dtype=torch.float32, device=dev)
        dk = torch.empty((1, prob.n, prob.h_kv, d), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)

        def estimate():
            if xattn:
                return vs.estimate_index_xattn(q, k, args.threshold)[0]
            if moba:
                return vs.estimate_index_moba(q, k, args.moba_block, args.moba_topk)
            if topp is None:
                return vs.estimate_index(q, k, prob.v_budget, prob.s_budget, cu)
            return vs.estimate_index_topp(q, k, prob.v_budget, prob.s_budget, [topp[0]] * Hq,
                                          [topp[1]] * Hq, cu)[0]

        idx = estimate()
        row_blocks = None
        row_pos = None
        phase_names = ("estimate", "fwd", "bwd")

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            ix = estimate()
            if ev is not None:
                ev[1].record(stream)
            vs.sparse_attn_fwd(q, k, v, ix, cu, out=o, lse=lse)
            if ev is not None:
                ev[2].record(stream)
            vs.sparse_attn_bwd(q, k, v, o, do, lse, ix, cu_seqlens=cu, dq=dq, dk=dk, dv=dv)
            if ev is not None:
                ev[3].record(stream)
    else:
        # One striped worker's ring share (64-token stripes, worker w of W):
        # the index is estimated once on the whole sequence (untimed); the
        # worker's rows and the W KV chunks are staged before timing.
        W, w = prob.stripe_world, prob.stripe_rank
        gq_all, gk_all = prob.q.to(dev), prob.k.to(dev)
        idx = vs.estimate_index(gq_all, gk_all, prob.v_budget, prob.s_budget, cu)
        torch.cuda.synchronize()
        del gq_all, gk_all
        row_pos = workloads_stripe(prob, W, w)
        row_blocks = row_pos[::64] // 64
        q = _stripe(prob.q, W, w).to(dev)
        do = _stripe(prob.do, W, w).to(dev)
        nq = q.shape[1]
        ring = [(w - t) % W for t in range(W)]
        chunks = [(u, _stripe(prob.k, W, u).to(dev), _stripe(prob.v, W, u).to(dev)) for u in ring]
        acc_o = torch.empty((1, nq, Hq, d), dtype=torch.float32, device=dev)
        acc_l = torch.empty((1, Hq, nq), dtype=torch.float32, device=dev)
        dq = torch.empty((1, nq, Hq, d), dtype=torch.float32, device=dev)
        dkv = [(torch.empty((1, nq, prob.h_kv, d), dtype=torch.float32, device=dev),
                torch.empty((1, nq, prob.h_kv, d), dtype=torch.float32, device=dev)) for _ in ring]
        phase_names = ("fwd", "bwd")
        # the same ring share as one call per pass: K / V hold the W chunks one
        # after the other (chunk u = the keys of rank u)
        k_all = torch.cat([c[1] for c in sorted(chunks, key=lambda c: c[0])], dim=1)
        v_all = torch.cat([c[2] for c in sorted(chunks, key=lambda c: c[0])], dim=1)
        o_one = torch.empty((1, nq, Hq, d), dtype=torch.float32, device=dev)
        l_one = torch.empty((1, Hq, nq), dtype=torch.float32, device=dev)
        dq_one = torch.empty_like(dq)
        dk_one = torch.empty((1, prob.n, prob.h_kv, d), dtype=torch.float32, device=dev)
        dv_one = torch.empty_like(dk_one)

        def step_one(ev=None):
            if ev is not None:
                ev[0].record(stream)
            vs.sparse_attn_fwd(q, k_all, v_all, idx, stripe=(W, w, "all"), out=o_one, lse=l_one, o_f32=True)
            if ev is not None:
                ev[1].record(stream)
            vs.sparse_attn_bwd(q, k_all, v_all, o_one, do, l_one, idx, dq=dq_one, dk=dk_one, dv=dv_one,
                               stripe=(W, w, "all"))
            if ev is not None:
                ev[2].record(stream)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            acc_o.zero_()
            acc_l.fill_(-float("inf"))
            for u, gk, gv in chunks:
                vs.sparse_attn_fwd(q, gk, gv, idx, stripe=(W, w, u), out=acc_o, lse=acc_l, merge=True)
            if ev is not None:
                ev[1].record(stream)
            delta = vs.attn_bwd_delta(acc_o, do)
            dq.zero_()
            for (u, gk, gv), (dk_u, dv_u) in zip(chunks, dkv):
                vs.sparse_attn_bwd(q, gk, gv, None, do, acc_l, idx, delta=delta, dq=dq, dk=dk_u, dv=dv_u,
                                   stripe=(W, w, u), accumulate=True)
            if ev is not None:
                ev[2].record(stream)

    lists = [(a.numpy(), b.numpy()) for a, b in idx.lists()]
    if xattn:
        # block selection: every entry is walked by the block-tile path of the
        # query-major kernels and the slash dK/dV kernel
        ent = int(accounting.block_selection_area(idx.block_selection(prob.n).numpy(), prob.n).sum())
        entries = {"all": ent, "slash": ent, "vertical": 0}
    elif moba:
        # per-row selection: the same tile paths, masked per row
        ent = int(accounting.row_selection_area(idx.row_mask.cpu().numpy(), prob.n, args.moba_block).sum())
        entries = {"all": ent, "slash": ent, "vertical": 0}
    else:
        ent_heads = accounting.executed_area(lists, cu, Hq, row_blocks=row_blocks)
        ent = int(ent_heads.sum())
        split = accounting.executed_split(lists, cu, Hq, row_blocks=row_blocks)
        entries = {"all": ent, "slash": int(split["slash"].sum()), "vertical": int(split["vertical"].sum())}
    dense = accounting.dense_causal_area(cu, row_positions=row_pos) * Hq
    log(f"index: executed entries {ent} of {dense} causal ({ent / dense:.4f})")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lib = vs._abi.lib()
    lib.vs_trace_enable(1)
    trace_read(vs)
    nev = len(phase_names) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    lib.vs_trace_enable(0)
    kern = trace_read(vs)
    ms = start.elapsed_time(stop) / args.steps
    phases = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
              for j, name in enumerate(phase_names)}
    exec_tf = 14 * d * ent / (ms * 1e-3) / 1e12
    dense_tf = 14 * d * dense / (ms * 1e-3) / 1e12
    log(f"step {ms:.3f} ms; phases {phases}")
    one_call = merge_rec = graph_rec = None
    if worker:
        for _ in range(args.warmup):
            step_one()
        ev1 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        lib.vs_trace_enable(1)
        start.record(stream)
        for i in range(args.steps):
            step_one(ev1[i])
        stop.record(stream)
        torch.cuda.synchronize()
        lib.vs_trace_enable(0)
        kern1 = trace_read(vs)
        ms1 = start.elapsed_time(stop) / args.steps
        one_call = {"ms_per_step": round(ms1, 4), "exec_tflops": round(14 * d * ent / (ms1 * 1e-3) / 1e12, 3),
                    "phases_ms": {"fwd": round(float(np.mean([e[0].elapsed_time(e[1]) for e in ev1])), 4),
                                  "bwd": round(float(np.mean([e[1].elapsed_time(e[2]) for e in ev1])), 4)},
                    "kernels_avg_ms": {n_: round(t_ / c_, 4) for n_, (c_, t_) in kern1.items()}}
        log(f"one call over all chunks: {ms1:.3f} ms per step; {one_call}")
        # the boundary's lse_merge on the worker's share (fp32 O [1, rows,
        # H_q, d] and LSE), a standalone call: read both results, write one
        o_part, l_part = acc_o.clone(), acc_l.clone()
        for _ in range(2):
            vs.lse_merge(acc_o, acc_l, o_part, l_part)
        torch.cuda.synchronize()
        lib.vs_trace_enable(1)
        for _ in range(10):
            vs.lse_merge(acc_o, acc_l, o_part, l_part)
        torch.cuda.synchronize()
        lib.vs_trace_enable(0)
        cnt_m, tot_m = trace_read(vs)["vs_lse_merge"]
        mb = 3 * acc_o.numel() * 4 + 3 * acc_l.numel() * 4
        avg_m = tot_m / cnt_m * 1e-3
        merge_rec = {"avg_ms": round(tot_m / cnt_m, 4), "alg_bytes": int(mb),
                     "alg_gbs": round(mb / avg_m / 1e9, 1), "alg_hbm_frac": round(mb / avg_m / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"lse_merge on the worker's share: {merge_rec}")
        graph_rec = ring_graph(step, stream, args, acc_o, acc_l, dq, dkv, ent, d)
        log(f"ring as a HIP graph: {graph_rec}")
    for name, (cnt, tot) in sorted(kern.items(), key=lambda x: -x[1][1]):
        log(f"  kernel {name}: {cnt} launches, avg {tot / cnt:.4f} ms, {tot / args.steps:.4f} ms per step")

    peak = PEAK_TFLOPS[prob.dtype]
    # counter figures are kept per workload for its default index (the
    # Vertical-Slash estimator with fixed budgets); other indices make other
    # walks, and their traffic is reported only from a file of their own
    traffic_key = prob.name if (args.estimator == "vs" and topp is None) else f"{prob.name}-{args.estimator}" + (
        "-topp" if topp is not None else "")
    seg_len = np.diff(np.asarray(cu))
    shape = {"batch": 1, "n": prob.n, "h_q": Hq, "h_kv": prob.h_kv, "d": d,
             "el": 2 if prob.dtype == "bf16" else 4, "n_lists": Hq * len(seg_len),
             "tiles": int(sum(-(-int(L) // 256) for L in seg_len)), "nb": prob.n // 64,
             "v_ent": int(sum(a_.size for a_, _ in lists)), "s_ent": int(sum(b_.size for _, b_ in lists))}
    # Per attention kernel: its own share of the method's work and the work it
    # issues, per step, and the rates over its time per step.
    per_kernel = {}
    for name, (cnt, tot) in kern.items():
        ms_step = tot / args.steps
        rec = {"launches_per_step": cnt / args.steps, "avg_ms": round(tot / cnt, 4),
               "ms_per_step": round(ms_step, 4)}
        if name in OWN_PER_ENTRY:
            e = entries[ENTRY_KIND[name]]
            own = OWN_PER_ENTRY[name] * d * e
            issued = ISSUED_PER_ENTRY[name] * d * e
            rec.update(own_tflop=round(own / 1e12, 4), own_tflops=round(own / (ms_step * 1e-3) / 1e12, 2),
                       own_frac=round(own / (ms_step * 1e-3) / 1e12 / peak, 4),
                       issued_tflops=round(issued / (ms_step * 1e-3) / 1e12, 2))
        if name == "vs_xa_cells":
            # causal cell logits: 16 sampled products of d per cell, nC (nC + 1) / 2 cells per head
            nC = prob.n // 16
            own = 2 * 16 * d * (nC * (nC + 1) // 2) * Hq
            rec.update(own_tflop=round(own / 1e12, 4), own_tflops=round(own / (ms_step * 1e-3) / 1e12, 2),
                       own_frac=round(own / (ms_step * 1e-3) / 1e12 / peak, 4))
        ab = hbm_alg_bytes(name, shape)
        if ab is not None:
            # bandwidth-bound kernels: algorithmic bytes (and the counters'
            # HBM bytes, when current) over the average launch
            avg = tot / cnt * 1e-3
            rec.update(alg_bytes=int(ab), alg_gbs=round(ab / avg / 1e9, 1),
                       alg_hbm_frac=round(ab / avg / 1e9 / HBM_PEAK_GBS, 4))
            hb = measured_traffic(name, traffic_key)
            if hb is not None:
                rec.update(hbm_bytes=hb, hbm_gbs=round(hb / avg / 1e9, 1))
        per_kernel[name] = rec

    # Roofline of the dominant kernel (largest time per step): its own share
    # of the method's matrix-core FLOPs per launch over its average launch
    # duration (HIP events on the launch's stream).
    dom = max(kern.items(), key=lambda x: x[1][1])[0]
    cnt, tot = kern[dom]
    avg_s = tot / cnt * 1e-3
    launches = cnt / args.steps
    traffic = measured_traffic(dom, traffic_key)
    if dom in OWN_PER_ENTRY:
        e = entries[ENTRY_KIND[dom]]
        ach = OWN_PER_ENTRY[dom] * d * e / launches / avg_s / 1e12
        iss = ISSUED_PER_ENTRY[dom] * d * e / launches / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": traffic,
                "avg_ms": round(tot / cnt, 4), "launches_per_step": launches,
                "own_flop_per_entry_per_dim": OWN_PER_ENTRY[dom],
                "executed_mfma": {"achieved": round(iss, 3), "frac": round(iss / peak, 4),
                                  "flop_per_entry_per_dim": ISSUED_PER_ENTRY[dom]}}
    else:
        roof = {"kernel": dom, "bound": "mfma", "achieved": None, "peak": peak, "unit": "TFLOP/s",
                "frac": None, "traffic": traffic, "avg_ms": round(tot / cnt, 4)}
    issued_all = sum(ISSUED_PER_ENTRY[n] * d * entries[ENTRY_KIND[n]] for n in OWN_PER_ENTRY if n in kern)

    if worker:
        wl = {"workload": prob.name, "batch": 1, "seq_len": prob.n, "stripe_world": prob.stripe_world,
              "worker": prob.stripe_rank, "worker_rows": int(row_pos.size), "kv_chunks": prob.stripe_world,
              "ring": "fwd per chunk with the merge fused (o_f32=2), delta, bwd per chunk accumulating dQ",
              "one_call": one_call, "ring_graph": graph_rec, "lse_merge": merge_rec}
    else:
        wl = {"workload": prob.name, "batch": 1, "seq_len": prob.n, "segments": len(cu) - 1}
    wl.update({"h_q": Hq, "h_kv": prob.h_kv, "head_dim": d, "block": 64,
               "v_budget": prob.v_budget[0] if len(set(prob.v_budget)) == 1 else list(prob.v_budget),
               "s_budget": prob.s_budget[0] if len(set(prob.s_budget)) == 1 else list(prob.s_budget),
               "estimator": (f"XAttention block selection, block 128, stride 16, threshold {args.threshold}"
                             if xattn else
                             f"MoBA gate, block {args.moba_block}, top-{args.moba_topk}" if moba else
                             "fixed budgets" if topp is None else
                             f"top-p p_v={topp[0]} p_s={topp[1]} (budgets as caps)"),
               "executed_entries": ent, "slash_entries": entries["slash"],
               "vertical_entries": entries["vertical"], "causal_entries": dense,
               "density": round(ent / dense, 5), "phases_ms": {k_: round(v_, 4) for k_, v_ in phases.items()},
               "kernels": per_kernel,
               "issued_mfma_tflops_per_step": round(issued_all / (ms * 1e-3) / 1e12, 2),
               "parallelism": "none"})
    out = {
        "metric": METRIC, "value": round(exec_tf, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": prob.dtype,
        "data": "synthetic",
        "dense_equiv_tflops": round(dense_tf, 3),
        "pct_bf16_peak_executed": round(100 * exec_tf / peak, 3),
        "config": wl,
        "roofline": roof,
        "cpu_baseline": None,
    }
    return out, lists, ent, row_blocks


def workloads_stripe(prob, W, w):
    import workloads
    return workloads.stripe_positions(prob.n, W, w).numpy()


def _stripe(x, W, w):
    import workloads
    return workloads.stripe_rows(x, W, w)


if __name__ == "__main__":
    main()
