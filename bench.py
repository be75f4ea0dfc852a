#!/usr/bin/env python3
"""Benchmark: Vertical-Slash sparse attention (index estimate + forward + backward) on one MI355X.

Workload (default): one Qwen2.5-3B-shaped attention layer at N = 131072, bf16,
16 Q / 2 KV heads, head_dim 128, causal, 64-token blocks, vertical budget 2048
and slash budget 8192 tokens, seeded synthetic Q/K/V/dO with RoPE and 0.1%
outlier keys.  One step = vs_estimate_index + vs_sparse_attn_fwd +
vs_sparse_attn_bwd over inputs already resident in HBM.

Prints one JSON line.  value = executed TFLOP/s = 14 * d * H_q * |M| / t_step
(|M| = valid entries of the estimated index per head; 4d forward + 10d
backward per entry); also dense-equivalent TFLOP/s over the causal area and
the fraction of the bf16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd sparse attn TFLOP/s (executed & dense-equiv), % bf16 MFMA peak, N=128K"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)


# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, each scaled by what the same counter reads for a plain copy of
# known size), keyed by kernel, with a digest of the kernel sources they were
# taken from: the figure is reported only while the sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_qwen2.5-3b-layer-n128k.json")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("source_sha256") != source_digest() or data.get("workload") != workload:
        return None
    ent = data.get("kernels", {}).get(kernel)
    return None if ent is None else int(ent["hbm_bytes_per_launch"])


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


def cpu_baseline(prob, lists, target_s, topp=None):
    """The CPU oracle, as it stands, on a bounded sample of the same workload.

    Sample: the estimator for one Q head (window scoring over all keys) and the
    support-form forward + backward for evenly spaced query blocks of that
    head, until about target_s seconds have passed.  The job time is
    extrapolated: estimator time x heads + (sample time / sample entries) x |M|.
    """
    import numpy as np
    import oracle
    from dynamic_sparse_attention_amd import accounting
    try:
        from threadpoolctl import threadpool_info
        cores = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    h = 0
    g = h * prob.h_kv // prob.h_q
    q = prob.q[0].to(dtype=__import__("torch").float64).numpy()
    k = prob.k[0].to(dtype=__import__("torch").float64).numpy()
    v = prob.v[0].to(dtype=__import__("torch").float64).numpy()
    do = prob.do[0].to(dtype=__import__("torch").float64).numpy()
    n = prob.n
    t0 = time.perf_counter()
    if topp is None:
        oracle.estimate_index(q[:, h:h + 1], k[:, g:g + 1], prob.cu_seqlens, prob.v_budget[:1],
                              prob.s_budget[:1])
    else:
        oracle.estimate_index_topp(q[:, h:h + 1], k[:, g:g + 1], prob.cu_seqlens, prob.v_budget[:1],
                                   prob.s_budget[:1], [topp[0]], [topp[1]])
    t_est = time.perf_counter() - t0
    iv, is_ = np.asarray(lists[h][0]), np.asarray(lists[h][1])
    index = {(0, 0): (iv[iv >= 0], is_[is_ >= 0])}
    nb = n // 64
    order = np.concatenate([np.arange(s, nb, 64) for s in range(64)])  # spread over the sequence
    pos = np.arange(n)
    done, t_fb = [], 0.0
    qh, doh = q[:, h:h + 1], do[:, h:h + 1]
    kg, vg = k[:, g:g + 1], v[:, g:g + 1]
    for blk in order:
        rows = pos[blk * 64:(blk + 1) * 64]
        t1 = time.perf_counter()
        O, L = oracle.attn_fwd_support(qh[rows], kg, vg, rows, pos, prob.cu_seqlens, index)
        D = oracle.bwd_delta(O, doh[rows])
        oracle.attn_bwd_support(qh[rows], kg, vg, doh[rows], L, D, rows, pos, prob.cu_seqlens, index)
        t_fb += time.perf_counter() - t1
        done.append(blk)
        if t_est + t_fb >= target_s:
            break
    ent = int(accounting.executed_area([lists[h]], prob.cu_seqlens, 1,
                                       row_blocks=np.asarray(done))[0])
    total_ent = int(sum(accounting.executed_area(lists, prob.cu_seqlens, prob.h_q)))
    job_s = t_est * prob.h_q + t_fb / max(ent, 1) * total_ent
    flops = 14 * prob.d * total_ent
    return {"value": round(flops / job_s / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle: estimator for 1 of {prob.h_q} heads ({t_est:.2f} s) and "
                       f"support-form fwd+bwd of {len(done)} of {nb} query blocks of that head "
                       f"({ent} entries, {t_fb:.2f} s); job time extrapolated to {job_s:.1f} s")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="workload id (3 = N=131072)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--topp", default=None, metavar="P_V,P_S",
                    help="estimate with top-p budgets (vs_estimate_index_topp) at these mass "
                         "fractions, the workload's budgets as caps")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dynamic_sparse_attention_amd as vs
    from dynamic_sparse_attention_amd import accounting
    import workloads

    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(dev)
        return
    t0 = time.time()
    prob = workloads.make_problem(args.workload)
    log(f"inputs {prob.name}: n={prob.n} in {time.time() - t0:.1f} s")
    cu = prob.cu_seqlens
    q, k, v, do = (t.to(dev) for t in (prob.q, prob.k, prob.v, prob.do))
    B, N, Hq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    dq = torch.empty((B, N, Hq, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, N, prob.h_kv, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)

    topp = None
    if args.topp:
        topp = tuple(float(x) for x in args.topp.split(","))
        if len(topp) != 2:
            raise SystemExit("--topp takes P_V,P_S")

    def estimate():
        if topp is None:
            return vs.estimate_index(q, k, prob.v_budget, prob.s_budget, cu)
        return vs.estimate_index_topp(q, k, prob.v_budget, prob.s_budget, [topp[0]] * Hq,
                                      [topp[1]] * Hq, cu)[0]

    idx = estimate()
    lists = [(a.numpy(), b.numpy()) for a, b in idx.lists()]
    ent_heads = accounting.executed_area(lists, cu, Hq)
    ent = int(ent_heads.sum())
    dense = accounting.dense_causal_area(cu) * Hq
    log(f"index: executed entries {ent} of {dense} causal ({ent / dense:.4f})")

    stream = torch.cuda.current_stream(dev)

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lib = vs._abi.lib()
    lib.vs_trace_enable(1)
    trace_read(vs)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
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
    phases = {"estimate": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
              "fwd": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
              "bwd": float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))}
    exec_tf = 14 * d * ent / (ms * 1e-3) / 1e12
    dense_tf = 14 * d * dense / (ms * 1e-3) / 1e12
    log(f"step {ms:.3f} ms; phases {phases}")
    for name, (cnt, tot) in sorted(kern.items(), key=lambda x: -x[1][1]):
        log(f"  kernel {name}: {cnt} launches, avg {tot / cnt:.4f} ms, {tot / args.steps:.4f} ms per step")

    # Roofline of the dominant kernel (largest time per step): algorithmic
    # matrix-core FLOPs per step, divided over the kernel's launches per step,
    # against its average launch duration.
    split = accounting.executed_split(lists, cu, Hq)
    alg = {"vs_fwd": 4 * d * ent,
           "vs_bwd_dq": 6 * d * ent,
           "vs_bwd_dkdv_slash": 8 * d * int(split["slash"].sum()),
           "vs_bwd_dkdv_cols": 8 * d * int(split["vertical"].sum())}
    dom = max(kern.items(), key=lambda x: x[1][1])[0]
    cnt, tot = kern[dom]
    avg_s = tot / cnt * 1e-3
    launches = cnt / args.steps
    traffic = measured_traffic(dom, prob.name)
    if dom in alg:
        ach = alg[dom] / launches / avg_s / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "avg_ms": round(tot / cnt, 4), "launches_per_step": launches}
    else:
        roof = {"kernel": dom, "bound": "mfma", "achieved": None, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": None, "traffic": traffic, "avg_ms": round(tot / cnt, 4)}
    per_kernel = {n: round(t / c, 4) for n, (c, t) in kern.items()}
    per_step = {n: round(t / args.steps, 4) for n, (c, t) in kern.items()}

    cpu = None
    if not args.no_cpu_baseline:
        t1 = time.time()
        cpu = cpu_baseline(prob, lists, args.cpu_seconds, topp)
        log(f"cpu baseline {cpu['value']} TFLOP/s in {time.time() - t1:.1f} s")

    out = {
        "metric": METRIC, "value": round(exec_tf, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "dense_equiv_tflops": round(dense_tf, 3),
        "pct_bf16_peak_executed": round(100 * exec_tf / PEAK_BF16_TFLOPS, 3),
        "config": {"workload": prob.name, "batch": 1, "seq_len": N, "h_q": Hq, "h_kv": prob.h_kv,
                   "head_dim": d, "block": 64, "v_budget": prob.v_budget[0],
                   "s_budget": prob.s_budget[0],
                   "estimator": "fixed budgets" if topp is None else
                   f"top-p p_v={topp[0]} p_s={topp[1]} (budgets as caps)",
                   "executed_entries": ent, "causal_entries": dense,
                   "density": round(ent / dense, 5), "phases_ms": {k_: round(v_, 4) for k_, v_ in phases.items()},
                   "kernels_avg_ms": per_kernel, "kernels_ms_per_step": per_step,
                   "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
