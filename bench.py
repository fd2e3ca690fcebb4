"""Benchmark: one draft -> schedule -> verify step per iteration on one MI355X.

Workload (default ``full_step``): B = 512 requests, K = 7 draft positions,
V = 151936, Markov rank r = 256, bf16 logits and factors, temperature 1,
early-stopping scheduler on a staircase SPS table (see
draft_verify_schedule_amd/workloads.py for the value laws).  A step is the
whole hot path: dspark_markov_draft (K sequential positions), dspark_schedule
and dspark_verify over the flattened batch the schedule chose.  Inputs are
resident in HBM before timing starts.  The target model's pass is out of
scope: its output rows (the flat [N, V] batch) are gathered once before the
timed loop; the confidences are inputs, so the schedule, and hence the flat
layout, is the same every step (checked after the timed loop).

Prints one JSON line: verified draft tokens/s (sum of l_r per step / step
time), the dominant kernel's roofline (algorithmic bytes per launch / mean
launch time from HIP events on the library's stream), and the CPU oracle
timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft tokens/sec/GPU at V=151936, K=7; HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_full_step.json")
KERNEL_SOURCES = ["draft.hip", "bias_tile.hpp", "common.hpp", "verify.hip"]


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "draft_verify_schedule_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="full_step")
    ap.add_argument("--mode", type=int, default=0, help="0 early stop, 1 global, 2 top-K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=512, help="requests in the oracle's timed sample")
    ap.add_argument("--cpu-steps", type=int, default=2, help="oracle steps in the timed sample")
    ap.add_argument("--no-next-rows", action="store_true", help="skip timing the rows beyond the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the hot path has no multi-GPU mode "
              "(requests shard across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__._ensure_built()
    import draft_verify_schedule_amd as ds
    from draft_verify_schedule_amd import workloads as wl

    dev = "cuda:0"
    torch.cuda.set_device(0)
    print("generating workload %s" % args.workload, file=sys.stderr, flush=True)
    w = wl.make(args.workload, device=dev)
    B, K, V, r = w.B, w.K, w.V, w.r
    T = w.temperature
    U, W1, W2, x0, c, sps = w.U, w.W1, w.W2, w.x0, w.c, w.sps

    # outputs and workspaces allocated once
    x = torch.empty((B, K), dtype=torch.int32, device=dev)
    q = torch.empty((B, K), dtype=torch.float32, device=dev)
    lse = torch.empty((B, K), dtype=torch.float32, device=dev)
    sch = {"a": torch.empty((B, K), dtype=torch.float32, device=dev),
           "ell": torch.empty(B, dtype=torch.int32, device=dev),
           "cu_seqlens": torch.empty(B + 1, dtype=torch.int32, device=dev),
           "n_admitted": torch.empty(1, dtype=torch.int32, device=dev),
           "theta": torch.empty(1, dtype=torch.float64, device=dev)}
    ws_d = torch.empty(max(256, ds.dspark_markov_draft_workspace_bytes(B, K, V, r)), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(max(256, ds.dspark_schedule_workspace_bytes(B, K)), dtype=torch.uint8, device=dev)
    ds.dspark_schedule(c, sps, args.mode, 0, out=sch, workspace=ws_s)
    cu0 = sch["cu_seqlens"].clone()
    N = int(cu0[-1].item())
    verified = int(sch["ell"].sum().item())
    P = wl.flat_target_rows(w.t, cu0)             # the target pass's output, gathered once
    ws_v = torch.empty(max(256, ds.dspark_verify_workspace_bytes(B, K, V, r, N)), dtype=torch.uint8, device=dev)
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step(s):
        ds.dspark_markov_draft(U, W1, W2, x0, T, w.rng_seed, s, out=(x, q, lse), workspace=ws_d)
        ds.dspark_schedule(c, sps, args.mode, 0, out=sch, workspace=ws_s)
        ds.dspark_verify(P, sch["cu_seqlens"], U, W1, W2, x0, x, q, lse, T, w.rng_seed, s, out=(n_acc, tok),
                         workspace=ws_v)

    print("warmup %d steps (N=%d verify rows, %d verified drafts/step)" % (args.warmup, N, verified),
          file=sys.stderr, flush=True)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    accepted = 0
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(args.warmup + s)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    accepted = int(n_acc.sum().item())
    assert torch.equal(sch["cu_seqlens"], cu0), "flat layout changed between steps"
    print("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step), file=sys.stderr, flush=True)

    # per-kernel mean launch time from HIP events on the library's stream
    prof_steps = min(args.steps, 10)
    ds.dspark_profiler_reset()
    ds.dspark_profiler_enable(True)
    for s in range(prof_steps):
        step(1000 + s)
    torch.cuda.synchronize()
    ds.dspark_profiler_enable(False)
    kt = ds.dspark_profiler_read()
    kernels = {k: {"launches": n, "mean_us": 1000.0 * ms / n} for k, (n, ms) in kt.items() if n}

    if args.calibrate_copy:
        a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # roofline of the dominant kernel: the fused bias-GEMM + softmax-partials pass
    dom = "draft_partials"
    per_launch_bytes = B * V * U.element_size() + V * r * 2 + B * r * 2
    mean_us = kernels[dom]["mean_us"]
    achieved = per_launch_bytes / (mean_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash() and tr.get("kernel") == dom:
            traffic = tr.get("bytes_per_launch")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
            "algorithmic_bytes_per_launch": per_launch_bytes, "mean_launch_us": round(mean_us, 2)}
    if "verify_rowstats" in kernels:
        vb = N * V * P.element_size()
        vus = kernels["verify_rowstats"]["mean_us"]
        roof["verify_rowstats"] = {"bytes": vb, "mean_us": round(vus, 2),
                                   "GB/s": round(vb / (vus * 1e-6) / 1e9, 1),
                                   "frac": round(vb / (vus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    next_rows = {} if args.no_next_rows else measure_next_rows(ds, w, x, lse, sch, ws_s, P, args)

    value = verified * args.steps / (total_ms * 1e-3)
    out = {"metric": METRIC, "value": round(value, 1), "unit": "verified draft tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": args.workload, "B": B, "K": K, "V": V, "r": r, "temperature": T,
                      "sched_mode": ["early_stop", "global", "topk"][args.mode], "verify_rows": N,
                      "verified_drafts_per_step": verified, "accepted_drafts_last_step": accepted,
                      "emitted_tokens_last_step": accepted + B},
           "roofline": roof, "kernels_us": {k: round(v["mean_us"], 2) for k, v in kernels.items()}}
    if next_rows:
        out["next_rows"] = next_rows

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args, verified, B)
    print(json.dumps(out), flush=True)


def measure_next_rows(ds, w, x, lse, sch, ws_s, P, args):
    """The rows built beyond the step, timed on the same workload with HIP
    events (library stream = torch's current stream), outside the step:
    the acceptance label of every drafted position, the asynchronous
    capacity schedule, the confidence head and STS, and the RNN head's draft
    and verification."""
    import torch
    B, K, V, r = w.B, w.K, w.V, w.r
    Pk = w.t[:, :K].contiguous()           # target rows judging positions 1..K
    c_lab = torch.empty((B, K), dtype=torch.float32, device=Pk.device)
    ws_l = torch.empty(max(256, ds.dspark_acceptance_label_workspace_bytes(B, K, V, r)), dtype=torch.uint8,
                       device=Pk.device)

    def timed(fn, n=5):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / n

    us_label = timed(lambda: ds.dspark_acceptance_label(Pk, w.U, w.W1, w.W2, w.x0, x, lse, w.temperature,
                                                        out=c_lab, workspace=ws_l))
    # algorithmic bytes: every target and draft row once, plus W2 once
    lab_bytes = 2 * B * K * V * Pk.element_size() + (V * r * 2 if r else 0)
    old = ds.dspark_schedule(w.c, w.sps, 1, 0, workspace=ws_s)    # capacity from the no-break search
    async_out = {k: torch.empty_like(v) for k, v in sch.items()}
    us_async = timed(lambda: ds.dspark_schedule_async(w.c, w.sps, old["n_admitted"], out=async_out,
                                                      workspace=ws_s))
    # confidence head on the drafted block: synthetic hidden states of a
    # 4096-wide backbone (bf16), head weights ~ N(0, 0.02^2)
    g = torch.Generator(device=Pk.device)
    g.manual_seed(2024)
    d = 4096
    H = (torch.randn((B, K, d), generator=g, device=Pk.device)).to(torch.bfloat16)
    w_h = torch.randn(d, generator=g, device=Pk.device) * 0.02
    w_e = torch.randn(max(r, 1), generator=g, device=Pk.device)[:r] * 0.02
    T_sts = torch.ones(K, device=Pk.device)
    c_head = torch.empty((B, K), dtype=torch.float32, device=Pk.device)
    us_head = timed(lambda: ds.dspark_confidence_head(H, w_h, w_e if r else None, 0.5, w.W1 if r else None, w.x0, x,
                                                      V, sts_temperature=T_sts, out=c_head))
    head_bytes = B * K * d * 2 + B * K * r * 2
    # STS over a held-out set of 100000 blocks, 121 temperatures, 15 bins
    Nh = 100000
    logits = torch.randn((Nh, K), generator=g, device=Pk.device) * 2.0 + 1.5
    surv = (torch.rand((Nh, K), generator=g, device=Pk.device) < 0.8).to(torch.uint8).cumprod(dim=1).to(torch.uint8)
    grid = torch.exp(torch.linspace(-1.386, 1.386, 121, device=Pk.device))
    us_sts = timed(lambda: ds.dspark_sts_fit(logits, surv, grid, 15), n=2)
    rnn = measure_rnn_head(ds, w, P, sch, timed, d) if (r >= 32 and r % 32 == 0) else None
    out = {"confidence_head": {"us": round(us_head, 1), "d": d, "bytes": head_bytes,
                                "GB/s": round(head_bytes / (us_head * 1e-6) / 1e9, 1)},
            "sts_fit": {"us": round(us_sts, 1), "held_out": Nh, "grid": 121, "bins": 15},
            "acceptance_label": {"us": round(us_label, 1), "algorithmic_bytes": lab_bytes,
                                 "GB/s": round(lab_bytes / (us_label * 1e-6) / 1e9, 1),
                                 "frac_hbm": round(lab_bytes / (us_label * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "mean_label": round(float(c_lab.mean()), 4)},
            "schedule_async": {"us": round(us_async, 1), "capacity": int(old["n_admitted"].item())}}
    if rnn:
        out["rnn_head"] = rnn
    return out


def measure_rnn_head(ds, w, P, sch, timed, d):
    """The RNN head on the same workload (hidden states of a d-wide backbone):
    one whole draft of the block per call (W2 to fp16, the hidden-state
    projection, then per position the gated update, the fused bias + softmax
    partials pass and the sampling), and verification of its drafts on the
    step's schedule."""
    import torch
    from draft_verify_schedule_amd import workloads
    B, K, V, r = w.B, w.K, w.V, w.r
    dev = w.U.device
    H, Wr = workloads.rnn_head(B, K, r, d, 1005, device=dev)
    out = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B, K, r), dtype=torch.float32, device=dev))
    ws = torch.empty(ds.dspark_rnn_draft_workspace_bytes(B, K, V, r, d), dtype=torch.uint8, device=dev)
    draft = lambda: ds.dspark_rnn_draft(w.U, H, Wr, w.W1, w.W2, w.x0, w.temperature, w.rng_seed, 0, out=out,
                                        workspace=ws)
    us_draft = timed(draft)
    ds.dspark_profiler_reset()
    ds.dspark_profiler_enable(True)
    for _ in range(3):
        draft()
    torch.cuda.synchronize()
    ds.dspark_profiler_enable(False)
    kern = {k: {"launches": n // 3, "mean_us": round(1000.0 * ms / n, 2)} for k, (n, ms) in
            ds.dspark_profiler_read().items() if n}
    x, q, lse, O = out
    N = P.shape[0]
    ws_v = torch.empty(ds.dspark_rnn_verify_workspace_bytes(B, K, V, r, N), dtype=torch.uint8, device=dev)
    vout = (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
    us_verify = timed(lambda: ds.dspark_rnn_verify(P, sch["cu_seqlens"], w.U, O, w.W2, w.x0, x, q, lse,
                                                   w.temperature, w.rng_seed, 0, out=vout, workspace=ws_v))
    # the fused pass of one position: U_k, the fp16 W2 and the output parts;
    # its MFMA work is the bias with o split in two (2 x 2 B r V flops)
    part_bytes = B * V * w.U.element_size() + V * r * 2 + B * r * 4
    part_us = kern.get("draft_partials", {}).get("mean_us")
    res = {"d": d, "draft_us": round(us_draft, 1), "drafted_tokens_per_s": round(B * K / (us_draft * 1e-6), 1),
           "verify_us": round(us_verify, 1), "verify_rows": N, "kernels": kern}
    if part_us:
        res["draft_partials"] = {"algorithmic_bytes": part_bytes, "GB/s": round(part_bytes / (part_us * 1e-6) / 1e9, 1),
                                 "frac_hbm": round(part_bytes / (part_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "mfma_TFLOP/s": round(4.0 * B * r * V / (part_us * 1e-6) / 1e12, 1)}
    hp = kern.get("rnn_hproj", {}).get("mean_us")
    if hp:
        res["rnn_hproj_TFLOP/s"] = round(2.0 * B * K * d * 3 * r / (hp * 1e-6) / 1e12, 1)
    return res


def cpu_baseline(w, args, verified, B):
    """The oracle (float64 NumPy, as it stands) on a bounded sample of the same
    workload: `cpu_steps` whole steps (schedule of all requests, draft + verify
    of `cpu_sample` requests, scaled linearly to all B when fewer), reported in
    the same unit as the GPU figure."""
    import numpy as np
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    n = min(args.cpu_sample, B)
    sample = np.linspace(0, B - 1, n).round().astype(np.int64)
    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    Us = f64(w.U[torch.as_tensor(sample, device=w.U.device)])
    W1 = f64(w.W1) if w.W1 is not None else None
    W2 = f64(w.W2).T.copy() if w.W2 is not None else None
    x0 = w.x0.cpu().numpy()[sample]
    c = w.c.cpu().numpy()
    sps = w.sps.cpu().numpy()
    tf = w.t[torch.as_tensor(sample, device=w.t.device)].cpu()
    print("cpu baseline: oracle, %d step(s) on %d of %d requests" % (args.cpu_steps, n, B), file=sys.stderr, flush=True)
    t_sched = t_req = 0.0
    for s in range(args.cpu_steps):
        t0 = time.perf_counter()
        sch = oracle.schedule_ref(c, sps, args.mode)
        t1 = time.perf_counter()
        d = oracle.draft_ref(Us, W1, W2, x0, w.temperature, w.rng_seed, s, request_ids=sample)
        t2 = time.perf_counter()
        ell = sch["ell"][sample]
        cu = np.concatenate([[0], np.cumsum(ell + 1)])
        P = torch.cat([tf[i, :ell[i] + 1] for i in range(n)]).to(torch.float64).numpy()
        t3 = time.perf_counter()
        oracle.verify_ref(P, cu, Us, W1, W2, x0, d["x"], w.temperature, w.rng_seed, s, request_ids=sample)
        t4 = time.perf_counter()
        t_sched += t1 - t0
        t_req += (t2 - t1) + (t4 - t3)
    step_s = (t_sched + t_req * B / n) / args.cpu_steps
    scaled = "" if n == B else ", scaled linearly to %d" % B
    return {"value": round(verified / step_s, 2), "unit": "verified draft tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d oracle step(s) of the same workload: schedule of all %d requests, draft + verify of %d%s; "
                      "%.1f s of oracle time, %.2f s per step" % (args.cpu_steps, B, n, scaled, t_sched + t_req, step_s)}


if __name__ == "__main__":
    main()
