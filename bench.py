"""Benchmark: MoE expert-parallel dispatch + combine on one MI355X.

One step = one ep_dispatch + one ep_combine over all W virtual ranks of the
workload (default: 8 ranks x 4096 tokens, hidden 7168 bf16, 256 experts,
top-8, FP32 routing weights dispatched and summed back; identity experts, so
the combine reads the dispatch's output rows in place). Inputs are generated
on the host from the seeded workload and are resident in HBM before the
timed region. Before timing, one call is checked bit for bit against the CPU
oracle, which is also timed on the host as the CPU baseline.

Prints one JSON line. `value` is payload HBM throughput (GB/s): algorithmic
payload bytes of one call (dispatch reads N rows and writes R rows, combine
reads R rows and writes N rows) over the time of one call.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "dispatch+combine µs/call and payload HBM GB/s (% of peak), EP8 H=7168 k=8"
KERNEL_SOURCES = [os.path.join(ROOT, "combine_route_amd", "csrc", f)
                  for f in ("ep_kernels.hip", "ep_kernels.h", "ep_plan.cpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """Per-launch HBM bytes measured by rocprofv3 counters, from the summary
    under profiles/, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_ceiling(torch, mib, steps, warmup):
    """Plain copy of mib MiB between two device buffers: reads and writes
    mib MiB each per launch."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_mib": mib, "bytes_moved_per_launch": 2 * n, "ms_per_copy": round(ms, 4),
                      "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (CPU baseline and the bit-exact check)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, time a plain device-to-device copy of MIB "
                         "MiB (the box's copy ceiling, and the known-size kernel that scales "
                         "rocprofv3's byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build runs all virtual "
              "expert-parallel ranks on one GPU; only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_ceiling(torch, args.copy_calibration, args.steps, args.warmup)
        return

    import combine_route_amd as cra
    import workloads

    wl = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
    if wl.expert != "identity" or wl.dispatch_dtype != wl.combine_dtype:
        print("bench.py times identity experts (combine reads the dispatched rows); "
              f"{wl.name} needs a different expert", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    inp = workloads.make_inputs(wl)
    print(f"[bench] inputs of {wl.name} generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    cfg = cra.make_config(W, H, M, wl.experts_per_rank, k, wl.dispatch_dtype, wl.combine_dtype,
                          scale_dim=wl.scale_dim, scale_type_size=4)
    op = cra.EpDispatchCombineOp(cfg, device=dev)
    x = inp["x"].to(dev)
    idx = inp["idx"].to(dev)
    w = inp["w"].to(dev)
    sc = None if inp["scales"] is None else inp["scales"].to(dev)
    ntok = inp["ntok"]
    stream = torch.cuda.current_stream()

    def step():
        op.dispatch(ntok, x, idx, w, sc, stream=stream)
        op.combine(op.out_x, op.out_weights, stream=stream)

    # -- correctness first, and the CPU baseline -----------------------------
    step()
    torch.cuda.synchronize()
    recv = op.recv_num_token.cpu().numpy()
    R = int(recv.sum())
    N = int(sum(ntok))
    check = "skipped"
    cpu_baseline = None
    row = H * (1 if wl.dispatch_dtype == "fp8" else 2)
    crow = H * 2
    sb = wl.scale_dim * 4
    P = min(W, k)
    payload_bytes = N * (row + sb) + R * (row + sb) + R * crow + N * crow
    if not args.no_cpu_baseline:
        import oracle

        xb = inp["x"].view(torch.uint8).numpy()
        scn = None if inp["scales"] is None else inp["scales"].numpy()
        t = time.perf_counter()
        ref = oracle.dispatch(W, M, k, wl.experts_per_rank, ntok, xb, inp["idx"].numpy(),
                              inp["w"].numpy(), scn)
        y = ref["out_x"].view(np.uint16).reshape(W, W * M, H)
        ro, rw = oracle.combine(W, M, k, H, oracle.BF16 if wl.combine_dtype == "bf16"
                                else oracle.FP16, ntok, ref["fwd"], y, ref["out_w"])
        cpu_s = time.perf_counter() - t
        cpu_baseline = {"value": round(payload_bytes / cpu_s / 1e9, 3), "unit": "GB/s",
                        "cores": 1, "kind": "oracle",
                        "sample": f"the whole {wl.name} workload, one dispatch+combine call, "
                                  f"single-threaded C oracle, {cpu_s:.2f} s"}
        print(f"[bench] oracle call took {cpu_s:.2f}s", file=sys.stderr, flush=True)
        ok = np.array_equal(recv, ref["recv"])
        for d in range(W):
            Rd = int(recv[d])
            ok = ok and np.array_equal(op.src_token_pos(d)[:Rd].cpu().numpy(),
                                       ref["src_pos"][d, :Rd])
            ok = ok and np.array_equal(op.out_x[d, :Rd].view(torch.uint8).cpu().numpy(),
                                       ref["out_x"][d, :Rd])
            ok = ok and np.array_equal(op.out_indices[d, :Rd].cpu().numpy(), ref["out_idx"][d, :Rd])
            ok = ok and np.array_equal(op.out_weights[d, :Rd].cpu().numpy().view(np.uint32),
                                       ref["out_w"][d, :Rd].view(np.uint32))
        g = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
        gw = op.combine_weights.cpu().numpy().view(np.uint32)
        for r in range(W):
            T = ntok[r]
            ok = ok and np.array_equal(g[r, :T], ro[r, :T])
            ok = ok and np.array_equal(gw[r, :T], rw[r, :T].view(np.uint32))
        del ref, y, ro, rw
        if not ok:
            print("bench.py: GPU results differ from the oracle; not timing", file=sys.stderr)
            sys.exit(1)
        check = "bit-exact vs oracle"

    # -- timed region ---------------------------------------------------------
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cra.ep_plan_set_timing(op.plan, True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    kern = {}
    for name, kid in (("route", cra.EP_KERNEL_ROUTE), ("scan", cra.EP_KERNEL_SCAN),
                      ("copy", cra.EP_KERNEL_COPY), ("combine", cra.EP_KERNEL_COMBINE)):
        c, ms = cra.ep_plan_kernel_time(op.plan, kid)
        kern[name] = ms / max(c, 1)
    cra.ep_plan_set_timing(op.plan, False)

    # algorithmic bytes per launch of the two large kernels
    has_w = 1
    copy_bytes = (N * (row + sb + 4 * k * (1 + has_w)) + R * (row + sb + 4 * k * (1 + has_w) + 4)
                  + N * P * 4)
    combine_bytes = R * crow + N * crow + N * P * 4 + has_w * (R * 4 * k + N * 4 * k)
    dom = "copy" if kern["copy"] >= kern["combine"] else "combine"
    dom_bytes = copy_bytes if dom == "copy" else combine_bytes
    achieved = dom_bytes / (kern[dom] * 1e-3) / 1e9
    kernel_name = {"copy": "ep_copy_kernel", "combine": "ep_combine_kernel"}[dom]
    traffic = read_traffic(wl.name, kernel_name)

    value = payload_bytes / (ms_per_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dispatch_dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "world_size": W, "tokens_per_rank": ntok[0] if
                   len(set(ntok)) == 1 else ntok, "hidden": H, "topk": k,
                   "experts": wl.num_experts, "dispatch_dtype": wl.dispatch_dtype,
                   "combine_dtype": wl.combine_dtype, "weights": True,
                   "launch": cra.ep_plan_get_launch(op.plan, ntok)},
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "payload_bytes_per_call": payload_bytes,
        "received_rows": R,
        "kernel_us": {k_: round(v * 1e3, 2) for k_, v in kern.items()},
        "check": check,
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": dom_bytes},
        "cpu_baseline": cpu_baseline,
    }
    op.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
