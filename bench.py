"""Benchmark: MoE expert-parallel dispatch + combine on one MI355X.

One step = one ep_dispatch + one ep_combine over all W virtual ranks of the
workload (default: 8 ranks x 4096 tokens, hidden 7168 bf16, 256 experts,
top-8, FP32 routing weights dispatched and summed back). With identity
experts the combine reads the dispatch's output rows in place; otherwise
the expert output is a seeded random bf16/fp16 buffer, written before the
timed region. Inputs are resident in HBM before the timed region. Before
timing, one call is checked bit for bit against the CPU oracle, which is
also timed on the host as the CPU baseline.

Prints one JSON line. `value` is payload HBM throughput in GB/s: the
algorithmic payload bytes of one call (dispatch reads N rows and writes R
rows, combine reads R rows and writes N rows; R = rows received) over the
time of one call.

Other modes (measurement tooling, no JSON line of the workload):
  --copy-calibration MIB   time a plain device-to-device copy of MIB MiB
  --summarize-stats CSV OUT.md CMD...          rocprofv3 --stats table
  --summarize-counters FETCH WRITE CAL_FETCH CAL_WRITE CAL_MIB WORKLOAD
                           per-launch HBM bytes of the two large kernels
"""
import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
METRIC = "dispatch+combine µs/call and payload HBM GB/s (% of peak), EP8 H=7168 k=8"
# the path's device code and the argument structs it is compiled against; a
# profile summary taken on other sources is not used (launch geometry, set by
# the host code, is in each line's "launch" field)
KERNEL_SOURCES = [os.path.join(ROOT, "combine_route_amd", "csrc", f)
                  for f in ("ep_kernels.hip", "ep_expert.hip", "ep_wire.hip", "ep_kernels.h",
                            "ep_device.h", "ep_standard.hip")]
KERNELS = {"copy": "ep_copy_kernel", "combine": "ep_combine_kernel"}
EXPERT_KERNELS = {"copy": "ex_copy_kernel", "combine": "ex_combine_kernel"}
STANDARD_KERNELS = {"copy": "sx_copy_kernel", "combine": "sx_combine_kernel"}
# counter summaries: label -> pattern over the demangled kernel name; the
# copy kernel's last template argument says whether it casts to E4M3, and
# the wire kernels name their wire in the template argument after the
# row group and units a lane (1 = FP8 block-128, 2 = MXFP4)
COUNTER_KERNELS = {
    "ep_copy_kernel": r"ep_copy_kernel<[^>]*, false>",
    "ep_combine_kernel": r"ep_combine_kernel<",
    "ex_copy_kernel": r"ex_copy_kernel<",
    "ex_combine_kernel": r"ex_combine_kernel<",
    "sx_copy_kernel": r"sx_copy_kernel<[^>]*, false>",
    "sx_copy_kernel_cast": r"sx_copy_kernel<[^>]*, true>",
    "sx_combine_kernel": r"sx_combine_kernel<[^>]*, 0>",
    "sx_combine_kernel_fp8_block128": r"sx_combine_kernel<[^>]*, 1>",
    "sx_combine_kernel_mxfp4": r"sx_combine_kernel<[^>]*, 2>",
    "ep_copy_kernel_cast": r"ep_copy_kernel<[^>]*, true>",
    # the quantizer runs on the W*W*M receive rows and on the W*Er*cap packed
    # rows, one instance for both: the smaller grid is the receive rows
    "ep_quantize_kernel_fp8_block128": (r"ep_quantize_kernel<1,", "min"),
    "ep_quantize_kernel_mxfp4": (r"ep_quantize_kernel<2,", "min"),
    "ep_quantize_kernel_packed_fp8_block128": (r"ep_quantize_kernel<1,", "max"),
    "ep_quantize_kernel_packed_mxfp4": (r"ep_quantize_kernel<2,", "max"),
    "ep_combine_wire_kernel_fp8_block128": r"ep_combine_wire_kernel<\d+, \d+, 1,",
    "ep_combine_wire_kernel_mxfp4": r"ep_combine_wire_kernel<\d+, \d+, 2,",
}


# the bench arguments of the counter runs that profiles/*_counters.txt record
COUNTER_RUN_ARGS = "--no-cpu-baseline --steps 3 --warmup 1 --no-small --rounds 0"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")


def read_traffic(workload: str, kernel: str):
    """Per-launch HBM bytes measured by rocprofv3 counters, from the summary
    under profiles/, if it was taken on the current kernel sources."""
    path = counters_path(kernel, workload)
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


def algorithmic_bytes(wl, ntok, recv_total):
    """Bytes one call must move (each byte read or written once)."""
    N, R = int(sum(ntok)), int(recv_total)
    k, P = wl.topk, min(wl.world_size, wl.topk)
    row = wl.hidden * (1 if wl.dispatch_dtype == "fp8" else 2)
    crow = wl.hidden * 2
    sb = wl.scale_dim * 4
    payload = N * (row + sb) + R * (row + sb) + R * crow + N * crow
    # dispatch copy: payload, scale, id and weight rows of N tokens read; of R
    # rows written, plus src_pos per row and the forward map per token
    copy = N * (row + sb + 8 * k) + R * (row + sb + 8 * k + 4) + N * P * 4
    # combine: R expert-output rows and their weights read, N rows and weight
    # rows written, forward map read
    combine = R * (crow + 4 * k) + N * (crow + 4 * k) + N * P * 4
    return payload, {"copy": copy, "combine": combine}


def expert_capacity(wl, ntok):
    """Rows kept per local expert in the expert-major measurement: twice the
    mean rows an expert receives under uniform routing (N * k / E), rounded up
    to 64, at most W * M. Rows past it would be dropped and are reported."""
    N = int(sum(ntok))
    mean = -(-N * wl.topk // wl.num_experts)
    return max(1, min(wl.world_size * wl.max_tokens, -(-2 * mean // 64) * 64))


def expert_bytes(wl, recv_total, pairs):
    """Bytes the expert-major copy and its inverse must move, each read or
    written once: R received rows, `pairs` kept (row, local expert) pairs."""
    R = int(recv_total)
    k, Pe = wl.topk, min(wl.topk, wl.experts_per_rank)
    row = wl.hidden * (1 if wl.dispatch_dtype == "fp8" else 2)
    crow = wl.hidden * 2
    sb = wl.scale_dim * 4
    # copy: each received row's payload, scale row, ids, weights and source
    # read once; each kept pair's payload and scale row and source info
    # written; the inverse's map and weights written for every row
    copy = R * (row + sb + 8 * k + 4) + pairs * (row + sb + 4) + R * Pe * 8
    # inverse: each kept pair's output read, each received row written, map
    # and weights read
    combine = pairs * crow + R * crow + R * Pe * 8
    return {"copy": copy, "combine": combine}


def measure_expert_major(args, cra, torch, np, wl, op, inp, stream):
    """The expert-major layout and its inverse (convert_dispatch_output,
    convert_combine_input) on the last dispatch of op: K timed steps of both,
    per-kernel HIP-event durations and their HBM rooflines."""
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    ntok = inp["ntok"]
    cap = expert_capacity(wl, ntok)
    op.expert_capacity = cap
    ex = op._expert_state()
    if wl.dispatch_dtype == wl.combine_dtype:
        py = ex["packed_x"]              # identity experts, in place
        py_kind = "identity, in place"
    else:
        g = torch.Generator(device="cuda").manual_seed(7)
        py = torch.randn((W, Er, cap, H), generator=g, device="cuda").to(
            ex["y"].dtype)
        py_kind = "random output"

    # the mixture path: routing weights recorded by the conversion and applied
    # by the inverse
    def step():
        op.convert_dispatch_output(op.out_x, op.out_indices, op.out_scales, op.out_weights,
                                   stream=stream)
        op.convert_combine_input(py, apply_weights=True, stream=stream)

    step()
    torch.cuda.synchronize()
    cnt = ex["packed_count"].cpu().numpy()
    recv = op.recv_num_token.cpu().numpy()
    check = "skipped"
    if not args.no_cpu_baseline:
        # the index outputs against the oracle (payload bytes are covered by
        # the parity tests): first 16 bytes of each row stand in for the row
        import oracle

        x16 = np.ascontiguousarray(inp["x"].view(torch.uint8).numpy()[:, :, :16])
        ref = oracle.dispatch(W, M, k, Er, ntok, x16, inp["idx"].numpy())
        o = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"], ref["out_x"],
                                 ref["out_idx"])
        ok = (np.array_equal(cnt, o["count"]) and np.array_equal(
            ex["packed_layout_range"].cpu().numpy(), o["layout_range"]))
        si = ex["packed_src_info"].cpu().numpy()
        for d in range(W):
            for j in range(Er):
                n = min(int(o["count"][d, j]), cap)
                ok = ok and np.array_equal(si[d, j, :n], o["src_info"][d, j, :n])
        if not ok:
            print("bench.py: expert-major indices differ from the oracle", file=sys.stderr)
            sys.exit(1)
        check = "counts, layout ranges and source info bit-exact vs oracle"
    for _ in range(args.warmup):
        step()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    cra.ep_plan_set_timing(op.plan, True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name, kid in (("count", cra.EP_KERNEL_EXPERT_COUNT), ("scan", cra.EP_KERNEL_EXPERT_SCAN),
                      ("copy", cra.EP_KERNEL_EXPERT_COPY),
                      ("combine", cra.EP_KERNEL_EXPERT_COMBINE)):
        c, t = cra.ep_plan_kernel_time(op.plan, kid)
        kern[name] = t / max(c, 1)
    cra.ep_plan_set_timing(op.plan, False)
    pairs = int(np.minimum(cnt, cap).sum())
    nb = expert_bytes(wl, recv.sum(), pairs)
    roof = {}
    for name, kname in EXPERT_KERNELS.items():
        a = nb[name] / (kern[name] * 1e-3) / 1e9
        roof[name] = {"bound": "hbm", "kernel": kname, "achieved": round(a, 2),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(a / PEAK_HBM_GBS, 4),
                      "traffic": read_traffic(wl.name, kname),
                      "algorithmic_bytes_per_launch": nb[name]}
    return {
        "what": "convert_dispatch_output + convert_combine_input on the dispatch above",
        "expert_capacity": cap, "kept_pairs": pairs,
        "dropped_rows": int(np.maximum(cnt - cap, 0).sum()),
        "expert_output": py_kind,
        "weighted": True,
        "us_per_call": round(ms * 1e3, 2),
        "kernel_us": {k_: round(v * 1e3, 2) for k_, v in kern.items()},
        "check": check,
        "roofline": roof,
    }


def standard_bytes(wl, N, pairs):
    """Bytes the fused dispatch copy and fused combine must move, each read or
    written once: N source tokens, `pairs` kept (token, expert) pairs."""
    k = wl.topk
    row = wl.hidden * (1 if wl.dispatch_dtype == "fp8" else 2)
    crow = wl.hidden * 2
    sb = wl.scale_dim * 4
    # dispatch: each token's payload, scale row and ids read once; each kept
    # pair's payload, scale row and source info written; the slot map written
    copy = N * (row + sb + 4 * k) + pairs * (row + sb + 4) + N * k * 4
    # combine: each kept pair's output read once; each token's row written;
    # its ids, slot map and weights read
    combine = pairs * crow + N * crow + N * k * 12
    return {"copy": copy, "combine": combine}


def measure_standard_moe(args, cra, torch, np, wl, op, inp, stream, x, idx, w, sc):
    """The fused expert-major path (dispatch_standard_moe, combine_standard_moe,
    weighted) against the two steps it replaces (dispatch, convert, weighted
    inverse, combine): both timed, and the fused results checked bit for bit
    against the two-step results on the same inputs."""
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    ntok = inp["ntok"]
    cap = op.expert_capacity
    ex = op._expert_state()
    if wl.dispatch_dtype == wl.combine_dtype:
        py = ex["packed_x"]              # identity experts, in place
    else:
        g = torch.Generator(device="cuda").manual_seed(7)
        py = torch.randn((W, Er, cap, H), generator=g, device="cuda").to(ex["y"].dtype)

    def two_step():
        op.dispatch(ntok, x, idx, w, sc, stream=stream)
        op.convert_dispatch_output(op.out_x, op.out_indices, op.out_scales, op.out_weights,
                                   stream=stream)
        y = op.convert_combine_input(py, apply_weights=True, stream=stream)
        op.combine(y, stream=stream)

    def fused():
        op.dispatch_standard_moe(x, None, sc, idx, num_tokens=ntok, stream=stream)
        op.combine_standard_moe(py, w, idx, stream=stream)

    two_step()
    torch.cuda.synchronize()
    ref = (op.combine_out.view(torch.int16).clone(), ex["packed_count"].clone(),
           ex["packed_layout_range"].clone())
    fused()
    torch.cuda.synchronize()
    ok = torch.equal(ex["packed_count"], ref[1]) and torch.equal(ex["packed_layout_range"], ref[2])
    got = op.combine_out.view(torch.int16)
    for r in range(W):
        ok = ok and torch.equal(got[r, :ntok[r]], ref[0][r, :ntok[r]])
    if not ok:
        print("bench.py: the fused path differs from the two-step path", file=sys.stderr)
        sys.exit(1)
    del ref
    ms_two = _timed(torch, stream, two_step, args.steps, args.warmup)
    ms = _timed(torch, stream, fused, args.steps, args.warmup)
    cra.ep_plan_set_timing(op.plan, True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fused()
    torch.cuda.synchronize()
    kern = {}
    for name, kid in (("count", cra.EP_KERNEL_STANDARD_COUNT),
                      ("scan", cra.EP_KERNEL_STANDARD_SCAN),
                      ("copy", cra.EP_KERNEL_STANDARD_COPY),
                      ("combine", cra.EP_KERNEL_STANDARD_COMBINE)):
        c, t = cra.ep_plan_kernel_time(op.plan, kid)
        kern[name] = t / max(c, 1)
    cra.ep_plan_set_timing(op.plan, False)
    cnt = ex["packed_count"].cpu().numpy()
    pairs = int(np.minimum(cnt, cap).sum())
    nb = standard_bytes(wl, int(sum(ntok)), pairs)
    roof = {name: _roof(nb[name], kern[name], kname, wl.name, kname)
            for name, kname in STANDARD_KERNELS.items()}
    return {
        "what": "dispatch_standard_moe + weighted combine_standard_moe",
        "expert_capacity": cap, "kept_pairs": pairs,
        "us_per_call": round(ms * 1e3, 2),
        "two_step_us_per_call": round(ms_two * 1e3, 2),
        "kernel_us": {k_: round(v * 1e3, 2) for k_, v in kern.items()},
        "check": "bit-exact vs the two-step path (dispatch, convert, weighted inverse, combine)",
        "roofline": roof,
    }


def _timed(torch, stream, fn, steps, warmup):
    """Average ms of fn() over `steps` calls between two HIP events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(steps):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def _kernel_ms(cra, torch, plan, kid, fn, steps):
    cra.ep_plan_set_timing(plan, True)
    torch.cuda.synchronize()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    c, ms = cra.ep_plan_kernel_time(plan, kid)
    cra.ep_plan_set_timing(plan, False)
    return ms / max(c, 1)


def _roof(nbytes, ms, kernel, workload, label):
    a = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(a, 2), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(a / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(workload, label),
            "algorithmic_bytes_per_launch": int(nbytes)}


def measure_quantized_wires(args, cra, torch, np, wl, inp, stream):
    """The quantized wires on the same workload: the dispatch with the
    on-the-fly FP8 cast (bf16 tokens received as E4M3), the send-side
    quantizer, and the combine from FP8 block-128 and MXFP4 rows."""
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    ntok = inp["ntok"]
    N, P = int(sum(ntok)), min(W, k)
    dev = torch.device("cuda:0")
    x = inp["x"].to(dev)
    idx = inp["idx"].to(dev)
    w = inp["w"].to(dev)
    out = {}
    if wl.dispatch_dtype in ("bf16", "fp16"):
        cfg = cra.make_config(W, H, M, Er, k, "fp8", wl.combine_dtype, dispatch_cast=wl.dispatch_dtype)
        op = cra.EpDispatchCombineOp(cfg, device=dev)
        step = lambda: op.dispatch(ntok, x, idx, w, stream=stream)
        ms = _timed(torch, stream, step, args.steps, args.warmup)
        kms = _kernel_ms(cra, torch, op.plan, cra.EP_KERNEL_COPY, step, args.steps)
        R = int(op.recv_num_token.sum().item())
        nb = N * (2 * H + 8 * k) + R * (H + 8 * k + 4) + N * P * 4
        out["dispatch_fp8_direct_cast"] = {
            "us_per_call": round(ms * 1e3, 2), "copy_kernel_us": round(kms * 1e3, 2),
            "received_bytes_saved": R * H,
            "roofline": _roof(nb, kms, "ep_copy_kernel (cast)", wl.name, "ep_copy_kernel_cast")}
        op.close()
        del op
        torch.cuda.empty_cache()
        # the same cast straight into the expert-major layout
        cap = expert_capacity(wl, ntok)
        op = cra.EpDispatchCombineOp(cfg, device=dev, with_weights=False, expert_capacity=cap)
        step = lambda: op.dispatch_standard_moe(x, None, None, idx, num_tokens=ntok,
                                                stream=stream)
        ms = _timed(torch, stream, step, args.steps, args.warmup)
        kms = _kernel_ms(cra, torch, op.plan, cra.EP_KERNEL_STANDARD_COPY, step, args.steps)
        pairs = int(op._expert_state()["packed_count"].clamp(max=cap).sum().item())
        nb = N * (2 * H + 4 * k) + pairs * (H + 4) + N * k * 4
        out["dispatch_standard_fp8_direct_cast"] = {
            "us_per_call": round(ms * 1e3, 2), "copy_kernel_us": round(kms * 1e3, 2),
            "expert_capacity": cap, "kept_pairs": pairs,
            "roofline": _roof(nb, kms, "sx_copy_kernel (cast)", wl.name, "sx_copy_kernel_cast")}
        op.close()
        del op
        torch.cuda.empty_cache()
    for name, wire, row, srow in (("fp8_block128", cra.EP_WIRE_FP8_BLOCK128, H, H // 128 * 4),
                                  ("mxfp4", cra.EP_WIRE_MXFP4, H // 2, H // 32)):
        cfg = cra.make_config(W, H, M, Er, k, wl.dispatch_dtype, wl.combine_dtype,
                              scale_dim=wl.scale_dim, scale_type_size=4, combine_wire=wire)
        op = cra.EpDispatchCombineOp(cfg, device=dev)
        sc = None if inp["scales"] is None else inp["scales"].to(dev)
        op.dispatch(ntok, x, idx, w, sc, stream=stream)
        R = int(op.recv_num_token.sum().item())
        # expert outputs: the received rows themselves (bf16), or seeded rows
        cdt = workloads_dtype(torch, wl.combine_dtype)
        if wl.dispatch_dtype == wl.combine_dtype:
            y = op.out_x
        else:
            g = torch.Generator(device="cuda").manual_seed(11)
            y = torch.randn((W, W * M, H), generator=g, device=dev).to(cdt)
        yq = torch.empty((W, W * M, row), dtype=torch.uint8, device=dev)
        ys = torch.empty((W, W * M, srow), dtype=torch.uint8, device=dev)
        # the send side converts the rows the combine reads: recv_num_token per rank
        qstep = lambda: cra.ep_quantize_rows(y, wire, yq, ys, stream=stream,
                                             counts=op.recv_num_token)
        qms = _timed(torch, stream, qstep, args.steps, args.warmup)
        cstep = lambda: op.combine(yq, op.out_weights, stream=stream, y_scales=ys)
        cms = _timed(torch, stream, cstep, args.steps, args.warmup)
        kms = _kernel_ms(cra, torch, op.plan, cra.EP_KERNEL_COMBINE, cstep, args.steps)
        rows = R
        qb = rows * (2 * H + row + srow)
        cb = R * (row + srow + 4 * k) + N * (2 * H + 4 * k) + N * P * 4
        # the fused path from quantized expert outputs: the packed outputs
        # quantized with the per-expert counts, then the fused combine
        cap = expert_capacity(wl, ntok)
        fop = cra.EpDispatchCombineOp(cfg, device=dev, with_weights=False, expert_capacity=cap)
        fex = fop._expert_state()
        fop.dispatch_standard_moe(x, None, sc, idx, num_tokens=ntok, stream=stream)
        pairs = int(fex["packed_count"].clamp(max=cap).sum().item())
        g = torch.Generator(device="cuda").manual_seed(13)
        py = torch.randn((W * Er, cap, H), generator=g, device=dev).to(cdt)
        pq = torch.empty((W * Er, cap, row), dtype=torch.uint8, device=dev)
        ps = torch.empty((W * Er, cap, srow), dtype=torch.uint8, device=dev)
        pstep = lambda: cra.ep_quantize_rows(py, wire, pq, ps, stream=stream,
                                             counts=fex["packed_count"].view(-1))
        pms = _timed(torch, stream, pstep, args.steps, args.warmup)
        fstep = lambda: fop.combine_standard_moe(pq, w, idx, stream=stream, input_scales=ps)
        fms = _timed(torch, stream, fstep, args.steps, args.warmup)
        fkms = _kernel_ms(cra, torch, fop.plan, cra.EP_KERNEL_STANDARD_COMBINE, fstep, args.steps)
        fb = pairs * (row + srow) + N * (2 * H + 12 * k)
        fused = {"quantize_us_per_call": round(pms * 1e3, 2), "kept_pairs": pairs,
                 "combine_us_per_call": round(fms * 1e3, 2),
                 "combine_kernel_us": round(fkms * 1e3, 2),
                 "roofline_combine": _roof(fb, fkms, "sx_combine_kernel (wire)", wl.name,
                                           "sx_combine_kernel_" + name)}
        fop.close()
        del fop, fex, py, pq, ps
        torch.cuda.empty_cache()
        out["combine_" + name] = {
            "standard_moe": fused,
            "wire_bytes_per_row": row + srow, "bf16_bytes_per_row": 2 * H,
            "combine_us_per_call": round(cms * 1e3, 2), "combine_kernel_us": round(kms * 1e3, 2),
            "quantize_us_per_call": round(qms * 1e3, 2),
            "quantize_rows": rows,
            "roofline_combine": _roof(cb, kms, "ep_combine_wire_kernel", wl.name,
                                      "ep_combine_wire_kernel_" + name),
            "roofline_quantize": _roof(qb, qms, "ep_quantize_kernel", wl.name,
                                       "ep_quantize_kernel_" + name)}
        op.close()
        del op, yq, ys
        torch.cuda.empty_cache()
    return out


def measure_samples(args, torch, stream, dispatch, combine, dispatch_on=None, combine_on=None):
    """The pages' sampling: rounds of per-call samples, each dispatch and
    combine bracketed by its own HIP events on the launch stream, reported as
    p50 and min; a point is flagged when the rounds' p50s spread by more than
    1.2x. The cold variant writes a 512 MiB scratch buffer before every sample,
    so the MALL holds none of the call's data when it starts. With
    dispatch_on / combine_on (the same calls on a given stream), the graph
    variant replays captured graphs instead: the dispatch alone, the combine
    alone, and the pair captured back to back in one graph."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def run(cold):
        rounds = []
        for _ in range(args.rounds):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(args.samples)]
            for e in ev:
                if cold:
                    scratch.fill_(cold)
                e[0].record(stream)
                dispatch()
                e[1].record(stream)
                combine()
                e[2].record(stream)
            torch.cuda.synchronize()
            rounds.append([(e[0].elapsed_time(e[1]) * 1e3, e[1].elapsed_time(e[2]) * 1e3,
                            e[0].elapsed_time(e[2]) * 1e3) for e in ev])
        flat = [t for r in rounds for t in r]

        def stat(i):
            v = sorted(t[i] for t in flat)
            return {"p50": round(v[len(v) // 2], 2), "min": round(v[0], 2)}

        p50s = [sorted(t[2] for t in r)[len(r) // 2] for r in rounds]
        spread = max(p50s) / min(p50s)
        return {"dispatch_us": stat(0), "combine_us": stat(1), "pair_us": stat(2),
                "round_p50_spread": round(spread, 3), "rejected": spread > 1.2}

    for _ in range(10):
        dispatch()
        combine()
    torch.cuda.synchronize()
    out = {"method": f"{args.rounds} rounds x {args.samples} eager calls after 10 warmups; "
                     "each dispatch and combine between HIP events on the launch stream",
           "warm": run(0)}
    out["cold"] = run(1)
    out["cold"]["method"] = "the same, with a 512 MiB device write before every sample"
    if dispatch_on is not None:
        out["graph"] = graph_samples(args, torch, stream, dispatch_on, combine_on)
    del scratch
    torch.cuda.empty_cache()
    return out


def graph_samples(args, torch, stream, dispatch_on, combine_on):
    """Graph-replay samples: three graphs captured on a side stream (the
    dispatch, the combine, and the pair back to back), 10 replays of each as
    warmup, then rounds of samples, each replaying the dispatch graph, the
    combine graph and the pair graph between HIP events."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graphs = []
    for fns in ((dispatch_on,), (combine_on,), (dispatch_on, combine_on)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for f in fns:
                    f(side)
        graphs.append(g)
    torch.cuda.synchronize()
    for _ in range(10):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    rounds = []
    for _ in range(args.rounds):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
              for _ in range(args.samples)]
        for e in ev:
            for i, g in enumerate(graphs):
                e[i].record(stream)
                g.replay()
            e[3].record(stream)
        torch.cuda.synchronize()
        rounds.append([tuple(e[i].elapsed_time(e[i + 1]) * 1e3 for i in range(3)) for e in ev])
    del graphs
    flat = [t for r in rounds for t in r]

    def stat(i):
        v = sorted(t[i] for t in flat)
        return {"p50": round(v[len(v) // 2], 2), "min": round(v[0], 2)}

    p50s = [sorted(t[2] for t in r)[len(r) // 2] for r in rounds]
    spread = max(p50s) / min(p50s)
    return {"method": f"{args.rounds} rounds x {args.samples} samples after 10 replays of each "
                      "graph; a sample replays the dispatch graph, the combine graph and the "
                      "pair (dispatch and combine captured back to back in one graph), each "
                      "between HIP events on the launch stream",
            "dispatch_us": stat(0), "combine_us": stat(1), "pair_us": stat(2),
            "round_p50_spread": round(spread, 3), "rejected": spread > 1.2}


def workloads_dtype(torch, name):
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


def host_cpu():
    """CPU model and logical CPU count of the host that runs the oracle."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "nproc": os.cpu_count()}


def device_copy_rate(torch, mib=1024, steps=5):
    """GB/s of a plain device-to-device copy of mib MiB (bytes read + written
    per second), the machine's own copy rate to set the path's rates against."""
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    rate = 2 * n * steps / (s.elapsed_time(e) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return rate


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


MEMORY_KERNELS = [  # label, pattern over the demangled name
    ("dispatch copy", r"ep_copy_kernel<8, 8, true, false, false>"),
    ("combine", r"ep_combine_kernel<\d+, \d+, 0, true>"),
    ("probe: read", r"ep_probe_kernel<0>"),
    ("probe: write", r"ep_probe_kernel<1>"),
    ("probe: 1:1 copy", r"ep_probe_kernel<2>"),
    ("probe: dispatch fan-out", r"ep_probe_kernel<3>"),
    ("probe: combine gather", r"ep_probe_kernel<4>"),
]


def summarize_memory(out_md, csv_paths, command):
    """Memory-side counters of the headline kernels and the access-pattern
    probes, per launch: TCC (L2) cycles stalled for want of DRAM read or
    write credits, TCC busy share, mean read and write latency at the L2's
    memory interface, and L1 address-translation misses."""
    import re

    vals = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            for label, pat in MEMORY_KERNELS:
                if re.search(pat, name):
                    vals.setdefault(label, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    mean = {lab: {c: sum(v) / len(v) for c, v in cs.items()} for lab, cs in vals.items()}

    def ratio(m, a, b):
        return m[a] / m[b] if a in m and b in m and m[b] else float("nan")

    out = ["# Memory-side counters of the headline kernels and the access-pattern probes", "",
           f"Kernel sources sha256[:16]: {kernel_source_hash()}", "",
           "Commands (from the repository root), one counter group a run:", ""]
    out += ["    " + c for c in command.split(" ;; ")]
    out += ["", "Per launch, means over the run's launches. TCC = the L2 (all channels summed); a "
            "credit stall is a TCC cycle in which a request could not go to DRAM for want of "
            "credits; latency is in-flight requests summed per cycle over requests "
            "(TCC_EA0_*_LEVEL / TCC_EA0_*REQ), in cycles.", "",
            "| kernel | write credit stall / TCC cycles | read credit stall / TCC cycles | "
            "TCC busy / TCC cycles | read latency (cycles) | write latency (cycles) | "
            "UTCL1 translation misses / requests |",
            "|---|---|---|---|---|---|---|"]
    for label, _ in MEMORY_KERNELS:
        m = mean.get(label)
        if not m:
            continue
        out.append(
            f"| {label} | {ratio(m, 'TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum', 'TCC_CYCLE_sum'):.3f} "
            f"| {ratio(m, 'TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum', 'TCC_CYCLE_sum'):.3f} "
            f"| {ratio(m, 'TCC_BUSY_sum', 'TCC_CYCLE_sum'):.3f} "
            f"| {ratio(m, 'TCC_EA0_RDREQ_LEVEL_sum', 'TCC_EA0_RDREQ_sum'):.0f} "
            f"| {ratio(m, 'TCC_EA0_WRREQ_LEVEL_sum', 'TCC_EA0_WRREQ_sum'):.0f} "
            f"| {ratio(m, 'TCP_UTCL1_TRANSLATION_MISS_sum', 'TCP_UTCL1_REQUEST_sum'):.5f} |")
    out += ["", "Raw means per launch:", "", "| kernel | counter | value |", "|---|---|---|"]
    for label, _ in MEMORY_KERNELS:
        for c, v in sorted(mean.get(label, {}).items()):
            out.append(f"| {label} | {c} | {v:.0f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_trace(out_md, eager_csv, graph_csv, skip_eager, skip_graph, steps, command):
    """Kernel durations and the gaps between kernels of the timed calls of one
    workload, eager launches against graph replay: for each mode, the calls
    [skip, skip + steps) of the trace (the call's kernels in start order:
    route, copy and combine, with a scan kernel between route and copy in
    large calls), medians of each kernel's duration, of the gaps between
    consecutive kernels of a call, of the gap from one call's combine to the
    next call's route, and of the call period."""
    import statistics

    def calls(path):
        rows = [r for r in csv.DictReader(open(path)) if "ep::" in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        out, i = [], 0
        while i + 2 < len(rows):
            n = [rows[i + j]["Kernel_Name"] for j in range(min(4, len(rows) - i))]
            span = (4 if len(n) == 4 and "ep_scan_kernel" in n[1] and "ep_copy_kernel" in n[2]
                    and "ep_combine_kernel" in n[3] else
                    3 if "ep_copy_kernel" in n[1] and "ep_combine_kernel" in n[2] else 0)
            if span and "ep_route_kernel" in n[0]:
                out.append([(int(r["Start_Timestamp"]) / 1e3, int(r["End_Timestamp"]) / 1e3)
                            for r in rows[i:i + span]])
                i += span
            else:
                i += 1
        return out

    lines = ["# Kernel trace: eager launches against graph replay", "",
             f"Kernel sources sha256[:16]: {kernel_source_hash()}", "",
             "Commands (from the repository root):", ""]
    lines += ["    " + c for c in command.split(" ;; ")]
    results = []
    for mode, path, skip in (("eager", eager_csv, skip_eager), ("graph replay", graph_csv,
                                                                   skip_graph)):
        c = calls(path)[skip: skip + steps]
        results.append((mode, c))
    k = len(results[0][1][0]) if results[0][1] else 3
    names = ["route", "scan", "copy", "combine"] if k == 4 else ["route", "copy", "combine"]
    lines += ["", "Medians over the timed calls, in microseconds (timestamps of the kernel trace):",
              "", "| mode | calls | " + " | ".join(names) + " | " +
              " | ".join(f"gap {names[j]} -> {names[j + 1]}" for j in range(k - 1)) +
              " | gap to the next call | call period |",
              "|---|---|" + "---|" * (2 * k - 1) + "---|---|"]
    med = lambda v: statistics.median(v) if v else float("nan")
    for mode, c in results:
        c = [x for x in c if len(x) == k]
        dur = [med([x[j][1] - x[j][0] for x in c]) for j in range(k)]
        gaps = [med([x[j + 1][0] - x[j][1] for x in c]) for j in range(k - 1)]
        g3 = med([c[i + 1][0][0] - c[i][-1][1] for i in range(len(c) - 1)])
        per = med([c[i + 1][0][0] - c[i][0][0] for i in range(len(c) - 1)])
        lines.append(f"| {mode} | {len(c)} | " + " | ".join(f"{d:.2f}" for d in dur) + " | " +
                     " | ".join(f"{g:.2f}" for g in gaps) + f" | {g3:.2f} | {per:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(csv_path, out_md, command):
    rows = list(csv.DictReader(open(csv_path)))
    out = ["# rocprofv3 kernel statistics", "",
           f"Kernel sources sha256[:16]: {kernel_source_hash()}", "",
           "Command (from the repository root):", "", "    " + command, "",
           "| kernel | calls | average us | min us | max us | share |",
           "|---|---|---|---|---|---|"]
    # the library's kernels one a line; the bench's own torch and runtime
    # kernels (input fills, random numbers, copies) summed in one line
    other_calls, other_ns, other_pct = 0, 0.0, 0.0
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        if "ep::" not in name:
            other_calls += int(r["Calls"])
            other_ns += float(r["TotalDurationNs"])
            other_pct += float(r["Percentage"])
            continue
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f}% |")
    if other_calls:
        out.append(f"| other kernels (torch and runtime: fills, random inputs, copies) | "
                   f"{other_calls} | {other_ns / other_calls / 1e3:.1f} | | | {other_pct:.2f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def _counter_means(path):
    """Mean counter value per (kernel, grid size, counter)."""
    sums, counts = {}, {}
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"])
        sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
        counts[key] = counts.get(key, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def summarize_counters(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_mib, workload):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the large kernels,
    each scaled by what the same counter reads for the calibration copy
    (cal_mib MiB read and cal_mib MiB written per launch)."""
    import re

    import workloads

    fetch, write = _counter_means(fetch_csv), _counter_means(write_csv)
    cal_f, cal_w = _counter_means(cal_fetch_csv), _counter_means(cal_write_csv)
    cal_bytes = cal_mib << 20
    # the calibration copy is the kernel that moved the most bytes in its run
    f_cal = max(v for (k, g, c), v in cal_f.items() if c == "FETCH_SIZE") * 1024
    w_cal = max(v for (k, g, c), v in cal_w.items() if c == "WRITE_SIZE") * 1024
    f_scale, w_scale = cal_bytes / f_cal, cal_bytes / w_cal
    wl = workloads.WORKLOADS[workload]

    def run_dir(csv_path):  # the -d directory of the rocprofv3 run that wrote csv_path
        return os.path.dirname(csv_path) or "."

    def pick(means, pattern, grid):
        hits = sorted((g, v) for (k, g, c), v in means.items() if re.search(pattern, k))
        if grid == "min":
            hits = hits[:1]
        elif grid == "max":
            hits = hits[-1:]
        if len(hits) > 1:
            raise SystemExit(f"several kernel instances or grids match {pattern!r}")
        return [v for g, v in hits]

    for kname, sel in COUNTER_KERNELS.items():
        pattern, grid = sel if isinstance(sel, tuple) else (sel, None)
        fk, wk = pick(fetch, pattern, grid), pick(write, pattern, grid)
        if not fk or not wk:
            continue
        rd = fk[0] * 1024 * f_scale
        wr = wk[0] * 1024 * w_scale
        lines = [f"# HBM traffic per launch of {kname}, workload {workload}",
                 "# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE, one run each;",
                 f"# each scaled by the same counter on a plain {cal_mib} MiB device copy",
                 "# Commands (from the repository root):",
                 f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {run_dir(fetch_csv)} -o run -- "
                 f"python -u bench.py {COUNTER_RUN_ARGS}",
                 f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {run_dir(write_csv)} -o run -- "
                 f"python -u bench.py {COUNTER_RUN_ARGS}",
                 f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d {run_dir(cal_fetch_csv)} -o run -- "
                 f"python -u bench.py --copy-calibration {cal_mib} --steps 3 --warmup 1",
                 f"#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d {run_dir(cal_write_csv)} -o run -- "
                 f"python -u bench.py --copy-calibration {cal_mib} --steps 3 --warmup 1",
                 f"#   python bench.py --summarize-counters {fetch_csv} {write_csv} {cal_fetch_csv} "
                 f"{cal_write_csv} {cal_mib} {workload}",
                 f"kernel_source_sha256_16: {kernel_source_hash()}",
                 f"fetch_size_kib_raw: {fk[0]:.1f}",
                 f"write_size_kib_raw: {wk[0]:.1f}",
                 f"fetch_scale: {f_scale:.4f}",
                 f"write_scale: {w_scale:.4f}",
                 f"hbm_read_bytes_per_launch: {rd:.0f}",
                 f"hbm_write_bytes_per_launch: {wr:.0f}",
                 f"hbm_bytes_per_launch: {rd + wr:.0f}"]
        with open(counters_path(kname, workload), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))


def measure_pattern_ceilings(cra, torch, wl, op, x, stream, kern_ms, launch, recv_total):
    """What this memory delivers on the path's own access patterns, in this
    process, on the same buffers (include/ep_probe.h): streaming reads, plain
    writes and a 1:1 copy of 14 KB rows, the dispatch copy's fan-out of each
    token row to its destination rows at the dispatch's own receive slots (the
    plan's forward map), and the combine's gather-sum of those rows back. The
    fan-out and gather move exactly the payload bytes of the copy and combine
    kernels, so a kernel's time over its pattern's time is the share of the
    pattern ceiling it reaches. Overwrites the op's outputs: the caller
    dispatches again before using them."""
    W, M, H = wl.world_size, wl.max_tokens, wl.hidden
    WM = W * M
    row = H * (1 if wl.dispatch_dtype == "fp8" else 2)
    N, R = W * M, int(recv_total)
    fmap, stride = cra.ep_probe_forward_map(op.plan)
    dpieces, dwaves = launch["dispatch_row_split"], launch["dispatch_waves"]
    sink = torch.empty(W * WM * dpieces * 4, dtype=torch.uint8, device="cuda")
    cpieces, cwaves = launch["combine_row_split"], launch["combine_waves"]
    probes = {
        # name: (kind, rows, src, dst, map, map_rows, pieces, waves, bytes)
        "read": (cra.EP_PROBE_READ, W * WM, op.out_x, sink, None, 0, dpieces, dwaves,
                 W * WM * row),
        "write": (cra.EP_PROBE_WRITE, W * WM, None, op.out_x, None, 0, dpieces, dwaves,
                  W * WM * row),
        "copy_1to1": (cra.EP_PROBE_COPY, N, x, op.out_x, None, 0, dpieces, dwaves, 2 * N * row),
        "fanout_dispatch": (cra.EP_PROBE_FANOUT, N, x, op.out_x, fmap, W * WM, dpieces, dwaves,
                            (N + R) * row),
        "gather_combine": (cra.EP_PROBE_GATHER, N, op.out_x, op.combine_out, fmap, W * WM,
                           cpieces, cwaves, (N + R) * row),
    }
    out = {"method": "include/ep_probe.h kernels on the op's own buffers, 2 warmups + 10 "
                     "launches between HIP events on the launch stream; 14 KB rows; fan-out "
                     "and gather through the dispatch's forward map (the same rows and bytes "
                     "as the payload of the copy and combine kernels)"}
    for name, (kind, rows, src, dst, mp, mrows, pieces, waves, nbytes) in probes.items():
        fn = (lambda kind=kind, rows=rows, src=src, dst=dst, mp=mp, mrows=mrows, pieces=pieces,
              waves=waves: cra.ep_probe_pattern(kind, row, rows, src, dst, mp, mrows, stride,
                                                pieces, waves, stream=stream))
        ms = _timed(torch, stream, fn, 10, 2)
        out[name] = {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "pct_of_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                     "bytes": int(nbytes)}
    # the kernels against their patterns: same payload bytes, so the ratio of
    # times; the kernels also move their metadata (ids, weights, maps)
    out["copy_kernel_pct_of_fanout"] = round(100 * out["fanout_dispatch"]["us"] /
                                             (kern_ms["copy"] * 1e3), 1)
    out["combine_kernel_pct_of_gather"] = round(100 * out["gather_combine"]["us"] /
                                                (kern_ms["combine"] * 1e3), 1)
    del sink
    return out


def run_oracle_call(oracle, np, wl, inp, y_host, in_place):
    """One dispatch + combine of the CPU oracle on the workload's inputs;
    returns (dispatch results, combine out, combine weights)."""
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
    import torch

    xb = inp["x"].view(torch.uint8).numpy()
    scn = None if inp["scales"] is None else inp["scales"].numpy()
    ref = oracle.dispatch(W, M, k, wl.experts_per_rank, inp["ntok"], xb, inp["idx"].numpy(),
                          inp["w"].numpy(), scn)
    y16 = (ref["out_x"].view(np.uint16).reshape(W, W * M, H) if in_place
           else y_host.view(torch.int16).numpy().view(np.uint16))
    ro, rw = oracle.combine(W, M, k, H, oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16,
                            inp["ntok"], ref["fwd"], y16, ref["out_w"])
    return ref, ro, rw


def cpu_baseline_all_cores(oracle, np, wl, payload_of, tokens=512):
    """The oracle, unchanged and single-threaded per call, run as one call per
    host core at once (ctypes releases the interpreter lock during each C
    call): aggregate payload GB/s over a bounded sample, the workload's shape
    with `tokens` tokens a rank (its first tokens, same ids and rows)."""
    import threading

    import torch

    import workloads

    W = wl.world_size
    sub = workloads.Workload(wl.name + f"_first{tokens}", W, tokens, wl.hidden,
                             wl.dispatch_dtype, wl.combine_dtype, wl.num_experts, wl.topk,
                             wl.scale_dim, wl.routing, wl.ragged, wl.expert, wl.seed_index)
    full = workloads.make_inputs(wl)
    inp = {"ntok": [min(t, tokens) for t in full["ntok"]],
           "x": full["x"][:, :tokens].contiguous(), "idx": full["idx"][:, :tokens].contiguous(),
           "w": full["w"][:, :tokens].contiguous(),
           "scales": None if full["scales"] is None else full["scales"][:, :tokens].contiguous()}
    del full
    cores = min(16, os.cpu_count() or 1)
    recv = []

    def one():
        ref, _, _ = run_oracle_call(oracle, np, sub, inp, None, True)
        recv.append(int(ref["recv"].sum()))

    one()                       # warmup, and the sample's received rows
    threads = [threading.Thread(target=one) for _ in range(cores)]
    t = time.perf_counter()
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    wall = time.perf_counter() - t
    nbytes = payload_of(sub, inp["ntok"], recv[0])
    return {"value": round(cores * nbytes / wall / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{cores} concurrent single-threaded oracle calls (dispatch + combine), "
                      f"each on the first {tokens} tokens of every rank of {wl.name}; "
                      f"{wall:.2f} s wall for all of them"}


def measure_small_workloads(args, cra, torch, np):
    """Every workload other than the headline, at its full size: µs per
    dispatch + combine call (eager launches and graph replay), per-kernel
    durations, payload GB/s against the 8 TB/s peak, the time the 70% mark
    asks for, and a bit-exact check against the oracle (whose time is that
    workload's CPU baseline)."""
    import workloads

    out = {}
    steps = max(args.small_steps, 1)
    for name, wl in workloads.WORKLOADS.items():
        if name == workloads.HEADLINE:
            continue
        W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
        inp = workloads.make_inputs(wl)
        cfg = cra.make_config(W, H, M, wl.experts_per_rank, k, wl.dispatch_dtype,
                              wl.combine_dtype, scale_dim=wl.scale_dim, scale_type_size=4)
        op = cra.EpDispatchCombineOp(cfg)
        dev = torch.device("cuda")
        x, idx, w = inp["x"].to(dev), inp["idx"].to(dev), inp["w"].to(dev)
        sc = None if inp["scales"] is None else inp["scales"].to(dev)
        ntok = inp["ntok"]
        in_place = wl.expert == "identity" and wl.dispatch_dtype == wl.combine_dtype
        if in_place:
            y_host, y = None, op.out_x
        else:   # a seeded expert output of the combine type
            g = torch.Generator().manual_seed(workloads.BASE_SEED + 77)
            y_host = torch.randn((W, W * M, H), generator=g).to(
                workloads.TORCH_DTYPE[wl.combine_dtype])
            y = y_host.to(dev)
        stream = torch.cuda.current_stream()

        def step():
            op.dispatch(ntok, x, idx, w, sc, stream=stream)
            op.combine(y, op.out_weights, stream=stream)

        step()
        torch.cuda.synchronize()
        recv = op.recv_num_token.cpu().numpy()
        payload, kb = algorithmic_bytes(wl, ntok, recv.sum())
        rec = {"workload": name}
        if not args.no_cpu_baseline:
            import oracle

            t = time.perf_counter()
            ref, ro, rw = run_oracle_call(oracle, np, wl, inp, y_host, in_place)
            cpu_s = time.perf_counter() - t
            ok = np.array_equal(recv, ref["recv"])
            gout = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
            gw = op.combine_weights.cpu().numpy().view(np.uint32)
            for d in range(W):
                Rd = int(recv[d])
                ok = ok and np.array_equal(op.out_x[d, :Rd].view(torch.uint8).cpu().numpy(),
                                           ref["out_x"][d, :Rd])
            for r in range(W):
                ok = ok and np.array_equal(gout[r, :ntok[r]], ro[r, :ntok[r]])
                ok = ok and np.array_equal(gw[r, :ntok[r]], rw[r, :ntok[r]].view(np.uint32))
            if not ok:
                print(f"bench.py: {name}: GPU results differ from the oracle", file=sys.stderr)
                sys.exit(1)
            rec["check"] = "bit-exact vs oracle (receive rows, combine rows and weights)"
            rec["cpu_baseline"] = {"value": round(payload / cpu_s / 1e9, 3), "unit": "GB/s",
                                   "cores": 1, "kind": "oracle",
                                   "sample": f"one call, {cpu_s * 1e3:.1f} ms"}
        ms = _timed(torch, stream, step, steps, 20)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            step()
        host_us = (time.perf_counter() - t) / steps * 1e6
        torch.cuda.synchronize()
        # one step captured in a HIP graph and replayed (the pages' method)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                op.dispatch(ntok, x, idx, w, sc, stream=side)
                op.combine(y, op.out_weights, stream=side)
        torch.cuda.synchronize()
        ms_graph = _timed(torch, stream, graph.replay, steps, 20)
        del graph
        # ten steps captured in one graph: the per-replay launch cost spread
        # over ten calls
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph10, stream=side):
                for _ in range(10):
                    op.dispatch(ntok, x, idx, w, sc, stream=side)
                    op.combine(y, op.out_weights, stream=side)
        torch.cuda.synchronize()
        ms_graph10 = _timed(torch, stream, graph10.replay, max(1, steps // 10), 2) / 10
        del graph10
        cra.ep_plan_set_timing(op.plan, True)
        torch.cuda.synchronize()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        kern = {}
        for kn, kid in (("route", cra.EP_KERNEL_ROUTE), ("scan", cra.EP_KERNEL_SCAN),
                        ("copy", cra.EP_KERNEL_COPY), ("combine", cra.EP_KERNEL_COMBINE)):
            c, t_ms = cra.ep_plan_kernel_time(op.plan, kid)
            if c:
                kern[kn] = round(t_ms / c * 1e3, 2)
        cra.ep_plan_set_timing(op.plan, False)
        rate = payload / (ms * 1e-3) / 1e9
        rec.update({
            "us_per_call": round(ms * 1e3, 2),
            "us_per_call_graph_replay": round(ms_graph * 1e3, 2),
            "us_per_call_graph_replay_10_calls_a_graph": round(ms_graph10 * 1e3, 2),
            "host_issue_us_per_call": round(host_us, 2),
            "kernel_us": kern,
            "payload_bytes_per_call": int(payload),
            "received_rows": int(recv.sum()),
            "payload_GBps": round(rate, 1),
            "frac_of_peak": round(rate / PEAK_HBM_GBS, 4),
            "us_at_70pct_of_peak": round(payload / (0.7 * PEAK_HBM_GBS * 1e9) * 1e6, 2),
            "launch": cra.ep_plan_get_launch(op.plan, ntok),
            "steps": steps,
        })
        op.close()
        del op, x, idx, w, sc, y
        torch.cuda.empty_cache()
        out[name] = rec
    return out


def placement_states(args):
    """The headline's dispatch copy and combine, per call, in four
    placements of the same buffers in one process: allocated fresh (A);
    again after a cast op of the same shape was allocated, used and released
    (B); again with nothing in between (C); after another such cast op (D).
    Prints one line a call; under rocprofv3 --pmc the calls' counters are
    told apart by their order."""
    import torch

    import combine_route_amd as cra
    import workloads

    wl = workloads.WORKLOADS[workloads.HEADLINE]
    W, M, k, H, Er = wl.world_size, wl.max_tokens, wl.topk, wl.hidden, wl.experts_per_rank
    inp = workloads.make_inputs(wl)
    ntok = inp["ntok"]
    x, idx, w = inp["x"].cuda(), inp["idx"].cuda(), inp["w"].cuda()
    stream = torch.cuda.current_stream()

    def phase(tag):
        op = cra.EpDispatchCombineOp(cra.make_config(W, H, M, Er, k, "bf16", "bf16"))
        cra.ep_plan_set_timing(op.plan, True)
        prev = (0.0, 0.0)
        for i in range(args.steps):
            op.dispatch(ntok, x, idx, w, stream=stream)
            op.combine(op.out_x, op.out_weights, stream=stream)
            torch.cuda.synchronize()
            # the plan's timers add up: this call's durations are the increments
            c1 = cra.ep_plan_kernel_time(op.plan, cra.EP_KERNEL_COPY)[1]
            c2 = cra.ep_plan_kernel_time(op.plan, cra.EP_KERNEL_COMBINE)[1]
            print(json.dumps({"phase": tag, "call": i, "copy_us": round((c1 - prev[0]) * 1e3, 1),
                              "combine_us": round((c2 - prev[1]) * 1e3, 1)}), flush=True)
            prev = (c1, c2)
        op.close()
        del op
        torch.cuda.empty_cache()

    def perturb():
        op = cra.EpDispatchCombineOp(cra.make_config(W, H, M, Er, k, "fp8", "bf16",
                                                     dispatch_cast="bf16"))
        for _ in range(3):
            op.dispatch(ntok, x, idx, w, stream=stream)
        torch.cuda.synchronize()
        op.close()
        del op
        torch.cuda.empty_cache()

    phase("A")
    perturb()
    phase("B")
    phase("C")
    perturb()
    phase("D")


def summarize_placement(out_md, timing_log, csv_paths, command, calls):
    """Per call of placement_states: kernel times and memory-side counters."""
    import re

    times = [json.loads(l) for l in open(timing_log) if l.startswith("{")]
    per = {}
    for path in csv_paths:
        for r in csv.DictReader(open(path)):
            n = r["Kernel_Name"]
            kind = ("copy" if re.search(r"ep_copy_kernel<8, 8, true, false, false>", n) else
                    "combine" if re.search(r"ep_combine_kernel<\d+, \d+, 0, true>", n) else None)
            if kind:
                key = (path, int(r["Dispatch_Id"]), kind)
                per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    lines = ["# The headline kernels in four placements of the same buffers", "",
             f"Kernel sources sha256[:16]: {kernel_source_hash()}", "",
             "Commands (from the repository root):", ""]
    lines += ["    " + c for c in command.split(" ;; ")]
    lines += ["", "Phases: A allocated fresh; B after a cast op of the same shape was "
              "allocated, used and released; C allocated again; D after another cast op. "
              "Kernel times from the library's HIP events (no profiler); counters from the "
              "profiled runs, the same calls in the same order.", "",
              "| phase | call | copy µs | combine µs | copy: read latency (cycles) | "
              "copy: write credit stall / TCC cycles | copy: TCC cycles (M) |",
              "|---|---|---|---|---|---|---|"]
    for kind in ("copy",):
        byfile = {}
        for (path, d, kd), v in sorted(per.items()):
            if kd == kind:
                byfile.setdefault(path, []).append(v)
    merged = [dict() for _ in range(len(times))]
    for path, vs in byfile.items():
        for i, v in enumerate(vs[:len(times)]):
            merged[i].update(v)
    for t, m in zip(times, merged):
        lat = (m["TCC_EA0_RDREQ_LEVEL_sum"] / m["TCC_EA0_RDREQ_sum"]
               if m.get("TCC_EA0_RDREQ_sum") else float("nan"))
        st = (m["TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum"] / m["TCC_CYCLE_sum"]
              if m.get("TCC_CYCLE_sum") else float("nan"))
        cyc = m.get("TCC_CYCLE_sum", float("nan")) / 1e6
        lines.append(f"| {t['phase']} | {t['call']} | {t['copy_us']} | {t['combine_us']} | "
                     f"{lat:.0f} | {st:.3f} | {cyc:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def rocprof_frac(workload, kernel_pattern, nbytes):
    """The dominant kernel's average duration in the committed rocprofv3
    summary of this workload, taken on the current kernel sources, and the
    roofline fraction it gives for nbytes per launch; None if there is none."""
    import re

    path = os.path.join(ROOT, "profiles", f"kernel_stats_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"Kernel sources sha256\[:16\]: (\w+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    for line in text.splitlines():
        if re.search(kernel_pattern, line):
            avg_us = float(line.split("|")[3])
            a = nbytes / (avg_us * 1e-6) / 1e9
            return {"average_us": avg_us, "achieved": round(a, 2),
                    "frac": round(a / PEAK_HBM_GBS, 4), "source": os.path.relpath(path, ROOT)}
    return None


def run(args):
    import numpy as np
    import torch

    import combine_route_amd as cra
    import workloads

    wl = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
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
    cdt = workloads.TORCH_DTYPE[wl.combine_dtype]
    in_place = wl.expert == "identity" and wl.dispatch_dtype == wl.combine_dtype
    if in_place:
        y_host = None
        y = op.out_x
    else:
        g = torch.Generator().manual_seed(workloads.BASE_SEED + 77)
        y_host = torch.randn((W, W * M, H), generator=g).to(cdt)
        y = y_host.to(dev)
    stream = torch.cuda.current_stream()

    def step():
        op.dispatch(ntok, x, idx, w, sc, stream=stream)
        op.combine(y, op.out_weights, stream=stream)

    # -- correctness first, and the CPU baseline -----------------------------
    step()
    torch.cuda.synchronize()
    recv = op.recv_num_token.cpu().numpy()
    payload_bytes, kernel_bytes = algorithmic_bytes(wl, ntok, recv.sum())
    check = "skipped"
    cpu_baseline = None
    if not args.no_cpu_baseline:
        import oracle

        # 1 warmup call, then the median of cpu_runs timed calls (each the whole
        # workload, single-threaded); the last call's results are checked
        times = []
        for i in range(1 + args.cpu_runs):
            t = time.perf_counter()
            ref, ro, rw = run_oracle_call(oracle, np, wl, inp, y_host, in_place)
            if i:
                times.append(time.perf_counter() - t)
            if i < args.cpu_runs:
                del ref, ro, rw
            print(f"[bench] oracle call {i} took {time.perf_counter() - t:.2f}s", file=sys.stderr,
                  flush=True)
        cpu_s = sorted(times)[len(times) // 2]
        cpu_baseline = {"value": round(payload_bytes / cpu_s / 1e9, 3), "unit": "GB/s",
                        "cores": 1, "kind": "oracle",
                        "sample": f"the whole {wl.name} workload: one dispatch+combine call of "
                                  f"the single-threaded C oracle; 1 warmup call, then the median "
                                  f"of {args.cpu_runs} timed calls: {cpu_s:.2f} s",
                        "samples_s": [round(v, 3) for v in times],
                        "host": host_cpu()}
        if args.cpu_all_cores:
            cpu_baseline["all_cores"] = cpu_baseline_all_cores(
                oracle, np, wl, lambda w_, nt, r: algorithmic_bytes(w_, nt, r)[0])
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
            if ref["out_scales"] is not None:
                ok = ok and np.array_equal(op.out_scales[d, :Rd].cpu().numpy(),
                                           ref["out_scales"][d, :Rd])
        gout = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
        gw = op.combine_weights.cpu().numpy().view(np.uint32)
        for r in range(W):
            T = ntok[r]
            ok = ok and np.array_equal(gout[r, :T], ro[r, :T])
            ok = ok and np.array_equal(gw[r, :T], rw[r, :T].view(np.uint32))
        del ref, ro, rw
        if not ok:
            print("bench.py: GPU results differ from the oracle; not timing", file=sys.stderr)
            sys.exit(1)
        check = "bit-exact vs oracle"

    # -- timed region: K steps between two HIP events on the launch stream ---
    for _ in range(args.warmup):
        step()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if args.graph:
        # one step captured in a HIP graph, replayed K times (no host launch
        # cost between kernels; the pages time their pairs this way)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                op.dispatch(ntok, x, idx, w, sc, stream=side)
                op.combine(y, op.out_weights, stream=side)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        end.record(stream)
    else:
        start.record(stream)
        for _ in range(args.steps):
            step()
        end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    # host time to issue K steps (no GPU wait), after a synchronised start:
    # when it approaches ms_per_step the host, not the GPU, sets the pace
    torch.cuda.synchronize()
    host_t0 = time.perf_counter()
    for _ in range(args.steps):
        if args.graph:
            graph.replay()
        else:
            step()
    host_us = (time.perf_counter() - host_t0) / args.steps * 1e6
    torch.cuda.synchronize()
    # -- the same K steps again with every kernel bracketed by HIP events on
    # its stream (the library records them), for per-kernel durations; the
    # records add small gaps between kernels, so this pass is not the value
    cra.ep_plan_set_timing(op.plan, True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = {}
    for name, kid in (("route", cra.EP_KERNEL_ROUTE), ("scan", cra.EP_KERNEL_SCAN),
                      ("copy", cra.EP_KERNEL_COPY), ("combine", cra.EP_KERNEL_COMBINE)):
        c, ms = cra.ep_plan_kernel_time(op.plan, kid)
        kern[name] = ms / max(c, 1)
    cra.ep_plan_set_timing(op.plan, False)
    samples = None
    if args.rounds > 0 and args.samples > 0:
        samples = measure_samples(
            args, torch, stream, lambda: op.dispatch(ntok, x, idx, w, sc, stream=stream),
            lambda: op.combine(y, op.out_weights, stream=stream),
            lambda s: op.dispatch(ntok, x, idx, w, sc, stream=s),
            lambda s: op.combine(y, op.out_weights, stream=s))

    ceilings = None
    uniform_tokens = all(t == M for t in ntok)
    if args.ceilings and uniform_tokens and wl.dispatch_dtype != "fp8":
        ceilings = measure_pattern_ceilings(cra, torch, wl, op, x, stream, kern,
                                            cra.ep_plan_get_launch(op.plan, ntok), recv.sum())
        step()                      # the op's outputs again, for what follows
        torch.cuda.synchronize()
        print(f"[bench] pattern ceilings done at {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)

    dom = "copy" if kern["copy"] >= kern["combine"] else "combine"
    achieved = kernel_bytes[dom] / (kern[dom] * 1e-3) / 1e9
    traffic = read_traffic(wl.name, KERNELS[dom])
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
        "config": {"workload": wl.name, "world_size": W,
                   "seed": f"{workloads.BASE_SEED} + 1000 * stream + {wl.seed_index}",
                   "tokens_per_rank": ntok[0] if len(set(ntok)) == 1 else ntok,
                   "hidden": H, "topk": k, "experts": wl.num_experts,
                   "dispatch_dtype": wl.dispatch_dtype, "combine_dtype": wl.combine_dtype,
                   "scale_dim": wl.scale_dim, "weights": True,
                   "expert": "identity, in place" if in_place else "seeded random output",
                   "launches": "graph replay" if args.graph else "eager",
                   "launch": cra.ep_plan_get_launch(op.plan, ntok)},
        "us_per_call": round(ms_per_step * 1e3, 2),
        "host_issue_us_per_call": round(host_us, 2),
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "payload_bytes_per_call": payload_bytes,
        "received_rows": int(recv.sum()),
        "kernel_us": {k_: round(v * 1e3, 2) for k_, v in kern.items()},
        "samples": samples,
        "check": check,
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom], "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": kernel_bytes[dom],
                     "frac_method": "algorithmic bytes per launch (payload and metadata) over "
                                    "the kernel's mean duration between HIP events recorded "
                                    "by the library on its stream, in this run",
                     "rocprof": rocprof_frac(wl.name, COUNTER_KERNELS[KERNELS[dom]],
                                             kernel_bytes[dom])},
        "pattern_ceilings": ceilings,
        "cpu_baseline": cpu_baseline,
    }
    def progress(what):
        print(f"[bench] {what} done at {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    progress(f"headline timing ({line['us_per_call']} us a call)")
    if not args.no_expert:
        line["expert_major"] = measure_expert_major(args, cra, torch, np, wl, op, inp, stream)
        progress("expert-major layout")
        line["standard_moe"] = measure_standard_moe(args, cra, torch, np, wl, op, inp, stream,
                                                    x, idx, w, sc)
        progress("fused expert-major path")
    if not args.no_wires:
        op.close()
        torch.cuda.empty_cache()
        line["quantized_wires"] = measure_quantized_wires(args, cra, torch, np, wl, inp, stream)
        progress("quantized wires")
    op.close()
    del op, x, idx, w, sc, y
    torch.cuda.empty_cache()
    if args.small and args.workload is None:
        line["workloads"] = measure_small_workloads(args, cra, torch, np)
        progress("the other workloads")
    # the machine's own device copy rate (1 GiB, torch), measured last so its
    # buffers take no part in the placement of the timed ones
    copy_rate = device_copy_rate(torch)
    line["device_copy_GBps"] = round(copy_rate, 1)
    line["pct_of_device_copy"] = round(100.0 * value / copy_rate, 2)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle (CPU baseline and the bit-exact check); for profiling")
    ap.add_argument("--no-expert", action="store_true",
                    help="skip the expert-major layout measurement")
    ap.add_argument("--no-wires", action="store_true",
                    help="skip the quantized-wire measurements")
    ap.add_argument("--rounds", type=int, default=4,
                    help="sampling rounds of per-call timings (0 skips the sampling)")
    ap.add_argument("--samples", type=int, default=30, help="per-call samples a round")
    ap.add_argument("--graph", action="store_true",
                    help="time K replays of one step captured in a HIP graph")
    ap.add_argument("--cpu-runs", type=int, default=3,
                    help="timed oracle calls after one warmup; the CPU baseline is their median")
    ap.add_argument("--no-cpu-all-cores", dest="cpu_all_cores", action="store_false",
                    help="skip the all-core oracle figure")
    ap.add_argument("--no-ceilings", dest="ceilings", action="store_false",
                    help="skip the access-pattern ceilings")
    ap.add_argument("--no-small", dest="small", action="store_false",
                    help="skip the other workloads (run with the headline by default)")
    ap.add_argument("--small-steps", type=int, default=200,
                    help="timed calls of each other workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    ap.add_argument("--summarize-stats", nargs="+", metavar="ARG")
    ap.add_argument("--summarize-counters", nargs=6, metavar="ARG")
    ap.add_argument("--placement-states", action="store_true",
                    help="the headline kernels, per call, in four placements of their buffers")
    ap.add_argument("--summarize-placement", nargs="+", metavar="ARG",
                    help="OUT.md TIMING_LOG COMMANDS CSV...")
    ap.add_argument("--summarize-memory", nargs="+", metavar="ARG",
                    help="OUT.md COMMANDS CSV...: memory-side counter summary")
    ap.add_argument("--summarize-trace", nargs=7, metavar="ARG",
                    help="OUT.md EAGER_CSV GRAPH_CSV SKIP_EAGER SKIP_GRAPH STEPS COMMANDS")
    args = ap.parse_args()

    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1],
                        " ".join(args.summarize_stats[2:]))
        return
    if args.summarize_placement:
        a = args.summarize_placement
        summarize_placement(a[0], a[1], a[3:], a[2], None)
        return
    if args.summarize_memory:
        a = args.summarize_memory
        summarize_memory(a[0], a[2:], a[1])
        return
    if args.summarize_trace:
        a = args.summarize_trace
        summarize_trace(a[0], a[1], a[2], int(a[3]), int(a[4]), int(a[5]), a[6])
        return
    if args.summarize_counters:
        a = args.summarize_counters
        summarize_counters(a[0], a[1], a[2], a[3], int(a[4]), a[5])
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: all virtual expert-parallel "
              "ranks run on one GPU, and only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)
    if args.placement_states:
        placement_states(args)
        return
    if args.copy_calibration:
        import torch

        copy_ceiling(torch, args.copy_calibration, args.steps, args.warmup)
        return
    run(args)


if __name__ == "__main__":
    main()
