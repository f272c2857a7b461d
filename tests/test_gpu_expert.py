"""GPU parity of the expert-major layout and its inverse, through the C ABI.

"MORI-EP User Guide", section 4 "Standard MoE Compatibility (DeepEP)":
convert_dispatch_output() and convert_combine_input(). Every comparison is
bit for bit against the CPU oracle fed its own dispatch outputs (never the
GPU's): per-expert counts, layout ranges, the packed rows, scale rows and
source info of every kept slot, and the inverse's rows for every received
row. Slots and rows the call must not write are filled with a sentinel first
and checked to still hold it.
"""
import numpy as np
import pytest
import torch

import combine_route_amd as cra
import oracle
import workloads

from test_gpu_parity import _say, compare_dispatch, config_of, gpu_dispatch, oracle_dispatch

pytestmark = pytest.mark.gpu

SENTINEL_BYTE = 0xA5
SENTINEL_INT = -7


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cra.load()


def _dims(wl):
    return wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden


def max_count(wl, ref):
    """Largest per-expert row count, from the oracle (capacity 1 keeps it cheap)."""
    W, M, k, Er, _ = _dims(wl)
    o = oracle.expert_layout(W, M, k, Er, 1, ref["recv"], ref["src_pos"], ref["out_x"][:, :, :16],
                             ref["out_idx"])
    return int(o["count"].max()) if o["count"].size else 0


def _fill_outputs(ex):
    ex["packed_x"].view(torch.uint8).fill_(SENTINEL_BYTE)
    if ex["packed_scales"] is not None:
        ex["packed_scales"].fill_(SENTINEL_BYTE)
    ex["packed_src_info"].fill_(SENTINEL_INT)
    ex["packed_count"].fill_(SENTINEL_INT)
    ex["packed_layout_range"].fill_(SENTINEL_INT)
    ex["y"].view(torch.uint8).fill_(SENTINEL_BYTE)


def compare_layout(wl, cap, op, ref_ex, tag, check_untouched=True):
    W, M, k, Er, H = _dims(wl)
    ex = op._expert_state()
    cnt = ex["packed_count"].cpu().numpy()
    assert np.array_equal(cnt, ref_ex["count"]), (tag, "count")
    lr = ex["packed_layout_range"].cpu().numpy()
    assert np.array_equal(lr, ref_ex["layout_range"]), (tag, "layout_range")
    si = ex["packed_src_info"].cpu().numpy()
    for d in range(W):
        px_d = ex["packed_x"][d].view(torch.uint8).reshape(Er, cap, -1)
        ps_d = None if ex["packed_scales"] is None else ex["packed_scales"][d]
        for j in range(Er):
            n = min(int(cnt[d, j]), cap)
            if n:
                got = px_d[j, :n].cpu().numpy()
                assert np.array_equal(got, ref_ex["px"][d, j, :n]), (tag, "packed_x", d, j)
                assert np.array_equal(si[d, j, :n], ref_ex["src_info"][d, j, :n]), (tag, "src_info")
                if ps_d is not None:
                    assert np.array_equal(ps_d[j, :n].cpu().numpy(), ref_ex["psc"][d, j, :n]), \
                        (tag, "packed_scales", d, j)
            if check_untouched and n < cap:
                assert (si[d, j, n:] == SENTINEL_INT).all(), (tag, "src_info written past", d, j)
                rest = px_d[j, n:]
                assert bool((rest == SENTINEL_BYTE).all()), (tag, "packed_x written past", d, j)
                if ps_d is not None:
                    assert bool((ps_d[j, n:] == SENTINEL_BYTE).all()), (tag, "scales past", d, j)


def compare_inverse(wl, ref, y_dev, ref_y, tag, check_untouched=True):
    W = wl.world_size
    g = y_dev.view(torch.int16).cpu().numpy().view(np.uint16)
    for d in range(W):
        R = int(ref["recv"][d])
        assert np.array_equal(g[d, :R], ref_y[d, :R]), (tag, "inverse", d)
        if check_untouched:
            assert (g[d, R:] == (SENTINEL_BYTE << 8 | SENTINEL_BYTE)).all(), (tag, "y past", d)


def random_outputs(wl, cap, seed):
    W, M, k, Er, H = _dims(wl)
    g = torch.Generator().manual_seed(seed)
    v = torch.randn((W, Er, cap, H), generator=g).to(workloads.TORCH_DTYPE[wl.combine_dtype])
    return v


def run_expert_case(wl, cap=None, cap_div=1, inp=None, launch=None, tag=None,
                    check_untouched=True, py="random", round_trip=False, weighted=False):
    """Dispatch on the GPU, convert, invert, and compare each stage with the
    oracle. cap: rows kept per expert (default: the largest count / cap_div).
    py: "random" expert outputs or "identity" (the packed rows themselves).
    weighted: the conversion gets the dispatched weights and the inverse
    applies them."""
    W, M, k, Er, H = _dims(wl)
    inp = inp or workloads.make_inputs(wl)
    ref = oracle_dispatch(wl, inp)
    if cap is None:
        cap = max(1, max_count(wl, ref) // cap_div)
    tag = tag or f"{wl.name} cap={cap}"
    _say(f"[case] {tag}: W={W} M={M} H={H} k={k} Er={Er} {wl.dispatch_dtype}->"
         f"{wl.combine_dtype} launch={launch}")
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=weighted, expert_capacity=cap)
    if launch is not None:
        op.set_launch(launch)
    ex = op._expert_state()
    if check_untouched:
        _fill_outputs(ex)
    gpu_dispatch(op, inp if weighted else dict(inp, w=None))
    torch.cuda.synchronize()
    compare_dispatch(wl, op, ref if weighted else dict(ref, out_w=None), tag)

    op.convert_dispatch_output(op.out_x, op.out_indices, op.out_scales,
                               op.out_weights if weighted else None)
    torch.cuda.synchronize()
    ref_ex = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"], ref["out_x"],
                                  ref["out_idx"], ref["out_scales"], fill=SENTINEL_INT)
    compare_layout(wl, cap, op, ref_ex, tag, check_untouched)

    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    if py == "identity":
        assert wl.dispatch_dtype == wl.combine_dtype
        py_dev = ex["packed_x"]
        py16 = ref_ex["px"].view(np.uint16)
    else:
        v = random_outputs(wl, cap, seed=sum(tag.encode()) % 10007)
        py_dev = v.cuda()
        py16 = v.view(torch.int16).numpy().view(np.uint16)
    y = op.convert_combine_input(py_dev, ex["packed_src_info"], ex["packed_layout_range"],
                                 apply_weights=weighted)
    torch.cuda.synchronize()
    ref_y = oracle.expert_combine(W, M, k, Er, cap, H, dt, ref["recv"], ref["out_idx"], py16,
                                  w=ref["out_w"] if weighted else None)
    compare_inverse(wl, ref, y, ref_y, tag, check_untouched)

    if round_trip:
        out, _ = op.combine(y)
        torch.cuda.synchronize()
        ro, _ = oracle.combine(W, M, k, H, dt, inp["ntok"], ref["fwd"], ref_y)
        g = out.view(torch.int16).cpu().numpy().view(np.uint16)
        for r in range(W):
            T = inp["ntok"][r]
            assert np.array_equal(g[r, :T], ro[r, :T]), (tag, "round trip combine", r)
    op.close()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    """Every workload at full size in the automatic launch geometry; no row
    dropped; identity experts where the element types match, and the whole
    chain through combine."""
    wl = workloads.WORKLOADS[name]
    identity = wl.dispatch_dtype == wl.combine_dtype
    run_expert_case(wl, check_untouched=name != workloads.HEADLINE,
                    py="identity" if identity else "random", round_trip=True)


SMALL = [
    workloads.custom("ex_ep2_t64_h256_k8", 2, 64, 256, 8, 16, "bf16", seed_index=501),
    workloads.custom("ex_ep4_t48_h128_fp16_k6", 4, 48, 128, 6, 24, "fp16", ragged=True,
                     seed_index=502),
    workloads.custom("ex_ep3_t40_h256_fp8_k5_s2", 3, 40, 256, 5, 12, "fp8", scale_dim=2,
                     seed_index=503),
    workloads.custom("ex_ep4_t32_h64_k16_zipf", 4, 32, 64, 16, 64, "bf16", routing="zipf",
                     seed_index=504),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("cap_div", [1, 2, 1000])
def test_capacity_drops(wl, cap_div):
    """Full capacity, half (rows dropped, counts still full) and capacity 1."""
    run_expert_case(wl, cap_div=cap_div)


@pytest.mark.parametrize("W,E,k", [(2, 300, 8), (1, 130, 9), (4, 520, 17), (2, 40, 33),
                                   (3, 66, 64), (64, 512, 8), (8, 64, 1), (1, 600, 12)])
def test_world_expert_topk_sweep(W, E, k):
    """More than 64 experts a rank (several mask words), more than 256 (the
    copy's positions over several LDS windows), every top-k bucket, 64
    source ranks, one rank."""
    M = 96 if W <= 8 else 12
    wl = workloads.custom(f"ex_sweep_W{W}_E{E}_k{k}", W, M, 128, k, E, "bf16", ragged=True,
                          seed_index=510 + W + k)
    run_expert_case(wl, round_trip=True)


@pytest.mark.parametrize("launch", [
    dict(expert_waves=1, expert_combine_waves=1),
    dict(expert_waves=16, expert_row_split=7, expert_combine_waves=16,
         expert_combine_row_split=5),
    dict(expert_row_split=1, expert_combine_row_split=1, expert_cache_policy=cra.EP_CACHE_STREAM),
    dict(expert_waves=3, expert_row_split=2, expert_cache_policy=cra.EP_CACHE_KEEP),
    # tiles shared between blocks: shares of 22, 13 (ragged tails), 1 row
    dict(expert_token_split=3),
    dict(expert_token_split=5, expert_waves=2, expert_row_split=1),
    dict(expert_token_split=64, expert_waves=1),
    # count and scan as two kernels (this call's tiles otherwise take one)
    dict(layout=cra.EP_LAYOUT_KERNELS),
])
def test_geometry_does_not_change_results(launch):
    wl = workloads.custom("ex_geom_ep4_t200_h1024", 4, 200, 1024, 8, 64, "bf16", ragged=True,
                          seed_index=520)
    run_expert_case(wl, launch=launch, cap_div=2)


@pytest.mark.parametrize("launch", [
    # inverse pieces of 512 and 256 columns: loaded a column chunk at a time
    # for all rows of a token before folding (pieces of at most 128 columns
    # fold row by row)
    dict(expert_combine_row_split=1, expert_combine_waves=4),
    dict(expert_combine_row_split=2, expert_combine_waves=3),
    # 64 columns, the largest one-column-a-lane piece; 16 waves
    dict(expert_combine_row_split=8, expert_combine_waves=16),
])
@pytest.mark.parametrize("weighted", [False, True])
def test_inverse_fold_kinds(launch, weighted):
    wl = workloads.custom("ex_fold_ep4_t150_h4096", 4, 150, 4096, 8, 64, "bf16", ragged=True,
                          seed_index=523)
    run_expert_case(wl, launch=launch, weighted=weighted, round_trip=True)


@pytest.mark.parametrize("weighted", [False, True])
def test_large_ragged_call(weighted):
    """The inverse of a large call (16 waves a block, rows numbered with the
    piece fastest, 1 KB pieces folded row by row), ragged ranks, a row of
    257 16-byte vectors."""
    wl = workloads.custom("ex_large_ragged_ep8_h2056", 8, 4096, 2056, 8, 256, "bf16",
                          seed_index=532)
    inp = dict(workloads.make_inputs(wl),
               ntok=[4096, 3001, 4095, 2048, 4096, 3333, 4000, 1])
    run_expert_case(wl, inp=inp, weighted=weighted, round_trip=True)


def test_empty_and_edge_counts():
    wl = workloads.custom("ex_edge_ep4_t70_h256", 4, 70, 256, 4, 32, "bf16", seed_index=521)
    for ntok in ([0, 0, 0, 0], [70, 0, 0, 1], [1, 1, 1, 1], [64, 65, 0, 70]):
        inp = workloads.make_inputs(wl)
        inp["ntok"] = ntok
        run_expert_case(wl, inp=inp, cap=8, tag=f"edges ntok={ntok}")


def test_invalid_and_duplicate_ids():
    wl = workloads.custom("ex_ids_ep4_t48_h256", 4, 48, 256, 6, 16, "bf16", seed_index=522)
    inp = workloads.make_inputs(wl)
    g = torch.Generator().manual_seed(9)
    idx = torch.randint(-3, 19, inp["idx"].shape, generator=g, dtype=torch.int32)
    idx[0, 0] = -1
    idx[1, :8] = idx[1, :8, :1]
    idx[2, :5, :3] = 5                   # one expert named three times
    inp["idx"] = idx.contiguous()
    run_expert_case(wl, inp=inp, tag="ex invalid+duplicate ids", round_trip=True)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_weighted_full_size(name):
    """The weighted inverse at full size, through combine (the mixture sum)."""
    wl = workloads.WORKLOADS[name]
    identity = wl.dispatch_dtype == wl.combine_dtype
    run_expert_case(wl, check_untouched=name != workloads.HEADLINE,
                    py="identity" if identity else "random", round_trip=True, weighted=True)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("cap_div", [1, 3])
def test_weighted_capacity_drops(wl, cap_div):
    run_expert_case(wl, cap_div=cap_div, weighted=True, tag=f"weighted {wl.name} /{cap_div}")


def test_weighted_repeated_ids_and_many_experts():
    """Repeated ids (their weights add up), invalid ids, and more than 64
    experts a rank (the LDS path for repeats)."""
    for wl in (workloads.custom("exw_ids_ep4_t48_h256", 4, 48, 256, 6, 16, "bf16",
                                seed_index=530),
               workloads.custom("exw_ep2_t40_h128_E300_k9", 2, 40, 128, 9, 300, "bf16",
                                seed_index=531)):
        inp = workloads.make_inputs(wl)
        g = torch.Generator().manual_seed(13)
        E = wl.num_experts
        idx = torch.randint(-2, E + 2, inp["idx"].shape, generator=g, dtype=torch.int32)
        idx[:, :6, 1] = idx[:, :6, 0]          # repeated experts
        inp["idx"] = idx.contiguous()
        run_expert_case(wl, inp=inp, weighted=True, round_trip=True, tag=f"weighted ids {wl.name}")


def test_weighted_needs_weights_at_conversion():
    wl = workloads.custom("exw_state_ep2_t32_h128", 2, 32, 128, 4, 8, "bf16", seed_index=532)
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=64)
    gpu_dispatch(op, inp)
    px, _, _, _ = op.convert_dispatch_output(op.out_x, op.out_indices)
    with pytest.raises(cra.EpError) as e:
        op.convert_combine_input(px, apply_weights=True)
    assert e.value.code == cra.EP_ERR_STATE and "no weights" in str(e.value)
    op.convert_dispatch_output(op.out_x, op.out_indices, None, op.out_weights)
    op.convert_combine_input(px, apply_weights=True)
    op.convert_combine_input(px)               # the plain sum still works
    torch.cuda.synchronize()
    op.close()


def test_state_errors_and_reconvert():
    wl = workloads.custom("ex_state_ep2_t32_h128", 2, 32, 128, 4, 8, "bf16", seed_index=523)
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=64)
    with pytest.raises(cra.EpError) as e:
        op.convert_combine_input(torch.zeros(1, device="cuda"))
    assert e.value.code == cra.EP_ERR_STATE
    gpu_dispatch(op, inp)
    ex = op._expert_state()
    py = torch.zeros_like(ex["packed_x"])
    with pytest.raises(cra.EpError) as e:
        op.convert_combine_input(py)      # no conversion yet
    assert e.value.code == cra.EP_ERR_STATE
    op.convert_dispatch_output(op.out_x, op.out_indices)
    op.convert_combine_input(py)
    gpu_dispatch(op, inp)                 # a new routing: the map is stale
    with pytest.raises(cra.EpError) as e:
        op.convert_combine_input(py)
    assert e.value.code == cra.EP_ERR_STATE and "dispatched again" in str(e.value)
    op.convert_dispatch_output(op.out_x, op.out_indices)
    op.convert_combine_input(py)
    with pytest.raises(ValueError):
        op.convert_combine_input(py, torch.zeros_like(ex["packed_src_info"]))
    torch.cuda.synchronize()
    op.close()


def test_deterministic_across_runs():
    """Two runs on fresh plans give the same bytes in every written slot."""
    wl = workloads.custom("ex_det_ep8_t256_h512", 8, 256, 512, 8, 128, "bf16", seed_index=524)
    inp = workloads.make_inputs(wl)
    runs = []
    for rep in range(2):
        op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=512)
        gpu_dispatch(op, inp)
        px, cnt, si, lr = op.convert_dispatch_output(op.out_x, op.out_indices)
        y = op.convert_combine_input(px)
        torch.cuda.synchronize()
        recv = op.recv_num_token.cpu()
        cnt = cnt.cpu()
        kept = [(d, j, int(cnt[d, j])) for d in range(8) for j in range(16)]
        runs.append(dict(
            cnt=cnt, lr=lr.cpu(),
            px=[px[d, j, :n].view(torch.int16).cpu() for d, j, n in kept],
            si=[si[d, j, :n].cpu() for d, j, n in kept],
            y=[y[d, :int(recv[d])].view(torch.int16).cpu() for d in range(8)]))
        op.close()
    a, b = runs
    assert torch.equal(a["cnt"], b["cnt"]) and torch.equal(a["lr"], b["lr"])
    for key in ("px", "si", "y"):
        for u, v in zip(a[key], b[key]):
            assert torch.equal(u, v), key


def test_graph_replay_matches_oracle():
    """Dispatch, conversion, inverse and combine captured in one HIP graph and
    replayed with new inputs (same counts) and eager work in between."""
    wl = workloads.custom("ex_graph_ep8_t128_h1024", 8, 128, 1024, 8, 256, "bf16",
                          seed_index=525)
    W, M, k, Er, H = _dims(wl)
    cap = 256
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=False, expert_capacity=cap)
    inp0 = workloads.make_inputs(wl)
    x, idx, ntok = inp0["x"].cuda(), inp0["idx"].cuda(), inp0["ntok"]
    _say("[case] expert graph capture")

    def step():
        op.dispatch(ntok, x, idx)
        px, _, _, _ = op.convert_dispatch_output(op.out_x, op.out_indices)
        y = op.convert_combine_input(px)
        op.combine(y)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        inp = workloads.make_inputs(wl, seed=2000 + rep)
        inp["ntok"] = ntok
        x.copy_(inp["x"])
        idx.copy_(inp["idx"])
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_dispatch(wl, inp)
        ref_ex = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"],
                                      ref["out_x"], ref["out_idx"], fill=SENTINEL_INT)
        compare_layout(wl, cap, op, ref_ex, f"graph {rep}", check_untouched=False)
        ref_y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, ref["recv"],
                                      ref["out_idx"], ref_ex["px"].view(np.uint16))
        compare_inverse(wl, ref, op._expert_state()["y"], ref_y, f"graph {rep}",
                        check_untouched=False)
        ro, _ = oracle.combine(W, M, k, H, oracle.BF16, ntok, ref["fwd"], ref_y)
        gout = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(gout, ro), f"graph {rep} combine"
        del junk
    op.close()


@pytest.mark.parametrize("two_kernels", [False, True])
def test_kernel_timing_counts_expert_launches(two_kernels):
    """Each conversion and inverse is timed per kernel; this small call counts
    and scans in one launch (timed as the scan) unless EP_LAYOUT_KERNELS asks
    for two."""
    wl = workloads.custom("ex_time_ep2_t64_h256", 2, 64, 256, 4, 8, "bf16", seed_index=526)
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=64)
    if two_kernels:
        op.set_launch(dict(layout=cra.EP_LAYOUT_KERNELS))
    cra.ep_plan_set_timing(op.plan, True)
    for _ in range(3):
        gpu_dispatch(op, inp)
        px, _, _, _ = op.convert_dispatch_output(op.out_x, op.out_indices)
        op.convert_combine_input(px)
    torch.cuda.synchronize()
    for kern in (cra.EP_KERNEL_EXPERT_COUNT, cra.EP_KERNEL_EXPERT_SCAN, cra.EP_KERNEL_EXPERT_COPY,
                 cra.EP_KERNEL_EXPERT_COMBINE):
        n, ms = cra.ep_plan_kernel_time(op.plan, kern)
        want = 0 if kern == cra.EP_KERNEL_EXPERT_COUNT and not two_kernels else 3
        assert n == want and (ms > 0) == (want > 0), (kern, n, ms)
    cra.ep_plan_set_timing(op.plan, False)
    op.close()


def _random_case(seed):
    rng = np.random.default_rng(7000 + seed)
    W = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 33, 64]))
    k = int(rng.choice([1, 2, 3, 4, 6, 8, 9, 16, 17, 31, 32, 40, 64]))
    Er = max(int(rng.integers(1, 100)), -(-k // W))   # E >= k: ids are distinct
    M = int(rng.integers(1, max(2, 3000 // (W * 4))))
    dd = str(rng.choice(["bf16", "fp16", "fp8"]))
    H = int(rng.choice([16, 64, 128, 200, 512])) if dd != "fp8" else int(rng.choice([16, 128, 512]))
    S = int(rng.choice([0, 0, 1, 4, 7])) if dd == "fp8" else 0
    wl = workloads.custom(f"ex_rand{seed}", W, M, H, k, W * Er, dd, scale_dim=S,
                          ragged=bool(rng.integers(0, 2)), seed_index=600 + seed)
    launch = None
    if rng.integers(0, 2):
        launch = dict(expert_waves=int(rng.integers(1, 17)),
                      expert_row_split=int(rng.integers(1, max(2, H // 8))),
                      expert_combine_waves=int(rng.integers(1, 17)),
                      expert_combine_row_split=int(rng.integers(1, max(2, H // 8))),
                      expert_cache_policy=int(rng.integers(0, 3)))
        launch["expert_row_split"] = min(launch["expert_row_split"],
                                         H * (1 if dd == "fp8" else 2) // 16)
        launch["expert_combine_row_split"] = min(launch["expert_combine_row_split"], H * 2 // 16)
    cap_div = int(rng.choice([1, 1, 2, 5]))
    if launch is not None:  # drawn last, so the draws above stay as they were
        launch["expert_token_split"] = int(rng.integers(0, 65))
    return wl, launch, cap_div


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(seed):
    wl, launch, cap_div = _random_case(seed)
    run_expert_case(wl, launch=launch, cap_div=cap_div, tag=f"ex random seed {seed}")
