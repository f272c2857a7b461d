"""GPU parity: the gfx950 library against the CPU oracle, through the C ABI.

Every comparison is bit for bit: routing (received-row counts, src_pos),
payload, id, weight and scale rows (rows below each rank's count), and the
combine (rows of present tokens) under the fixed summation order. Inputs are
the seeded workloads; the combine's input comes from the oracle's dispatch
outputs through a simulated expert, never from the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import combine_route_amd as cra
import oracle
import workloads

import experts

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cra.load()


def config_of(wl):
    return cra.make_config(wl.world_size, wl.hidden, wl.max_tokens, wl.experts_per_rank,
                           wl.topk, wl.dispatch_dtype, wl.combine_dtype, scale_dim=wl.scale_dim,
                           scale_type_size=4)


def oracle_dispatch(wl, inp):
    xb = inp["x"].view(torch.uint8).numpy()
    sc = None if inp["scales"] is None else inp["scales"].numpy()
    w = None if inp["w"] is None else inp["w"].numpy()
    return oracle.dispatch(wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank,
                           inp["ntok"], xb, inp["idx"].numpy(), w, sc)


def gpu_dispatch(op, inp, stream=None):
    dev = lambda t: None if t is None else t.cuda()
    args = (dev(inp["x"]), dev(inp["idx"]), dev(inp["w"]), dev(inp["scales"]))
    op.dispatch(inp["ntok"], *args, stream=stream)
    return args


def compare_dispatch(wl, op, ref, tag=""):
    W = wl.world_size
    recv = op.recv_num_token.cpu().numpy()
    assert np.array_equal(recv, ref["recv"]), (tag, recv, ref["recv"])
    for d in range(W):
        R = int(recv[d])
        if R == 0:
            continue
        sp = op.src_token_pos(d)[:R].cpu().numpy()
        assert np.array_equal(sp, ref["src_pos"][d, :R]), (tag, "src_pos", d)
        gx = op.out_x[d, :R].view(torch.uint8).cpu().numpy()
        assert np.array_equal(gx, ref["out_x"][d, :R]), (tag, "out_x", d)
        gi = op.out_indices[d, :R].cpu().numpy()
        assert np.array_equal(gi, ref["out_idx"][d, :R]), (tag, "out_idx", d)
        if ref["out_w"] is not None:
            gw = op.out_weights[d, :R].cpu().numpy().view(np.uint32)
            assert np.array_equal(gw, ref["out_w"][d, :R].view(np.uint32)), (tag, "out_w", d)
        if ref["out_scales"] is not None:
            gs = op.out_scales[d, :R].cpu().numpy()
            assert np.array_equal(gs, ref["out_scales"][d, :R]), (tag, "out_scales", d)


def upload_rows(y16, recv, torch_dtype):
    """[W, WM, H] uint16 host rows -> device tensor; only received rows copied."""
    W, WM, H = y16.shape
    y_dev = torch.zeros((W, WM, H), dtype=torch_dtype, device="cuda")
    for d in range(W):
        R = int(recv[d])
        if R:
            y_dev[d, :R] = torch.from_numpy(np.ascontiguousarray(y16[d, :R]).view(np.int16)).view(
                torch_dtype).cuda()
    return y_dev


def compare_combine(wl, ntok, out, out_w, ref_out, ref_w, tag=""):
    g = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(wl.world_size):
        T = ntok[r]
        assert np.array_equal(g[r, :T], ref_out[r, :T]), (tag, "combine", r)
    if ref_w is not None:
        gw = out_w.cpu().numpy().view(np.uint32)
        for r in range(wl.world_size):
            T = ntok[r]
            assert np.array_equal(gw[r, :T], ref_w[r, :T].view(np.uint32)), (tag, "weights", r)


def combine_dtype_code(wl):
    return oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16


def run_case(wl, inp=None, launch=None, y16=None, tag=None, op=None, combine_twice=False):
    tag = tag or wl.name
    _say(f"[case] {tag}: W={wl.world_size} M={wl.max_tokens} H={wl.hidden} k={wl.topk} "
         f"{wl.dispatch_dtype}->{wl.combine_dtype} launch={launch}")
    inp = inp or workloads.make_inputs(wl)
    ref = oracle_dispatch(wl, inp)
    own = op is None
    op = op or cra.EpDispatchCombineOp(config_of(wl), with_weights=inp["w"] is not None)
    if launch is not None:
        op.set_launch(launch)
    gpu_dispatch(op, inp)
    torch.cuda.synchronize()
    compare_dispatch(wl, op, ref, tag)
    if y16 is None:
        y16 = experts.expert_output(wl, ref, inp)
    tdt = workloads.TORCH_DTYPE[wl.combine_dtype]
    y_dev = upload_rows(y16, ref["recv"], tdt)
    yw_dev = None
    if ref["out_w"] is not None:
        yw_dev = torch.from_numpy(ref["out_w"]).cuda()
    ref_out, ref_w = oracle.combine(wl.world_size, wl.max_tokens, wl.topk, wl.hidden,
                                    combine_dtype_code(wl), inp["ntok"], ref["fwd"], y16,
                                    ref["out_w"])
    for rep in range(2 if combine_twice else 1):
        out, out_w = op.combine(y_dev, yw_dev)
        torch.cuda.synchronize()
        compare_combine(wl, inp["ntok"], out, out_w, ref_out, ref_w, f"{tag} combine#{rep}")
    if own:
        op.close()
    return inp, ref


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    """Each workload at its full size, in the automatic launch geometry (the
    one the benchmark times for the headline workload)."""
    run_case(workloads.WORKLOADS[name])


@pytest.mark.parametrize("name", ["ep2_t16_h256_bf16_k2", "ep4_t256_h4096_bf16_k8",
                                  "ep4_ragged1024_h2048_fp16_k64"])
def test_random_expert_outputs(name):
    wl = workloads.WORKLOADS[name]
    g = torch.Generator().manual_seed(99)
    y = torch.randn((wl.world_size, wl.world_size * wl.max_tokens, wl.hidden), generator=g)
    y16 = y.to(workloads.TORCH_DTYPE[wl.combine_dtype]).view(torch.int16).numpy().view(np.uint16)
    run_case(wl, y16=y16, tag=name + "/randomY")


SWEEP = [(W, k) for W in (1, 2, 3, 4, 8, 16) for k in (1, 2, 7, 8, 9, 31, 32, 33, 63, 64)]


@pytest.mark.parametrize("W,k", SWEEP, ids=[f"W{W}k{k}" for W, k in SWEEP])
def test_topk_and_world_sweep(W, k):
    """Ragged token counts (a tile boundary and a ragged tail), k from 1 to 64
    (slots past 32), world sizes 1 to 16; experts per rank chosen so k
    distinct ids exist."""
    Er = max(1, -(-k // W)) + 3
    wl = workloads.custom(f"sweep_W{W}_k{k}", W, 80, 264, k, W * Er, "bf16", ragged=True,
                          seed_index=200 + W * 100 + k)
    run_case(wl)


@pytest.mark.parametrize("launch", [
    dict(tile_tokens=16), dict(tile_tokens=32), dict(tile_tokens=64),
    dict(tile_tokens=64, dispatch_waves=1, combine_waves=1),
    dict(tile_tokens=16, dispatch_waves=16, combine_waves=16),
    dict(dispatch_row_split=3, combine_row_split=5),
    dict(dispatch_row_split=64, combine_row_split=64, dispatch_waves=2),
    dict(cache_policy=cra.EP_CACHE_STREAM), dict(cache_policy=cra.EP_CACHE_KEEP),
    dict(tile_tokens=64, dispatch_row_split=1, cache_policy=cra.EP_CACHE_STREAM),
    dict(layout=cra.EP_LAYOUT_KERNELS), dict(layout=cra.EP_LAYOUT_SCAN_IN_COPY),
    dict(layout=cra.EP_LAYOUT_IN_COPY),
    dict(layout=cra.EP_LAYOUT_SCAN_IN_COPY, tile_tokens=64, dispatch_row_split=1),
    dict(layout=cra.EP_LAYOUT_IN_COPY, tile_tokens=32, dispatch_row_split=3),
    dict(layout=cra.EP_LAYOUT_KERNELS, tile_tokens=16, dispatch_row_split=2),
    dict(tile_tokens=64, dispatch_token_split=8),
    dict(tile_tokens=32, dispatch_token_split=5, dispatch_row_split=3, dispatch_waves=3),
    dict(tile_tokens=16, dispatch_token_split=64, dispatch_waves=1),
    dict(layout=cra.EP_LAYOUT_SCAN_IN_COPY, tile_tokens=64, dispatch_token_split=4,
         dispatch_row_split=2),
    dict(layout=cra.EP_LAYOUT_IN_COPY, tile_tokens=32, dispatch_token_split=3),
], ids=str)
def test_geometry_does_not_change_results(launch):
    wl = workloads.custom("geom_ep4_t300_h4096", 4, 300, 4096, 8, 256, "bf16", ragged=True,
                          seed_index=300)
    run_case(wl, launch=launch)


# Token counts of a call above the large-call threshold (at least 512 tiles of
# 32 tokens: here 773), ragged, with a rank of one token.
LARGE_RAGGED_NTOK = [4096, 3001, 4095, 2048, 4096, 3333, 4000, 1]


@pytest.mark.parametrize("W,k,H,dtype,ntok", [
    (8, 8, 2056, "bf16", LARGE_RAGGED_NTOK),
    (8, 8, 1000, "bf16", LARGE_RAGGED_NTOK),
    (8, 8, 7168, "bf16", LARGE_RAGGED_NTOK),
    (8, 2, 2056, "bf16", LARGE_RAGGED_NTOK),     # at most 2 rows a token
    (4, 64, 2048, "fp16", [4096, 4096, 4095, 4096]),  # every token on every rank
], ids=["h2056", "h1000", "h7168", "k2", "k64_fp16"])
def test_large_ragged_call(W, k, H, dtype, ntok):
    """Large calls number the dispatch copy's blocks and the combine's waves
    with the row piece fastest and fold pieces of at most 2 KB row by row.
    Ragged ranks and rows that the pieces do not divide (H = 2056: 257
    16-byte vectors in 4 pieces of 65; H = 1000: one piece of 125)."""
    wl = workloads.custom(f"large_ep{W}_k{k}_h{H}_{dtype}", W, 4096, H, k, 256, dtype,
                          seed_index=531)
    inp = dict(workloads.make_inputs(wl), ntok=list(ntok))
    op = cra.EpDispatchCombineOp(config_of(wl))
    auto = cra.ep_plan_get_launch(op.plan, inp["ntok"])
    assert auto["combine_waves"] == 16, auto  # the large-call combine
    run_case(wl, inp=inp, op=op, combine_twice=True)
    op.close()


def test_edge_token_counts():
    wl = workloads.custom("edges_ep4_t64_h512", 4, 64, 512, 8, 64, "bf16", seed_index=400)
    for ntok in ([0, 0, 0, 0], [64, 0, 64, 0], [0, 0, 0, 1], [64, 64, 64, 64], [1, 63, 17, 0]):
        inp = workloads.make_inputs(wl)
        inp["ntok"] = list(ntok)
        run_case(wl, inp=inp, tag=f"edges ntok={ntok}")


def test_invalid_and_duplicate_ids():
    wl = workloads.custom("ids_ep4_t48_h256", 4, 48, 256, 6, 16, "bf16", seed_index=401)
    inp = workloads.make_inputs(wl)
    g = torch.Generator().manual_seed(5)
    idx = torch.randint(-3, 19, inp["idx"].shape, generator=g, dtype=torch.int32)  # some invalid
    idx[0, 0] = -1                      # token with no rank at all
    idx[1, :8] = idx[1, :8, :1]         # rows of one repeated id
    inp["idx"] = idx.contiguous()
    run_case(wl, inp=inp, tag="invalid+duplicate ids")


def test_max_world_and_topk():
    wl = workloads.custom("ep64_t24_h256_k64", 64, 24, 256, 64, 256, "bf16", ragged=True,
                          seed_index=402)
    run_case(wl)


def test_scales_of_other_widths():
    for S, sts in ((3, 4), (16, 1), (6, 2), (2, 8)):
        wl = workloads.custom(f"sc{S}x{sts}", 4, 40, 512, 8, 64, "fp8", "bf16", seed_index=403)
        inp = workloads.make_inputs(wl)
        g = torch.Generator().manual_seed(S)
        nbytes = S * sts
        raw = torch.randint(0, 256, (4, 40, nbytes), generator=g, dtype=torch.uint8)
        inp["scales"] = raw
        ref = oracle_dispatch(wl, inp)
        cfg = cra.make_config(4, 512, 40, 16, 8, "fp8", "bf16", scale_dim=S, scale_type_size=sts)
        op = cra.EpDispatchCombineOp(cfg)
        _say(f"[case] scales S={S} size={sts}")
        gpu_dispatch(op, inp)
        torch.cuda.synchronize()
        compare_dispatch(wl, op, ref, f"scales {S}x{sts}")
        op.close()


def test_no_weights():
    wl = workloads.custom("noweights_ep4_t40", 4, 40, 512, 8, 64, "bf16", seed_index=404)
    inp = workloads.make_inputs(wl)
    inp["w"] = None
    run_case(wl, inp=inp, tag="no weights")


def test_double_combine_after_one_dispatch():
    run_case(workloads.WORKLOADS["ep4_t256_h4096_bf16_k8"], combine_twice=True,
             tag="double combine")


def test_two_plans_interleaved():
    wa = workloads.custom("inter_a", 4, 96, 1024, 8, 64, "bf16", seed_index=405)
    wb = workloads.custom("inter_b", 4, 96, 1024, 8, 64, "bf16", ragged=True, seed_index=406)
    ia, ib = workloads.make_inputs(wa), workloads.make_inputs(wb)
    ra, rb = oracle_dispatch(wa, ia), oracle_dispatch(wb, ib)
    opa = cra.EpDispatchCombineOp(config_of(wa))
    opb = cra.EpDispatchCombineOp(config_of(wb))
    _say("[case] two plans interleaved")
    gpu_dispatch(opa, ia)
    gpu_dispatch(opb, ib)
    ya = upload_rows(experts.identity(wa, ra), ra["recv"], torch.bfloat16)
    yb = upload_rows(experts.identity(wb, rb), rb["recv"], torch.bfloat16)
    oa, _ = opa.combine(ya)
    ob, _ = opb.combine(yb)
    torch.cuda.synchronize()
    compare_dispatch(wa, opa, ra, "a")
    compare_dispatch(wb, opb, rb, "b")
    for wl, inp, ref, out in ((wa, ia, ra, oa), (wb, ib, rb, ob)):
        ro, _ = oracle.combine(4, 96, 8, 1024, oracle.BF16, inp["ntok"], ref["fwd"],
                               experts.identity(wl, ref))
        compare_combine(wl, inp["ntok"], out, None, ro, None, wl.name)
    opa.close()
    opb.close()


def test_two_plans_on_two_streams():
    """Two plans enqueued on two streams (default priority) for ten rounds
    without a synchronisation in between, so their kernels can run at the
    same time: plans share no device state, so each matches the oracle."""
    wa = workloads.custom("conc_a", 8, 256, 2048, 8, 256, "bf16", seed_index=407)
    wb = workloads.custom("conc_b", 4, 512, 4096, 8, 64, "bf16", ragged=True, seed_index=408)
    ia, ib = workloads.make_inputs(wa), workloads.make_inputs(wb)
    ra, rb = oracle_dispatch(wa, ia), oracle_dispatch(wb, ib)
    opa = cra.EpDispatchCombineOp(config_of(wa))
    opb = cra.EpDispatchCombineOp(config_of(wb))
    da = tuple(t.cuda() for t in (ia["x"], ia["idx"], ia["w"]))
    db = tuple(t.cuda() for t in (ib["x"], ib["idx"], ib["w"]))
    ya = upload_rows(experts.identity(wa, ra), ra["recv"], torch.bfloat16)
    yb = upload_rows(experts.identity(wb, rb), rb["recv"], torch.bfloat16)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    _say("[case] two plans on two streams")
    for _ in range(10):
        opa.dispatch(ia["ntok"], *da, stream=sa)
        opb.dispatch(ib["ntok"], *db, stream=sb)
        oa, _ = opa.combine(ya, stream=sa)
        ob, _ = opb.combine(yb, stream=sb)
    torch.cuda.synchronize()
    compare_dispatch(wa, opa, ra, "a")
    compare_dispatch(wb, opb, rb, "b")
    for wl, inp, ref, out in ((wa, ia, ra, oa), (wb, ib, rb, ob)):
        ro, _ = oracle.combine(wl.world_size, wl.max_tokens, wl.topk, wl.hidden, oracle.BF16,
                               inp["ntok"], ref["fwd"], experts.identity(wl, ref))
        compare_combine(wl, inp["ntok"], out, None, ro, None, wl.name)
    opa.close()
    opb.close()


def test_deterministic_across_runs():
    wl = workloads.WORKLOADS["ep4_ragged1024_h2048_fp16_k64"]
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl))
    _say("[case] determinism")
    snaps = []
    for _ in range(3):
        gpu_dispatch(op, inp)
        out, _ = op.combine(op.out_x)
        torch.cuda.synchronize()
        snaps.append((op.recv_num_token.cpu().clone(), op.src_token_pos(0).cpu().clone(),
                      out.view(torch.int16).cpu().clone()))
    for s in snaps[1:]:
        for a, b in zip(snaps[0], s):
            assert torch.equal(a, b)
    op.close()


def test_graph_replay_matches_eager_and_oracle():
    """Dispatch + combine captured in one HIP graph; replayed with new input
    contents (same token counts), with eager work and synchronisations in
    between; every replay equals the oracle for its inputs."""
    wl = workloads.custom("graph_ep8_t128_h1024", 8, 128, 1024, 8, 256, "bf16", seed_index=407)
    op = cra.EpDispatchCombineOp(config_of(wl))
    inp0 = workloads.make_inputs(wl)
    x = inp0["x"].cuda()
    idx = inp0["idx"].cuda()
    w = inp0["w"].cuda()
    ntok = inp0["ntok"]
    _say("[case] graph capture")
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        op.dispatch(ntok, x, idx, w)
        op.combine(op.out_x, op.out_weights)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op.dispatch(ntok, x, idx, w)
        op.combine(op.out_x, op.out_weights)
    torch.cuda.synchronize()
    for rep in range(4):
        inp = workloads.make_inputs(wl, seed=1000 + rep)
        inp["ntok"] = ntok
        x.copy_(inp["x"])
        idx.copy_(inp["idx"])
        w.copy_(inp["w"])
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_dispatch(wl, inp)
        compare_dispatch(wl, op, ref, f"graph replay {rep}")
        ro, rw = oracle.combine(8, 128, 8, 1024, oracle.BF16, ntok, ref["fwd"],
                                experts.identity(wl, ref), ref["out_w"])
        compare_combine(wl, ntok, op.combine_out, op.combine_weights, ro, rw, f"graph {rep}")
        del junk
    op.close()


def test_kernel_timing_counts_launches():
    wl = workloads.WORKLOADS["ep2_t16_h256_bf16_k2"]
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl))
    op.set_launch(dict(layout=cra.EP_LAYOUT_KERNELS))
    cra.ep_plan_set_timing(op.plan, True)
    for _ in range(3):
        gpu_dispatch(op, inp)
        op.combine(op.out_x)
    torch.cuda.synchronize()
    for kern in range(4):
        c, ms = cra.ep_plan_kernel_time(op.plan, kern)
        assert c == 3 and ms > 0.0
    # with the scan in the copy kernel, no scan launch is timed; with the
    # whole layout there, no routing launch either
    op.set_launch(dict(layout=cra.EP_LAYOUT_SCAN_IN_COPY))
    gpu_dispatch(op, inp)
    op.set_launch(dict(layout=cra.EP_LAYOUT_IN_COPY))
    gpu_dispatch(op, inp)
    torch.cuda.synchronize()
    assert cra.ep_plan_kernel_time(op.plan, cra.EP_KERNEL_ROUTE)[0] == 4
    assert cra.ep_plan_kernel_time(op.plan, cra.EP_KERNEL_SCAN)[0] == 3
    assert cra.ep_plan_kernel_time(op.plan, cra.EP_KERNEL_COPY)[0] == 5
    cra.ep_plan_set_timing(op.plan, False)
    op.close()


@pytest.mark.parametrize("layout", [1, 2, 3], ids=["kernels", "scan_in_copy", "in_copy"])
def test_layout_placement_many_tiles(layout):
    """Every layout placement, over more tiles than the automatic limits."""
    wl = workloads.custom("layout_ep8_t700_h256_k8", 8, 700, 256, 8, 64, "bf16", ragged=True,
                          seed_index=408)
    run_case(wl, launch=dict(tile_tokens=16 if layout != 3 else 32, layout=layout))


def test_layout_in_copy_rejects_what_does_not_fit():
    wl = workloads.custom("layout_k32", 4, 64, 256, 32, 64, "bf16", seed_index=409)
    op = cra.EpDispatchCombineOp(config_of(wl))
    with pytest.raises(cra.EpError):
        op.set_launch(dict(layout=cra.EP_LAYOUT_IN_COPY))  # k > 16
    op.close()
    wl = workloads.custom("layout_many_tiles", 64, 128, 256, 8, 128, "bf16", seed_index=410)
    op = cra.EpDispatchCombineOp(config_of(wl))
    op.set_launch(dict(layout=cra.EP_LAYOUT_IN_COPY, tile_tokens=16))  # 512 tiles x 64 ranks
    inp = workloads.make_inputs(wl)
    with pytest.raises(cra.EpError):
        gpu_dispatch(op, inp)
    op.close()


def test_argument_cache_follows_new_tensors_and_counts():
    """The op reuses checked arguments only for the same tensors and counts."""
    wl = workloads.custom("cache_ep4_t64_h512", 4, 64, 512, 8, 64, "bf16", seed_index=411)
    op = cra.EpDispatchCombineOp(config_of(wl))
    _say("[case] argument cache")
    for seed, ntok in ((None, [64, 64, 64, 64]), (7, [64, 64, 64, 64]), (7, [3, 0, 64, 17])):
        inp = workloads.make_inputs(wl, seed)
        inp["ntok"] = ntok
        ref = oracle_dispatch(wl, inp)
        gpu_dispatch(op, inp)  # new tensor objects every time
        torch.cuda.synchronize()
        compare_dispatch(wl, op, ref, f"seed {seed} ntok {ntok}")
    # same tensor objects, new contents: the cached arguments still apply
    x, idx, w = inp["x"].cuda(), inp["idx"].cuda(), inp["w"].cuda()
    for seed in (8, 9):
        nxt = workloads.make_inputs(wl, seed)
        nxt["ntok"] = ntok
        x.copy_(nxt["x"])
        idx.copy_(nxt["idx"])
        w.copy_(nxt["w"])
        op.dispatch(ntok, x, idx, w)
        torch.cuda.synchronize()
        compare_dispatch(wl, op, oracle_dispatch(wl, nxt), f"in place seed {seed}")
    op.close()


def test_binding_rejects_small_or_host_tensors():
    wl = workloads.WORKLOADS["ep2_t16_h256_bf16_k2"]
    op = cra.EpDispatchCombineOp(config_of(wl))
    inp = workloads.make_inputs(wl)
    with pytest.raises(ValueError):
        op.dispatch(inp["ntok"], inp["x"], inp["idx"].cuda(), inp["w"].cuda())  # host x
    with pytest.raises(ValueError):
        op.dispatch(inp["ntok"], inp["x"].cuda()[:, :8], inp["idx"].cuda(), inp["w"].cuda())
    op.close()


def _random_case(seed):
    """A seeded random configuration and launch override, small enough for the
    oracle to finish in well under a second."""
    rng = np.random.default_rng(10_000 + seed)
    W = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 64]))
    k = int(rng.integers(1, 65))
    Er = int(rng.integers(max(1, -(-k // W)), max(1, -(-k // W)) + 6))
    M = int(rng.integers(1, 97))
    dd = str(rng.choice(["bf16", "fp16", "fp8"]))
    cd = "fp16" if dd == "fp16" else str(rng.choice(["bf16", "fp16"]))
    H = 16 * int(rng.integers(1, 49))
    S, sts = 0, 4
    if dd == "fp8" and rng.random() < 0.7:
        sts = int(rng.choice([1, 2, 4, 8]))
        S = int(rng.integers(1, 20)) * (4 // min(sts, 4))
    wl = workloads.custom(f"rand{seed}", W, M, H, k, W * Er, dd, cd, ragged=bool(rng.random() < 0.6),
                          seed_index=500 + seed)
    launch = {}
    if rng.random() < 0.7:
        launch = dict(tile_tokens=int(rng.choice([16, 32, 64])),
                      dispatch_waves=int(rng.integers(1, 17)),
                      dispatch_row_split=int(rng.integers(1, max(2, H // 8))),
                      combine_waves=int(rng.integers(1, 17)),
                      combine_row_split=int(rng.integers(1, max(2, H // 8))),
                      cache_policy=int(rng.integers(0, 3)),
                      layout=int(rng.choice([0, 1, 2] + ([3] if k <= 16 else []))))
        launch["dispatch_row_split"] = min(launch["dispatch_row_split"],
                                           H * (1 if dd == "fp8" else 2) // 16)
        launch["combine_row_split"] = min(launch["combine_row_split"], H * 2 // 16)
        launch["dispatch_token_split"] = int(rng.integers(0, 65))
    return wl, S, sts, launch


@pytest.mark.parametrize("seed", range(24))
def test_random_configurations(seed):
    wl, S, sts, launch = _random_case(seed)
    inp = workloads.make_inputs(wl)
    if S:
        g = torch.Generator().manual_seed(seed)
        inp["scales"] = torch.randint(0, 256, (wl.world_size, wl.max_tokens, S * sts),
                                      generator=g, dtype=torch.uint8)
    cfg = cra.make_config(wl.world_size, wl.hidden, wl.max_tokens, wl.experts_per_rank, wl.topk,
                          wl.dispatch_dtype, wl.combine_dtype, scale_dim=S, scale_type_size=sts)
    op = cra.EpDispatchCombineOp(cfg)
    if launch.get("layout") == 3:
        tt = launch["tile_tokens"]
        tiles = sum(-(-t // tt) for t in inp["ntok"])
        if tiles * wl.world_size > 4096:
            launch["layout"] = 2
    g = torch.Generator().manual_seed(seed + 1)
    y = torch.randn((wl.world_size, wl.world_size * wl.max_tokens, wl.hidden), generator=g)
    y16 = y.to(workloads.TORCH_DTYPE[wl.combine_dtype]).view(torch.int16).numpy().view(np.uint16)
    run_case(wl, inp=inp, launch=launch, y16=y16, op=op,
             tag=f"random seed {seed} S={S}x{sts}")
    op.close()


def test_soak_500_rounds():
    """500 dispatch + combine rounds on one plan, alternating two inputs: every
    round's outputs equal the first round's for the same input, bit for bit
    (the pages' benches soak 500 rounds)."""
    wl = workloads.custom("soak_ep4_t96_h512", 4, 96, 512, 8, 64, "bf16", ragged=True,
                          seed_index=420)
    op = cra.EpDispatchCombineOp(config_of(wl))
    inps = [workloads.make_inputs(wl, seed=4000 + i) for i in range(2)]
    dev = [tuple(None if t is None else t.cuda() for t in (i["x"], i["idx"], i["w"]))
           for i in inps]
    _say("[case] soak 500 rounds")
    first = [None, None]
    for rnd in range(500):
        j = rnd % 2
        x, idx, w = dev[j]
        ntok = inps[j]["ntok"]
        op.dispatch(ntok, x, idx, w)
        out, out_w = op.combine(op.out_x, op.out_weights)
        # rows t < T_r only: the others keep whatever the other input left
        got = (op.recv_num_token.clone(),
               *[out[r, :ntok[r]].view(torch.int16).clone() for r in range(4)],
               *[out_w[r, :ntok[r]].clone() for r in range(4)])
        if first[j] is None:
            first[j] = got
        elif rnd % 7 == 0 or rnd >= 490:
            assert all(torch.equal(a, b) for a, b in zip(got, first[j])), ("soak", rnd)
    torch.cuda.synchronize()
    # the first rounds themselves against the oracle
    for j in range(2):
        ref = oracle_dispatch(wl, inps[j])
        assert np.array_equal(first[j][0].cpu().numpy(), ref["recv"])
    op.close()
