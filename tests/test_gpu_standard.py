"""GPU parity of the fused expert-major dispatch and combine, through the C ABI.

"MORI-EP User Guide", section 4 "Standard MoE Compatibility (DeepEP)":
dispatch_standard_moe (dispatch and format conversion in one call) and
combine_standard_moe. Their results are defined as those of the two-step
path: dispatch, then convert_dispatch_output; convert_combine_input, then
combine. So the oracle here is the oracle's two steps (oracle.dispatch ->
oracle.expert_layout; oracle.expert_combine -> oracle.combine), each pinned
on its own; every comparison is bit for bit, and the fused results are also
compared with the GPU's own two-step path. Slots and rows the calls must not
write are filled with a sentinel first and checked to still hold it.
"""
import numpy as np
import pytest
import torch

import combine_route_amd as cra
import oracle
import workloads

from test_gpu_expert import (SENTINEL_BYTE, SENTINEL_INT, SMALL, _dims, _fill_outputs,
                             compare_layout, max_count, random_outputs)
from test_gpu_parity import _say, config_of, gpu_dispatch, oracle_dispatch

pytestmark = pytest.mark.gpu

SENTINEL_WORD = SENTINEL_BYTE << 8 | SENTINEL_BYTE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cra.load()


def _dev(t):
    return None if t is None else t.cuda()


def two_step_on_gpu(wl, inp, cap, py_dev, weighted, launch=None):
    """The GPU's own dispatch -> convert -> inverse -> combine, on a fresh op."""
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=weighted, expert_capacity=cap)
    if launch is not None:
        op.set_launch(launch)
    gpu_dispatch(op, inp if weighted else dict(inp, w=None))
    px, cnt, si, lr = op.convert_dispatch_output(op.out_x, op.out_indices, op.out_scales,
                                                 op.out_weights if weighted else None)
    y = op.convert_combine_input(py_dev, apply_weights=weighted)
    out, _ = op.combine(y)
    torch.cuda.synchronize()
    res = dict(cnt=cnt.cpu(), lr=lr.cpu(), out=out.view(torch.int16).cpu(),
               px=(px[0] if isinstance(px, tuple) else px).view(torch.uint8).cpu(),
               si=si.cpu())
    op.close()
    return res


def run_standard_case(wl, cap=None, cap_div=1, inp=None, launch=None, tag=None,
                      check_untouched=True, py="random", weighted=False, two_step=True):
    """Fused dispatch and combine on the GPU, each compared with the oracle's
    two steps (and, with two_step, with the GPU's two-step path)."""
    W, M, k, Er, H = _dims(wl)
    inp = inp or workloads.make_inputs(wl)
    ref = oracle_dispatch(wl, inp)
    if cap is None:
        cap = max(1, max_count(wl, ref) // cap_div)
    tag = tag or f"std {wl.name} cap={cap}"
    _say(f"[case] {tag}: W={W} M={M} H={H} k={k} Er={Er} {wl.dispatch_dtype}->"
         f"{wl.combine_dtype} weighted={weighted} launch={launch}")
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=False, expert_capacity=cap)
    if launch is not None:
        op.set_launch(launch)
    ex = op._expert_state()
    if check_untouched:
        _fill_outputs(ex)
        op.combine_out.view(torch.uint8).fill_(SENTINEL_BYTE)
    x, idx, sc = _dev(inp["x"]), _dev(inp["idx"]), _dev(inp["scales"])
    op.dispatch_standard_moe(x, None, sc, idx, num_tokens=inp["ntok"])
    torch.cuda.synchronize()
    ref_ex = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"], ref["out_x"],
                                  ref["out_idx"], ref["out_scales"], fill=SENTINEL_INT)
    compare_layout(wl, cap, op, ref_ex, tag, check_untouched)

    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    if py == "identity":
        assert wl.dispatch_dtype == wl.combine_dtype
        py_dev = ex["packed_x"].clone()
        py16 = ref_ex["px"].view(np.uint16)
    elif py == "neg_zero":
        v = torch.full((W, Er, cap, H), -0.0, dtype=workloads.TORCH_DTYPE[wl.combine_dtype])
        py_dev = v.cuda()
        py16 = v.view(torch.int16).numpy().view(np.uint16)
    else:
        v = random_outputs(wl, cap, seed=sum(tag.encode()) % 10007)
        py_dev = v.cuda()
        py16 = v.view(torch.int16).numpy().view(np.uint16)
    w = _dev(inp["w"]) if weighted else None
    out = op.combine_standard_moe(py_dev, w, idx)
    torch.cuda.synchronize()
    ref_y = oracle.expert_combine(W, M, k, Er, cap, H, dt, ref["recv"], ref["out_idx"], py16,
                                  w=ref["out_w"] if weighted else None)
    ro, _ = oracle.combine(W, M, k, H, dt, inp["ntok"], ref["fwd"], ref_y)
    g = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(W):
        T = inp["ntok"][r]
        assert np.array_equal(g[r, :T], ro[r, :T]), (tag, "fused combine", r)
        if check_untouched:
            assert (g[r, T:] == SENTINEL_WORD).all(), (tag, "combine rows past T_r", r)

    if two_step:
        gs = two_step_on_gpu(wl, inp, cap, py_dev, weighted, launch)
        assert torch.equal(gs["cnt"], ex["packed_count"].cpu()), (tag, "two-step count")
        assert torch.equal(gs["lr"], ex["packed_layout_range"].cpu()), (tag, "two-step ranges")
        gout = torch.from_numpy(g.view(np.int16))
        for r in range(W):
            T = inp["ntok"][r]
            assert torch.equal(gs["out"][r, :T], gout[r, :T]), (tag, "two-step combine", r)
    op.close()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    """Every workload at full size in the automatic launch geometry, no pair
    dropped; identity experts where the element types match."""
    wl = workloads.WORKLOADS[name]
    identity = wl.dispatch_dtype == wl.combine_dtype
    run_standard_case(wl, check_untouched=name != workloads.HEADLINE,
                      py="identity" if identity else "random",
                      two_step=name != workloads.HEADLINE)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_weighted_full_size(name):
    wl = workloads.WORKLOADS[name]
    run_standard_case(wl, check_untouched=False, weighted=True,
                      two_step=name != workloads.HEADLINE)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("cap_div", [1, 2, 1000])
@pytest.mark.parametrize("weighted", [False, True])
def test_capacity_drops(wl, cap_div, weighted):
    """Full capacity, half (pairs dropped, counts still full) and capacity 1,
    where whole ranks of a token can lose every pair."""
    run_standard_case(wl, cap_div=cap_div, weighted=weighted,
                      tag=f"std {wl.name} /{cap_div} w={weighted}")


def _zero_workload():
    return workloads.custom("std_zero_ep4_t64_h128_k6", 4, 64, 128, 6, 24, "bf16", ragged=True,
                            seed_index=550)


@pytest.mark.parametrize("cap_div", [1, 3, 1000])
@pytest.mark.parametrize("weighted", [False, True])
def test_signed_zero_with_dropped_ranks(cap_div, weighted):
    """Every expert output -0.0: a token's sum is -0.0 unless one of its ranks
    lost all its pairs, whose +0 rows turn it to +0; the fused combine must
    place those +0 terms exactly where the two-step path has them (weighted,
    each term is weight * -0.0 = -0.0)."""
    run_standard_case(_zero_workload(), cap_div=cap_div, py="neg_zero", weighted=weighted,
                      tag=f"std -0 /{cap_div} w={weighted}")


@pytest.mark.parametrize("W,E,k", [(2, 300, 8), (1, 130, 9), (4, 520, 17), (2, 40, 33),
                                   (3, 66, 64), (64, 512, 8), (8, 64, 1), (16, 48, 24),
                                   (2, 1100, 12)])
def test_world_expert_topk_sweep(W, E, k):
    """More than 64 experts (several mask words), more than 256 (repeats in
    LDS, positions over several LDS windows), at most 64 (register repeats),
    every top-k bucket, 64 source ranks, one rank, more ranks a token than a
    fold group holds."""
    M = 96 if W <= 8 else 12
    wl = workloads.custom(f"std_sweep_W{W}_E{E}_k{k}", W, M, 128, k, E, "bf16", ragged=True,
                          seed_index=560 + W + k)
    run_standard_case(wl, cap_div=2 if W % 2 else 1, weighted=W % 2 == 0)


@pytest.mark.parametrize("launch", [
    dict(expert_waves=1, expert_combine_waves=1),
    dict(expert_waves=16, expert_row_split=7, expert_combine_waves=16,
         expert_combine_row_split=5),
    dict(expert_row_split=1, expert_combine_row_split=1, expert_cache_policy=cra.EP_CACHE_STREAM),
    dict(expert_waves=3, expert_row_split=2, expert_cache_policy=cra.EP_CACHE_KEEP),
    # tiles shared between blocks: shares of 22, 13 (ragged tails), 1 token
    dict(expert_token_split=3),
    dict(expert_token_split=5, expert_waves=2, expert_row_split=1),
    dict(expert_token_split=64, expert_waves=1),
    # count and scan as two kernels (this call's 16 tiles otherwise take one)
    dict(layout=cra.EP_LAYOUT_KERNELS),
])
def test_geometry_does_not_change_results(launch):
    wl = workloads.custom("std_geom_ep4_t200_h1024", 4, 200, 1024, 8, 64, "bf16", ragged=True,
                          seed_index=570)
    run_standard_case(wl, launch=launch, cap_div=2, weighted=True)


@pytest.mark.parametrize("cap_div,weighted", [(1, True), (2, False)])
def test_large_ragged_call(cap_div, weighted):
    """The fused path on a large call (waves numbered token by token with the
    piece fastest, 2 KB pieces, 8 waves a block), ragged ranks, a row of 257
    16-byte vectors, with and without capacity drops."""
    wl = workloads.custom("sx_large_ragged_ep8_h2056", 8, 4096, 2056, 8, 256, "bf16",
                          seed_index=533)
    inp = dict(workloads.make_inputs(wl),
               ntok=[4096, 3001, 4095, 2048, 4096, 3333, 4000, 1])
    run_standard_case(wl, cap_div=cap_div, inp=inp, weighted=weighted)


def test_empty_and_edge_counts():
    wl = workloads.custom("std_edge_ep4_t70_h256", 4, 70, 256, 4, 32, "bf16", seed_index=571)
    for ntok in ([0, 0, 0, 0], [70, 0, 0, 1], [1, 1, 1, 1], [64, 65, 0, 70]):
        inp = workloads.make_inputs(wl)
        inp["ntok"] = ntok
        run_standard_case(wl, inp=inp, cap=8, tag=f"std edges ntok={ntok}")


def test_invalid_and_duplicate_ids():
    """Ids outside [0, E) select nothing; a repeated expert is one pair and,
    weighted, its slots' weights add up."""
    wl = workloads.custom("std_ids_ep4_t48_h256", 4, 48, 256, 6, 16, "bf16", seed_index=572)
    inp = workloads.make_inputs(wl)
    g = torch.Generator().manual_seed(19)
    idx = torch.randint(-3, 19, inp["idx"].shape, generator=g, dtype=torch.int32)
    idx[0, 0] = -1
    idx[1, :8] = idx[1, :8, :1]
    idx[2, :5, :3] = 5
    inp["idx"] = idx.contiguous()
    for weighted in (False, True):
        run_standard_case(wl, inp=inp, weighted=weighted, cap=8,
                          tag=f"std invalid+duplicate ids w={weighted}")


def test_fp8_scales_and_fp16_combine():
    for wl in (workloads.custom("std_fp8_ep3_t40_h256_k5_s2", 3, 40, 256, 5, 12, "fp8",
                                scale_dim=2, seed_index=573),
               workloads.custom("std_fp16_ep4_t48_h128_k6", 4, 48, 128, 6, 24, "fp16",
                                ragged=True, seed_index=574)):
        run_standard_case(wl, cap_div=2, weighted=True)


def test_state_and_interleaving_with_the_two_step_path():
    """The fused combine needs a fused dispatch on the expert plan; a
    conversion on the same expert plan ends it (they share the map's space),
    and a fused dispatch ends the conversion."""
    wl = workloads.custom("std_state_ep2_t32_h128", 2, 32, 128, 4, 8, "bf16", seed_index=575)
    inp = workloads.make_inputs(wl)
    op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=64)
    x, idx = inp["x"].cuda(), inp["idx"].cuda()
    with pytest.raises(cra.EpError) as e:
        op.combine_standard_moe(torch.zeros(1, device="cuda"), None, idx)
    assert e.value.code == cra.EP_ERR_STATE
    px, _, _, _ = op.dispatch_standard_moe(x, None, None, idx, num_tokens=inp["ntok"])
    py = px.clone()
    op.combine_standard_moe(py, None, idx)
    gpu_dispatch(op, inp)                         # the plan's own routing: no effect
    op.combine_standard_moe(py, None, idx)
    op.convert_dispatch_output(op.out_x, op.out_indices)
    with pytest.raises(cra.EpError) as e:
        op.combine_standard_moe(py, None, idx)
    assert e.value.code == cra.EP_ERR_STATE
    op.convert_combine_input(py)
    op.dispatch_standard_moe(x, None, None, idx, num_tokens=inp["ntok"])
    with pytest.raises(cra.EpError) as e:
        op.convert_combine_input(py)
    assert e.value.code == cra.EP_ERR_STATE
    op.combine_standard_moe(py, None, idx)
    torch.cuda.synchronize()
    op.close()


def test_deterministic_across_runs():
    wl = workloads.custom("std_det_ep8_t256_h512", 8, 256, 512, 8, 128, "bf16", seed_index=576)
    inp = workloads.make_inputs(wl)
    runs = []
    for rep in range(2):
        op = cra.EpDispatchCombineOp(config_of(wl), expert_capacity=300)
        x, idx, w = inp["x"].cuda(), inp["idx"].cuda(), inp["w"].cuda()
        px, cnt, si, lr = op.dispatch_standard_moe(x, w, None, idx, num_tokens=inp["ntok"])
        out = op.combine_standard_moe(px, w, idx)
        torch.cuda.synchronize()
        cnt = cnt.cpu()
        kept = [(d, j, min(int(cnt[d, j]), 300)) for d in range(8) for j in range(16)]
        runs.append(dict(cnt=cnt, lr=lr.cpu(),
                         px=[px[d, j, :n].view(torch.int16).cpu() for d, j, n in kept],
                         si=[si[d, j, :n].cpu() for d, j, n in kept],
                         out=out.view(torch.int16).cpu()))
        op.close()
    a, b = runs
    assert torch.equal(a["cnt"], b["cnt"]) and torch.equal(a["lr"], b["lr"])
    assert torch.equal(a["out"], b["out"])
    for key in ("px", "si"):
        for u, v in zip(a[key], b[key]):
            assert torch.equal(u, v)


def test_graph_replay_matches_oracle():
    """Fused dispatch + weighted fused combine captured in one HIP graph and
    replayed with new input contents (same token counts), with eager work
    and synchronisations in between; every replay equals the oracle's two
    steps for its inputs."""
    wl = workloads.custom("std_graph_ep4_t96_h512", 4, 96, 512, 8, 64, "bf16", seed_index=577)
    W, M, k, Er, H = _dims(wl)
    cap = 40
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=False, expert_capacity=cap)
    inp0 = workloads.make_inputs(wl)
    x, idx, w = inp0["x"].cuda(), inp0["idx"].cuda(), inp0["w"].cuda()
    ntok = inp0["ntok"]
    ex = op._expert_state()
    py = torch.empty_like(ex["packed_x"])

    def step():
        px, *_ = op.dispatch_standard_moe(x, None, None, idx, num_tokens=ntok)
        py.copy_(px)                      # identity experts: a copy kernel, no memset
        op.combine_standard_moe(py, w, idx)

    _say("[case] fused path graph capture")
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
    for rep in range(4):
        inp = workloads.make_inputs(wl, seed=2000 + rep)
        inp["ntok"] = ntok
        x.copy_(inp["x"])
        idx.copy_(inp["idx"])
        w.copy_(inp["w"])
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_dispatch(wl, inp)
        ref_ex = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"],
                                      ref["out_x"], ref["out_idx"], fill=SENTINEL_INT)
        compare_layout(wl, cap, op, ref_ex, f"graph replay {rep}", check_untouched=False)
        ref_y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, ref["recv"],
                                      ref["out_idx"], ref_ex["px"].view(np.uint16),
                                      w=ref["out_w"])
        ro, _ = oracle.combine(W, M, k, H, oracle.BF16, ntok, ref["fwd"], ref_y)
        got = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
        for r in range(W):
            assert np.array_equal(got[r, :ntok[r]], ro[r, :ntok[r]]), ("graph", rep, r)
        del junk
    op.close()


WIRES = {"fp8_block128": (cra.EP_WIRE_FP8_BLOCK128, oracle.WIRE_FP8_BLOCK128),
         "mxfp4": (cra.EP_WIRE_MXFP4, oracle.WIRE_MXFP4)}


def run_standard_wire_case(wl, name, cap_div=1, weighted=False, tag=None, cols=None,
                           neg_zero=False):
    """The fused combine from quantized expert outputs: the packed outputs are
    quantized on the GPU with the per-expert counts (checked against the
    oracle's quantizer on every kept row), then the oracle's own codes go to
    the fused combine, compared with the oracle's wire inverse and combine."""
    cw, ow = WIRES[name]
    W, M, k, Er, H = _dims(wl)
    inp = workloads.make_inputs(wl)
    ref = oracle_dispatch(wl, inp)
    cap = max(1, max_count(wl, ref) // cap_div)
    tag = tag or f"std wire {name} {wl.name} cap={cap} w={weighted}"
    _say(f"[case] {tag}: W={W} M={M} H={H} k={k} Er={Er}")
    cfg = cra.make_config(W, H, M, Er, k, wl.dispatch_dtype, wl.combine_dtype,
                          scale_dim=wl.scale_dim, scale_type_size=4, combine_wire=cw)
    op = cra.EpDispatchCombineOp(cfg, with_weights=False, expert_capacity=cap)
    x, idx, sc = _dev(inp["x"]), _dev(inp["idx"]), _dev(inp["scales"])
    _, cnt, _, _ = op.dispatch_standard_moe(x, None, sc, idx, num_tokens=inp["ntok"])
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    cdt = workloads.TORCH_DTYPE[wl.combine_dtype]
    # up to 512 distinct seeded rows, repeated over the packed rows, so the
    # oracle quantizes few rows
    g = torch.Generator().manual_seed(sum(tag.encode()) % 10007)
    base = min(512, W * Er * cap)
    if neg_zero:  # every expert output -0.0 (all-zero blocks, sign kept in the codes)
        vb = torch.full((base, H), -0.0, dtype=cdt)
    else:
        vb = (torch.randn((base, H), generator=g)
              * torch.exp(torch.randn((base, 1), generator=g))).to(cdt)
    cb, sb = oracle.quantize_rows(vb.view(torch.int16).numpy().view(np.uint16), dt, ow)
    sel = np.arange(W * Er * cap) % base
    v = vb[torch.from_numpy(sel)]
    codes, scales = cb[sel], sb[sel]
    row, srow = (H, H // 128 * 4) if cw == cra.EP_WIRE_FP8_BLOCK128 else (H // 2, H // 32)
    # the send side on the GPU: only the kept rows of each expert are converted
    yq = torch.zeros((W * Er, cap, row), dtype=torch.uint8, device="cuda")
    ys = torch.zeros((W * Er, cap, srow), dtype=torch.uint8, device="cuda")
    cra.ep_quantize_rows(v.cuda().view(W * Er, cap, H), cw, yq, ys, counts=cnt.view(-1))
    torch.cuda.synchronize()
    gq, gs = yq.cpu().numpy(), ys.cpu().numpy()
    cn = cnt.cpu().numpy().reshape(-1)
    cq = codes.reshape(W * Er, cap, row)
    cs = scales.view(np.uint8).reshape(W * Er, cap, srow)
    for e in range(W * Er):
        n = min(int(cn[e]), cap)
        assert np.array_equal(gq[e, :n], cq[e, :n]), (tag, "quantized rows", e)
        assert np.array_equal(gs[e, :n], cs[e, :n]), (tag, "quantized scales", e)
    w = _dev(inp["w"]) if weighted else None
    out = op.combine_standard_moe(torch.from_numpy(cq.copy()).cuda(), w, idx,
                                  input_scales=torch.from_numpy(cs.copy()).cuda())
    torch.cuda.synchronize()
    # cols: the oracle sees only the first cols columns of every row (and
    # their scale blocks); every column's sums depend on that column alone
    Ho = cols or H
    oc = codes[:, :Ho if cw == cra.EP_WIRE_FP8_BLOCK128 else Ho // 2]
    osc = scales[:, :Ho // 128] if cw == cra.EP_WIRE_FP8_BLOCK128 else scales[:, :Ho // 32]
    ref_y = oracle.expert_combine_wire(W, M, k, Er, cap, Ho, dt, ow, ref["recv"], ref["out_idx"],
                                       np.ascontiguousarray(oc).reshape(W, Er, cap, -1),
                                       np.ascontiguousarray(osc).reshape(W, Er, cap, -1),
                                       w=ref["out_w"] if weighted else None)
    ro, _ = oracle.combine(W, M, k, Ho, dt, inp["ntok"], ref["fwd"], ref_y)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(W):
        T = inp["ntok"][r]
        assert np.array_equal(got[r, :T, :Ho], ro[r, :T]), (tag, "fused wire combine", r)
    op.close()


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("wl_name", ["ep8_t128_h7168_fp8_k8_zipf",
                                     "ep4_ragged1024_h2048_fp16_k64"])
def test_wire_full_size(name, wl_name):
    """Two workloads at full size (the oracle's wire inverse of the headline's
    1.9 G packed elements would take minutes; its wire combines are covered
    by the rank-level wire tests and the bench's checks)."""
    run_standard_wire_case(workloads.WORKLOADS[wl_name], name, weighted=True)


@pytest.mark.parametrize("name", list(WIRES))
def test_wire_headline_first_block(name):
    """The headline at full size in the bench's geometry; the oracle checks the
    first 128 columns of every token (its wire inverse of all 7168 would take
    minutes), the GPU computes whole rows."""
    run_standard_wire_case(workloads.WORKLOADS[workloads.HEADLINE], name, weighted=True,
                           cols=128)


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("cap_div", [1, 1000])
@pytest.mark.parametrize("weighted", [False, True])
def test_wire_signed_zero_with_dropped_ranks(name, cap_div, weighted):
    """The signed-zero case from quantized rows: -0.0 survives the quantizer
    and the decode, and +0 rows of ranks that lost every pair land where the
    two steps put them."""
    run_standard_wire_case(_zero_workload(), name, cap_div=cap_div, weighted=weighted,
                           neg_zero=True, tag=f"std wire {name} -0 /{cap_div} w={weighted}")


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("W,E,k,H,cap_div,weighted", [
    (2, 16, 8, 256, 2, False), (4, 64, 16, 1024, 1, True), (16, 48, 24, 128, 3, True),
    (3, 12, 5, 384, 1000, False)])
def test_wire_shapes_and_drops(name, W, E, k, H, cap_div, weighted):
    wl = workloads.custom(f"stdw_W{W}_E{E}_k{k}_H{H}", W, 40 if W <= 4 else 12, H, k, E, "bf16",
                          ragged=True, seed_index=580 + W + k)
    run_standard_wire_case(wl, name, cap_div=cap_div, weighted=weighted)


@pytest.mark.parametrize("H,k", [(160, 6), (96, 24)])
def test_mxfp4_scale_rows_not_whole_dwords(H, k):
    """MXFP4 at H not a multiple of 128: the scale rows are read by bytes."""
    wl = workloads.custom(f"stdw_mx_H{H}_k{k}", 4, 24, H, k, 32, "bf16", ragged=True,
                          seed_index=590 + k)
    run_standard_wire_case(wl, "mxfp4", cap_div=2, weighted=True)


def _random_standard_case(seed):
    """A seeded random configuration for the fused path, small enough for the
    oracle to finish in well under a second."""
    rng = np.random.default_rng(30_000 + seed)
    W = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 64]))
    k = int(rng.integers(1, 65))
    Er = int(rng.integers(max(1, -(-k // W)), max(1, -(-k // W)) + 6))
    M = int(rng.integers(1, 97)) if W <= 16 else int(rng.integers(1, 13))
    dd = str(rng.choice(["bf16", "fp16", "fp8"]))
    cd = "fp16" if dd == "fp16" else str(rng.choice(["bf16", "fp16"]))
    H = 16 * int(rng.integers(1, 33))
    S = int(rng.integers(1, 20)) if dd == "fp8" and rng.random() < 0.7 else 0
    wl = workloads.custom(f"std_rand{seed}", W, M, H, k, W * Er, dd, cd, scale_dim=S,
                          routing=str(rng.choice(["uniform", "zipf"])) if W * Er >= 2 * k
                          else "uniform", ragged=bool(rng.random() < 0.6),
                          seed_index=700 + seed)
    launch = None
    if rng.random() < 0.7:
        row_vecs = H * (1 if dd == "fp8" else 2) // 16
        launch = dict(expert_waves=int(rng.integers(1, 17)),
                      expert_row_split=int(rng.integers(1, max(2, row_vecs + 1))),
                      expert_combine_waves=int(rng.integers(1, 17)),
                      expert_combine_row_split=int(rng.integers(1, max(2, H * 2 // 16 + 1))),
                      expert_cache_policy=int(rng.integers(0, 3)))
    cap_div, weighted = int(rng.choice([1, 2, 5, 1000])), bool(rng.random() < 0.5)
    if launch is not None:  # drawn last, so the draws above stay as they were
        launch["expert_token_split"] = int(rng.integers(0, 65))
    return wl, launch, cap_div, weighted


@pytest.mark.parametrize("seed", range(48))
def test_random_configurations(seed):
    wl, launch, cap_div, weighted = _random_standard_case(seed)
    run_standard_case(wl, cap_div=cap_div, launch=launch, weighted=weighted,
                      tag=f"std random {seed}")


def test_soak_500_rounds():
    """500 fused dispatch + weighted combine rounds on one plan, alternating two
    inputs, with capacity drops: every round's counts, layout ranges and
    combine output equal the first round's for the same input, bit for bit;
    the first rounds are checked against the oracle."""
    wl = workloads.custom("std_soak_ep4_t96_h512", 4, 96, 512, 8, 64, "bf16", ragged=True,
                          seed_index=590)
    W, M, k, Er, H = _dims(wl)
    inps = [workloads.make_inputs(wl, seed=5000 + i) for i in range(2)]
    refs = [oracle_dispatch(wl, i) for i in inps]
    cap = max(1, min(max_count(wl, r) for r in refs) // 2)
    op = cra.EpDispatchCombineOp(config_of(wl), with_weights=False, expert_capacity=cap)
    dev = [(i["x"].cuda(), i["idx"].cuda(), i["w"].cuda()) for i in inps]
    v = random_outputs(wl, cap, seed=590)
    py = v.cuda()
    _say("[case] fused soak 500 rounds")
    first = [None, None]
    for rnd in range(500):
        j = rnd % 2
        x, idx, w = dev[j]
        ntok = inps[j]["ntok"]
        _, cnt, _, lr = op.dispatch_standard_moe(x, None, None, idx, num_tokens=ntok)
        out = op.combine_standard_moe(py, w, idx)
        # rows t < T_r only: the others keep whatever the other input left
        got = (cnt.clone(), lr.clone(),
               *[out[r, :ntok[r]].view(torch.int16).clone() for r in range(W)])
        if first[j] is None:
            first[j] = got
        elif rnd % 7 == 0 or rnd >= 490:
            assert all(torch.equal(a, b) for a, b in zip(got, first[j])), ("fused soak", rnd)
    torch.cuda.synchronize()
    py16 = v.view(torch.int16).numpy().view(np.uint16)
    for j in range(2):
        ref = refs[j]
        ref_ex = oracle.expert_layout(W, M, k, Er, cap, ref["recv"], ref["src_pos"], ref["out_x"],
                                      ref["out_idx"], ref["out_scales"], fill=SENTINEL_INT)
        assert np.array_equal(first[j][0].cpu().numpy(), ref_ex["count"]), ("soak count", j)
        assert np.array_equal(first[j][1].cpu().numpy(), ref_ex["layout_range"]), ("soak lr", j)
        ref_y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, ref["recv"],
                                      ref["out_idx"], py16, w=ref["out_w"])
        ro, _ = oracle.combine(W, M, k, H, oracle.BF16, inps[j]["ntok"], ref["fwd"], ref_y)
        for r in range(W):
            T = inps[j]["ntok"][r]
            g = first[j][2 + r].cpu().numpy().view(np.uint16)
            assert np.array_equal(g, ro[r, :T]), ("soak combine", j, r)
    op.close()
