"""The entry point that allocates nothing (ep_plan_static: a plan over the
library's static scratch) against the one that takes a caller's workspace
(ep_plan_create): the same dispatch and combine through each, on two calls
in a row, the second smaller, compared byte for byte: receive counts,
received payload, id, weight and scale rows, src_token_pos, and the
combine's rows and weights. Also the same static plan reused after a
destroy."""
import ctypes

import numpy as np
import pytest
import torch

import combine_route_amd as cra
import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run(plan, cfg, wl, inp, y_from_out):
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
    WM = W * M
    eb = workloads.ELEM_BYTES[wl.dispatch_dtype]
    dev = torch.device("cuda")
    sts = 4 if wl.scale_dim else 0
    out = dict(
        out_x=torch.zeros((W, WM, H * eb), dtype=torch.uint8, device=dev),
        out_idx=torch.full((W, WM, k), -7, dtype=torch.int32, device=dev),
        out_w=torch.zeros((W, WM, k), dtype=torch.float32, device=dev),
        out_sc=(torch.zeros((W, WM, wl.scale_dim * sts), dtype=torch.uint8, device=dev)
                if wl.scale_dim else None),
        recv=torch.zeros(W, dtype=torch.int32, device=dev),
        comb=torch.zeros((W, M, H), dtype=workloads.TORCH_DTYPE[wl.combine_dtype], device=dev),
        comb_w=torch.zeros((W, M, k), dtype=torch.float32, device=dev))
    x, idx, w = inp["x"].to(dev), inp["idx"].to(dev), inp["w"].to(dev)
    sc = None if inp["scales"] is None else inp["scales"].view(torch.uint8).to(dev)
    cra.ep_dispatch(plan, cfg, inp["ntok"], x, idx, w, sc, out["out_x"], out["out_idx"],
                    out["out_w"], out["out_sc"], out["recv"])
    y = out["out_x"] if y_from_out else torch.randn(
        (W, WM, H), generator=torch.Generator().manual_seed(5)).to(
            workloads.TORCH_DTYPE[wl.combine_dtype]).to(dev)
    cra.ep_combine(plan, cfg, y, out["out_w"], out["comb"], out["comb_w"])
    torch.cuda.synchronize()
    # the plan's src_token_pos, copied out of its workspace (device to device)
    src = _from_device_ptr(cra.ep_get_src_token_pos(plan, 0), W * WM * 4).view(torch.int32)
    return out, src.view(W, WM)


def _from_device_ptr(ptr, nbytes):
    """A uint8 device tensor copied from nbytes at device address ptr."""
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert lib.hipMemcpy(dst.data_ptr(), ptr, nbytes, 3) == 0  # device to device
    return dst


def _compare(wl, a, b, tag):
    (oa, sa), (ob, sb) = a, b
    recv = oa["recv"].cpu().numpy()
    assert np.array_equal(recv, ob["recv"].cpu().numpy()), tag
    for d in range(wl.world_size):
        R = int(recv[d])
        for key in ("out_x", "out_idx", "out_w", "out_sc"):
            if oa[key] is None:
                continue
            assert torch.equal(oa[key][d, :R].view(torch.uint8), ob[key][d, :R].view(torch.uint8)), \
                (tag, key, d)
        assert torch.equal(sa[d, :R], sb[d, :R]), (tag, "src_pos", d)
    # combine rows of every rank (rows past a rank's tokens are zero in both)
    assert torch.equal(oa["comb"].view(torch.int16), ob["comb"].view(torch.int16)), \
        (tag, "combine")
    assert torch.equal(oa["comb_w"].view(torch.int32), ob["comb_w"].view(torch.int32)), \
        (tag, "combine weights")


CASES = [
    # the larger call first, then a smaller one on the same static scratch
    workloads.custom("static_ep8_t512_h2048_bf16_k8", 8, 512, 2048, 8, 256, "bf16",
                     seed_index=801),
    workloads.custom("static_ep4_t96_h1024_fp8_k6", 4, 96, 1024, 6, 32, "fp8", "bf16",
                     scale_dim=8, ragged=True, seed_index=802),
]


def test_static_plan_equals_workspace_plan_on_two_calls():
    for i, wl in enumerate(CASES):
        _say(f"[case] static plan call {i}: {wl.name}")
        inp = workloads.make_inputs(wl)
        cfg = cra.make_config(wl.world_size, wl.hidden, wl.max_tokens, wl.experts_per_rank,
                              wl.topk, wl.dispatch_dtype, wl.combine_dtype,
                              scale_dim=wl.scale_dim, scale_type_size=4)
        assert cra.ep_workspace_bytes(cfg) <= cra.EP_STATIC_SCRATCH_BYTES
        ws = torch.empty(cra.ep_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        ref_plan = cra.ep_plan_create(cfg, ws)
        in_place = wl.dispatch_dtype == wl.combine_dtype
        ref = _run(ref_plan, cfg, wl, inp, in_place)
        cra.ep_plan_destroy(ref_plan)
        splan = cra.ep_plan_static(cfg)
        got = _run(splan, cfg, wl, inp, in_place)
        _compare(wl, ref, got, wl.name)
        # the same static plan, destroyed (emptied, not freed) and made again
        cra.ep_plan_destroy(splan)
        assert cra.ep_plan_static(cfg) == splan
        again = _run(splan, cfg, wl, inp, in_place)
        _compare(wl, ref, again, wl.name + " again")
        cra.ep_plan_destroy(splan)
        del ws
