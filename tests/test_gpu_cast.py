"""GPU parity of the dispatch's on-the-fly FP8 cast (fp8_direct_cast, named
by "MORI-EP User Guide" section 10 and "gfx1250 EPv2: ..." PR 726), through
the C ABI: bf16 / fp16 tokens are received as OCP E4M3 codes (round to
nearest even, saturating at 448, NaN -> 0x7F). The oracle casts the inputs
with its own E4M3 encoder and dispatches the codes; every received byte,
id, weight and scale row is compared bit for bit, and one case sends every
16-bit word through the cast.
"""
import numpy as np
import pytest
import torch

import combine_route_amd as cra
import oracle
import workloads

from test_gpu_parity import _say, compare_dispatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cra.load()


def run_cast_case(W, M, H, k, E, src, ntok=None, x=None, launch=None, scale_dim=0, seed=0,
                  tag=None):
    tdt = torch.bfloat16 if src == "bf16" else torch.float16
    wl = workloads.custom(f"cast_W{W}_M{M}_H{H}_k{k}_{src}", W, M, H, k, E, "bf16",
                          ragged=ntok is None, seed_index=900 + seed)
    tag = tag or wl.name
    _say(f"[case] dispatch cast {tag} launch={launch}")
    inp = workloads.make_inputs(wl)
    if ntok is not None:
        inp["ntok"] = ntok
    if x is None:
        g = torch.Generator().manual_seed(seed)
        x = (torch.randn((W, M, H), generator=g) * torch.exp(torch.randn((W, M, 1), generator=g)
                                                              * 3)).to(tdt)
    sc = None
    if scale_dim:
        g = torch.Generator().manual_seed(seed + 1)
        sc = torch.randint(0, 256, (W, M, scale_dim * 4), generator=g, dtype=torch.uint8)
    words = x.view(torch.int16).numpy().view(np.uint16)
    codes = oracle.cast_to_e4m3(words, oracle.BF16 if src == "bf16" else oracle.FP16)
    ref = oracle.dispatch(W, M, k, E // W, inp["ntok"], codes, inp["idx"].numpy(),
                          inp["w"].numpy(), None if sc is None else sc.numpy())
    cfg = cra.make_config(W, H, M, E // W, k, "fp8", "bf16", scale_dim=scale_dim,
                          scale_type_size=4, dispatch_cast=src)
    op = cra.EpDispatchCombineOp(cfg)
    if launch:
        op.set_launch(launch)
    op.dispatch(inp["ntok"], x.cuda(), inp["idx"].cuda(), inp["w"].cuda(),
                None if sc is None else sc.cuda())
    torch.cuda.synchronize()
    compare_dispatch(wl, op, ref, tag)
    op.close()


def test_every_16_bit_word_through_the_cast():
    for src, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        x = torch.from_numpy(w.view(np.int16)).view(tdt).reshape(1, 1, 65536)
        run_cast_case(1, 1, 65536, 1, 4, src, ntok=[1], x=x, tag=f"every {src} word")


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("W,M,H,k,E", [(8, 4096, 7168, 8, 256), (8, 128, 7168, 8, 256),
                                       (2, 16, 256, 2, 8), (4, 300, 2048, 64, 256),
                                       (3, 50, 128, 5, 12), (16, 20, 512, 8, 64)])
def test_cast_dispatch_matches_oracle(src, W, M, H, k, E):
    full = M == 4096
    run_cast_case(W, M, H, k, E, src, ntok=[M] * W if full else None, seed=W + k + H)


@pytest.mark.parametrize("launch", [dict(dispatch_row_split=5, dispatch_waves=3),
                                    dict(tile_tokens=64, layout=cra.EP_LAYOUT_SCAN_IN_COPY),
                                    dict(layout=cra.EP_LAYOUT_KERNELS,
                                         cache_policy=cra.EP_CACHE_STREAM),
                                    dict(tile_tokens=64, dispatch_token_split=8,
                                         dispatch_row_split=2),
                                    dict(tile_tokens=16, dispatch_token_split=3,
                                         dispatch_waves=5)])
def test_cast_geometry_and_scales(launch):
    run_cast_case(4, 200, 1024, 8, 64, "bf16", launch=launch, scale_dim=8, seed=31,
                  tag=f"cast geometry {launch}")


@pytest.mark.parametrize("src", ["bf16", "fp16"])
@pytest.mark.parametrize("W,M,H,k,E,cap_div,scale_dim", [
    (8, 4096, 7168, 8, 256, 1, 0),     # the headline, nothing dropped
    (4, 300, 2048, 64, 256, 2, 0),     # top-64, pairs dropped
    (3, 50, 128, 5, 12, 3, 2),         # scale rows, few experts
    (16, 20, 512, 8, 64, 1, 0),
])
def test_fused_cast_dispatch_matches_oracle(src, W, M, H, k, E, cap_div, scale_dim):
    """dispatch_standard_moe with a cast config: the packed rows hold the E4M3
    codes of the cast (the oracle's cast, dispatch and expert layout)."""
    from test_gpu_expert import SENTINEL_INT, _fill_outputs, compare_layout
    tdt = torch.bfloat16 if src == "bf16" else torch.float16
    wl = workloads.custom(f"fcast_W{W}_M{M}_H{H}_k{k}_{src}", W, M, H, k, E, "bf16",
                          ragged=True, seed_index=950 + W + k)
    _say(f"[case] fused cast dispatch {wl.name} cap/{cap_div} scales={scale_dim}")
    inp = workloads.make_inputs(wl)
    g = torch.Generator().manual_seed(W * 31 + k)
    x = (torch.randn((W, M, H), generator=g) * torch.exp(torch.randn((W, M, 1), generator=g)
                                                          * 3)).to(tdt)
    sc = None
    if scale_dim:
        sc = torch.randint(0, 256, (W, M, scale_dim * 4), generator=g, dtype=torch.uint8)
    words = x.view(torch.int16).numpy().view(np.uint16)
    codes = oracle.cast_to_e4m3(words, oracle.BF16 if src == "bf16" else oracle.FP16)
    ref = oracle.dispatch(W, M, k, E // W, inp["ntok"], codes, inp["idx"].numpy(), None,
                          None if sc is None else sc.numpy())
    full = oracle.expert_layout(W, M, k, E // W, 1, ref["recv"], ref["src_pos"],
                                ref["out_x"][:, :, :16], ref["out_idx"])
    cap = max(1, int(full["count"].max()) // cap_div)
    ref_ex = oracle.expert_layout(W, M, k, E // W, cap, ref["recv"], ref["src_pos"],
                                  ref["out_x"], ref["out_idx"], ref["out_scales"],
                                  fill=SENTINEL_INT)
    cfg = cra.make_config(W, H, M, E // W, k, "fp8", "bf16", scale_dim=scale_dim,
                          scale_type_size=4, dispatch_cast=src)
    op = cra.EpDispatchCombineOp(cfg, with_weights=False, expert_capacity=cap)
    ex = op._expert_state()
    _fill_outputs(ex)
    op.dispatch_standard_moe(x.cuda(), None, None if sc is None else sc.cuda(),
                             inp["idx"].cuda(), num_tokens=inp["ntok"])
    torch.cuda.synchronize()
    compare_layout(wl, cap, op, ref_ex, wl.name)
    op.close()
