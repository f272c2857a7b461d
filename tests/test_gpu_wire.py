"""GPU parity of the quantized combine wire, through the C ABI.

The wire formats (FP8 E4M3 with FP32 scales per 128 elements; MXFP4) follow
the OCP OFP8 and MX v1.0 specifications, as the oracle does; the pages name
fp8_blockwise and fp4 with e8m0 scales ("gfx1250 EPv2: ..." PR 726; "MORI-EP
User Guide", section 10). Every comparison is bit for bit: codes and scales
of ep_quantize_rows against the oracle's quantizer, every in-range bf16
value through the element conversions, and the combine from wire rows (the
oracle's own quantized rows, uploaded) against the oracle's combine.
"""
import numpy as np
import pytest
import torch

import combine_route_amd as cra
import oracle
import workloads

from test_gpu_parity import _say, compare_dispatch, gpu_dispatch, oracle_dispatch

pytestmark = pytest.mark.gpu

WIRES = {"fp8_block128": (cra.EP_WIRE_FP8_BLOCK128, oracle.WIRE_FP8_BLOCK128),
         "mxfp4": (cra.EP_WIRE_MXFP4, oracle.WIRE_MXFP4)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cra.load()


def rows_of(seed, n, H, dtype, spread=4.0):
    """Rows with magnitudes spread over many binades per 32-element group,
    some all-zero groups and some tiny (subnormal-range) ones."""
    g = torch.Generator().manual_seed(seed)
    mag = torch.exp(torch.randn((n, H // 32, 1), generator=g) * spread)
    v = torch.randn((n, H // 32, 32), generator=g) * mag
    v[:, ::7] = 0.0
    v[:, 3::11] *= 1e-38
    return v.reshape(n, H).to(dtype)


def gpu_quantize(v, wire):
    n, H = v.shape
    if wire == cra.EP_WIRE_FP8_BLOCK128:
        out = torch.empty((n, H), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, H // 128), dtype=torch.float32, device="cuda")
    else:
        out = torch.empty((n, H // 2), dtype=torch.uint8, device="cuda")
        sc = torch.empty((n, H // 32), dtype=torch.uint8, device="cuda")
    cra.ep_quantize_rows(v.cuda(), wire, out, sc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), sc.cpu().numpy()


def words(v):
    return v.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("n,H", [(1, 128), (5, 384), (33, 1024), (300, 7168)])
def test_quantize_matches_oracle(name, dtype, n, H):
    cw, ow = WIRES[name]
    _say(f"[case] quantize {name} {dtype} n={n} H={H}")
    v = rows_of(n * 7 + H, n, H, dtype, spread=2.0 if dtype == torch.float16 else 4.0)
    got_c, got_s = gpu_quantize(v, cw)
    ref_c, ref_s = oracle.quantize_rows(words(v), oracle.BF16 if dtype == torch.bfloat16
                                        else oracle.FP16, ow)
    assert np.array_equal(got_c, ref_c)
    assert np.array_equal(got_s.view(np.uint8), ref_s.view(np.uint8))


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("G,R,H,counts", [
    (3, 40, 7168, [0, 40, 17]),     # two pieces a row; an empty and a full group
    (4, 9, 2048, [9, 1, 100, -3]),  # a count past the group and a negative one
    (2, 130, 128, [129, 64]),
])
def test_quantize_with_row_counts(name, dtype, G, R, H, counts):
    """Only the first counts[g] rows of each group are converted; every other
    byte of the outputs keeps its previous value."""
    cw, ow = WIRES[name]
    _say(f"[case] quantize counts {name} {dtype} G={G} R={R} H={H} {counts}")
    v = rows_of(G * R + H, G * R, H, dtype, spread=2.0 if dtype == torch.float16 else 4.0)
    row, srow = (H, H // 128 * 4) if cw == cra.EP_WIRE_FP8_BLOCK128 else (H // 2, H // 32)
    out = torch.full((G, R, row), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((G, R, srow), 0x5A, dtype=torch.uint8, device="cuda")
    cnt = torch.tensor(counts, dtype=torch.int32, device="cuda")
    cra.ep_quantize_rows(v.reshape(G, R, H).cuda(), cw, out, sc, counts=cnt)
    torch.cuda.synchronize()
    got_c, got_s = out.cpu().numpy(), sc.cpu().numpy()
    ref_c, ref_s = oracle.quantize_rows(words(v), oracle.BF16 if dtype == torch.bfloat16
                                        else oracle.FP16, ow)
    ref_c = ref_c.reshape(G, R, row)
    ref_s = ref_s.view(np.uint8).reshape(G, R, srow)
    for g, c in enumerate(counts):
        keep = min(max(c, 0), R)
        assert np.array_equal(got_c[g, :keep], ref_c[g, :keep])
        assert np.array_equal(got_s[g, :keep], ref_s[g, :keep])
        assert (got_c[g, keep:] == 0xA5).all() and (got_s[g, keep:] == 0x5A).all()


def test_e4m3_conversion_of_every_in_range_bf16_value():
    """Blocks whose largest magnitude is 448 have scale 1: each code is then
    the direct E4M3 conversion of the bf16 value itself."""
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    keep = torch.isfinite(v) & (v.float().abs() < 448)
    vals = v[keep]
    nb = -(-vals.numel() // 127)
    blocks = torch.zeros((nb, 128), dtype=torch.bfloat16)
    blocks[:, 0] = 448.0
    flat = blocks[:, 1:].reshape(-1)
    flat[:vals.numel()] = vals
    blocks[:, 1:] = flat.reshape(nb, 127)
    rows = blocks.reshape(-1, 1024) if nb % 8 == 0 else blocks.reshape(nb, 128)
    got_c, got_s = gpu_quantize(rows, cra.EP_WIRE_FP8_BLOCK128)
    assert (got_s == 1.0).all()
    ref = oracle.cast_to_e4m3(words(rows), oracle.BF16)
    assert np.array_equal(got_c, ref)


def test_e2m1_conversion_of_every_bf16_value_below_8():
    """Blocks whose largest magnitude is 4 have scale 2^0: each code is then
    the E2M1 conversion of the value itself."""
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    keep = torch.isfinite(v) & (v.float().abs() <= 4)
    vals = v[keep]
    nb = -(-vals.numel() // 31)
    blocks = torch.zeros((nb, 32), dtype=torch.bfloat16)
    blocks[:, 0] = 4.0
    flat = blocks[:, 1:].reshape(-1)
    flat[:vals.numel()] = vals
    blocks[:, 1:] = flat.reshape(nb, 31)
    got_c, got_s = gpu_quantize(blocks, cra.EP_WIRE_MXFP4)
    assert (got_s == 127).all()
    ref_c, _ = oracle.quantize_rows(words(blocks), oracle.BF16, oracle.WIRE_MXFP4)
    assert np.array_equal(got_c, ref_c)


def run_wire_case(wl, name, launch=None, with_weights=True, tag=None, ntok=None):
    cw, ow = WIRES[name]
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
    tag = tag or f"{wl.name} {name}"
    _say(f"[case] wire combine {tag}: W={W} M={M} H={H} k={k} launch={launch} ntok={ntok}")
    inp = workloads.make_inputs(wl)
    if ntok is not None:
        inp["ntok"] = list(ntok)
    if not with_weights:
        inp["w"] = None
    ref = oracle_dispatch(wl, inp)
    cfg = cra.make_config(W, H, M, wl.experts_per_rank, k, wl.dispatch_dtype, wl.combine_dtype,
                          scale_dim=wl.scale_dim, scale_type_size=4, combine_wire=cw)
    op = cra.EpDispatchCombineOp(cfg, with_weights=with_weights)
    if launch:
        op.set_launch(launch)
    gpu_dispatch(op, inp)
    torch.cuda.synchronize()
    compare_dispatch(wl, op, ref, tag)
    # expert outputs: up to 4096 seeded bf16/fp16 rows quantized by the
    # oracle, repeated over the [W][W*M] rows
    cdt = workloads.TORCH_DTYPE[wl.combine_dtype]
    base = min(4096, W * W * M)
    yb = rows_of(W * M + H, base, H, cdt, spread=2.0 if cdt == torch.float16 else 4.0)
    assert torch.isfinite(yb).all()                  # the wire takes finite rows
    cb, sb = oracle.quantize_rows(words(yb), oracle.BF16 if wl.combine_dtype == "bf16"
                                  else oracle.FP16, ow)
    sel = np.arange(W * W * M) % base
    codes, scales = cb[sel], sb[sel]
    yq = torch.from_numpy(codes.reshape(W, W * M, -1)).cuda()
    ys = torch.from_numpy(scales.reshape(W, W * M, -1)).cuda()
    yw = None if ref["out_w"] is None else torch.from_numpy(ref["out_w"]).cuda()
    out, out_w = op.combine(yq, yw, y_scales=ys)
    torch.cuda.synchronize()
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    ro = oracle.combine_wire(W, M, k, H, dt, ow, inp["ntok"], ref["fwd"],
                             codes.reshape(W, W * M, -1), scales.reshape(W, W * M, -1))
    g = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(W):
        T = inp["ntok"][r]
        assert np.array_equal(g[r, :T], ro[r, :T]), (tag, "wire combine", r)
    if yw is not None:
        # the weight sums do not depend on the payload: an 8-wide dummy
        _, rw = oracle.combine(W, M, k, 8, dt, inp["ntok"], ref["fwd"],
                               np.zeros((W, W * M, 8), np.uint16), ref["out_w"])
        gw = out_w.cpu().numpy().view(np.uint32)
        for r in range(W):
            T = inp["ntok"][r]
            assert np.array_equal(gw[r, :T], rw[r, :T].view(np.uint32)), (tag, "weights", r)
    op.close()


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("wl_name", ["ep8_t4096_h7168_bf16_k8", "ep8_t128_h7168_fp8_k8_zipf",
                                     "ep4_ragged1024_h2048_fp16_k64"])
def test_wire_combine_full_size(name, wl_name):
    run_wire_case(workloads.WORKLOADS[wl_name], name)


@pytest.mark.parametrize("name", list(WIRES))
def test_wire_combine_large_ragged_call(name):
    """A large call (waves numbered token by token with the piece fastest,
    pieces of about 1.75 KB of codes, 4 waves a block), ragged ranks, and a
    row of 41 FP8 scale blocks (2 pieces of 168 and 160 16-element units)."""
    wl = workloads.custom("wire_large_ragged_ep8_h5248", 8, 4096, 5248, 8, 256, "bf16",
                          seed_index=534)
    run_wire_case(wl, name, ntok=[4096, 3001, 4095, 2048, 4096, 3333, 4000, 1])


@pytest.mark.parametrize("name", list(WIRES))
@pytest.mark.parametrize("W,k,H", [(1, 1, 128), (2, 2, 256), (3, 9, 384), (16, 8, 1024),
                                   (64, 64, 128)])
def test_wire_combine_shapes(name, W, k, H):
    M = 40 if W <= 16 else 6
    wl = workloads.custom(f"wire_W{W}_k{k}_H{H}", W, M, H, k, max(k, W * 4), "bf16",
                          ragged=True, seed_index=800 + W + k)
    run_wire_case(wl, name, with_weights=W % 2 == 0)


@pytest.mark.parametrize("W,k,H", [(2, 2, 32), (3, 9, 160), (4, 16, 1184), (16, 24, 96)])
def test_mxfp4_combine_scale_rows_not_whole_dwords(W, k, H):
    """MXFP4 takes any H that is a multiple of 32: with H / 32 scale bytes a
    row not a multiple of 4, the scale rows are read byte by byte; k > 8
    rows a token also reloads them per group of rows."""
    M = 40 if W <= 4 else 6
    wl = workloads.custom(f"wire_mx_W{W}_k{k}_H{H}", W, M, H, k, max(k, W * 4), "bf16",
                          ragged=True, seed_index=840 + W + k)
    run_wire_case(wl, "mxfp4", with_weights=True)


@pytest.mark.parametrize("launch", [dict(combine_waves=1, combine_row_split=3),
                                    dict(combine_waves=16, cache_policy=cra.EP_CACHE_STREAM),
                                    dict(combine_row_split=7, cache_policy=cra.EP_CACHE_KEEP)])
def test_wire_geometry_does_not_change_results(launch):
    wl = workloads.custom("wire_geom_ep4_t200_h1024", 4, 200, 1024, 8, 64, "bf16", ragged=True,
                          seed_index=820)
    for name in WIRES:
        run_wire_case(wl, name, launch=launch, tag=f"geom {name} {launch}")


@pytest.mark.parametrize("name", list(WIRES))
def test_wire_decode_of_every_code(name):
    """One token with one contribution whose codes are all 256 byte values
    (FP8: scale 1 and another power of two; MXFP4: several scale codes):
    the combine's output is each decoded value, exact in bf16; the FP8 NaN
    codes must come out NaN."""
    cw, ow = WIRES[name]
    H = 512
    wl = workloads.custom(f"wire_codes_{name}", 1, 1, H, 1, 4, "bf16", seed_index=830)
    inp = workloads.make_inputs(wl)
    inp["ntok"] = [1]
    ref = oracle_dispatch(wl, inp)
    cfg = cra.make_config(1, H, 1, 4, 1, "bf16", "bf16", combine_wire=cw)
    op = cra.EpDispatchCombineOp(cfg, with_weights=False)
    gpu_dispatch(op, dict(inp, w=None))
    codes = np.tile(np.arange(256, dtype=np.uint8), 2)
    if cw == cra.EP_WIRE_FP8_BLOCK128:
        y = codes.reshape(1, 1, H)
        ys = np.array([1.0, 1.0, 2.0 ** -3, 2.0 ** 5], np.float32).reshape(1, 1, 4)
    else:
        y = codes[:H // 2].reshape(1, 1, H // 2)
        ys = np.array([127, 100, 150, 120, 127, 131, 90, 140, 127, 126, 128, 127, 127, 110, 145,
                       127], np.uint8).reshape(1, 1, H // 32)
    out, _ = op.combine(torch.from_numpy(y).cuda(), None, y_scales=torch.from_numpy(ys).cuda())
    torch.cuda.synchronize()
    ro = oracle.combine_wire(1, 1, 1, H, oracle.BF16, ow, [1], ref["fwd"], y, ys)
    g = out.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0]
    r = ro[0, 0]
    nan_g = (g & 0x7F80) == 0x7F80
    nan_g &= (g & 0x7F) != 0
    nan_r = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_r)
    assert np.array_equal(g[~nan_g], r[~nan_r])
    op.close()


@pytest.mark.parametrize("name", list(WIRES))
def test_wire_decode_of_every_scale(name):
    """Every scale a quantizer of finite inputs can write, each on its own
    block, through the combine's decoder: MXFP4 E8M0 codes 0 to 254 (code 0
    is 2^-127, a subnormal FP32 scale) over all 256 byte values of element
    codes; FP8 block-128 scales 2^-149 (the smallest subnormal) to 2^127 and
    subnormal, normal and odd-significand values. Bit for bit against the
    oracle's decode (NaN codes: any NaN)."""
    cw, ow = WIRES[name]
    if cw == cra.EP_WIRE_MXFP4:
        H = 32 * 255
        ys = np.arange(255, dtype=np.uint8).reshape(1, 1, H // 32)
        y = np.tile(np.arange(256, dtype=np.uint8), H // 2 // 256 + 1)[:H // 2].reshape(1, 1, H // 2)
    else:
        e = np.arange(-149, 128, 4)
        sc = np.concatenate([np.ldexp(1.0, e), np.ldexp(1.5, e[::3]), [3.0e-39, 1.17e-38, 0.7,
                                                                      1.2345678]])
        H = 128 * len(sc)
        ys = sc.astype(np.float32).reshape(1, 1, len(sc))
        y = np.tile(np.arange(256, dtype=np.uint8), H // 256 + 1)[:H].reshape(1, 1, H)
    _say(f"[case] every scale {name} H={H}")
    wl = workloads.custom(f"wire_scales_{name}", 1, 1, H, 1, 4, "bf16", seed_index=833)
    inp = workloads.make_inputs(wl)
    inp["ntok"] = [1]
    ref = oracle_dispatch(wl, inp)
    cfg = cra.make_config(1, H, 1, 4, 1, "bf16", "bf16", combine_wire=cw)
    op = cra.EpDispatchCombineOp(cfg, with_weights=False)
    gpu_dispatch(op, dict(inp, w=None))
    out, _ = op.combine(torch.from_numpy(np.ascontiguousarray(y)).cuda(), None,
                        y_scales=torch.from_numpy(np.ascontiguousarray(ys)).cuda())
    torch.cuda.synchronize()
    ro = oracle.combine_wire(1, 1, 1, H, oracle.BF16, ow, [1], ref["fwd"], y, ys)
    g = out.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0]
    r = ro[0, 0]
    nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    nan_r = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_r)
    assert np.array_equal(g[~nan_g], r[~nan_r])
    op.close()


def test_graph_replay_of_dispatch_quantize_and_wire_combine():
    """Dispatch, the send-side quantizer over the received rows (row counts on
    the device) and the MXFP4 wire combine captured in one HIP graph;
    replayed with new inputs, with eager work in between; every replay
    equals the oracle."""
    wl = workloads.custom("wire_graph_ep4_t96_h512", 4, 96, 512, 8, 64, "bf16", seed_index=850)
    W, M, k, H = wl.world_size, wl.max_tokens, wl.topk, wl.hidden
    cw, ow = WIRES["mxfp4"]
    cfg = cra.make_config(W, H, M, wl.experts_per_rank, k, "bf16", "bf16", combine_wire=cw)
    op = cra.EpDispatchCombineOp(cfg)
    inp0 = workloads.make_inputs(wl)
    x, idx, w = inp0["x"].cuda(), inp0["idx"].cuda(), inp0["w"].cuda()
    ntok = inp0["ntok"]
    yq = torch.zeros((W, W * M, H // 2), dtype=torch.uint8, device="cuda")
    ys = torch.zeros((W, W * M, H // 32), dtype=torch.uint8, device="cuda")

    def step():
        op.dispatch(ntok, x, idx, w)
        cra.ep_quantize_rows(op.out_x, cw, yq, ys, counts=op.recv_num_token)
        op.combine(yq, op.out_weights, y_scales=ys)

    _say("[case] wire graph capture")
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
        inp = workloads.make_inputs(wl, seed=3000 + rep)
        inp["ntok"] = ntok
        x.copy_(inp["x"])
        idx.copy_(inp["idx"])
        w.copy_(inp["w"])
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle_dispatch(wl, inp)
        # the oracle's quantizer over the oracle's received rows (identity experts)
        rows = ref["out_x"].view(np.uint16).reshape(W * W * M, H)
        codes, scales = oracle.quantize_rows(rows, oracle.BF16, ow)
        ro = oracle.combine_wire(W, M, k, H, oracle.BF16, ow, ntok, ref["fwd"],
                                 codes.reshape(W, W * M, -1), scales.reshape(W, W * M, -1))
        got = op.combine_out.view(torch.int16).cpu().numpy().view(np.uint16)
        for r in range(W):
            assert np.array_equal(got[r, :ntok[r]], ro[r, :ntok[r]]), ("wire graph", rep, r)
        del junk
    op.close()
