"""Pins for the oracle's quantized wires: E4M3 and E2M1 conversions, FP8
block-128 and MXFP4 row quantization, and the combine from wire rows.

The pages name fp8_direct_cast, fp8_blockwise and fp4 with e8m0 scales
("gfx1250 EPv2: ..." PR 726; "MORI-EP User Guide", section 10) without
defining them; the oracle follows the formats' published specifications
(OCP OFP8 for E4M3, OCP MX v1.0 for E2M1, E8M0 and the MX conversion), with
the readings listed in its header.

Pins, none of which calls the oracle through itself:
* E4M3 decoding of all 256 codes against torch's float8_e4m3fn, and the
  specification's landmarks (448, 2^-6, 2^-9, NaN codes);
* E4M3 encoding of every bf16 and every fp16 word against torch's
  float8_e4m3fn conversion wherever that is finite (|v| <= 448), and
  saturation / NaN handling by hand beyond;
* E2M1 values equal the specification's list, and hand-derived ties;
* FP8 block-128: scale within one ulp of amax / 448, the largest element at
  the largest code, every element within half a step of the code grid; and
  bit for bit, computed in torch from the reading's arithmetic: scale =
  fl32(amax / 448), code = E4M3(fl32(v * fl32(448 / amax))) by torch's
  float8_e4m3fn conversion (round to nearest even);
* MXFP4: the block's largest magnitude lands in [4, 8) after scaling, every
  element within half a step of the E2M1 grid or saturated;
* combine from wire rows equals the plain combine of the dequantized rows
  whenever those are exact in bf16 (power-of-two scales).
"""
import numpy as np
import pytest
import torch

import oracle

E4M3 = torch.float8_e4m3fn


def test_e4m3_decode_matches_torch_and_the_specification():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(E4M3).float().numpy()
    got = np.array([oracle.e4m3_to_f32(c) for c in codes], np.float32)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert set(np.flatnonzero(np.isnan(got))) == {0x7F, 0xFF}
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0


@pytest.mark.parametrize("dtype,tdt", [(oracle.BF16, torch.bfloat16), (oracle.FP16, torch.float16)])
def test_e4m3_direct_cast_of_every_16_bit_word(dtype, tdt):
    words = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.cast_to_e4m3(words, dtype)
    v = torch.from_numpy(words.view(np.int16)).view(tdt).float()
    finite = torch.isfinite(v) & (v.abs() <= 448)
    ref = v[finite].to(E4M3).view(torch.uint8).numpy()
    assert np.array_equal(got[finite.numpy()], ref)
    vn = v.numpy()
    big = np.isfinite(vn) & (np.abs(vn) > 448) | np.isinf(vn)
    assert (got[big & (vn > 0)] == 0x7E).all() and (got[big & (vn < 0)] == 0xFE).all()
    assert (got[np.isnan(vn)] == 0x7F).all()


def test_e2m1_values_and_ties():
    assert [oracle.e2m1_to_f32(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [oracle.e2m1_to_f32(c) for c in range(8, 16)] == [-0.0, -0.5, -1, -1.5, -2, -3, -4,
                                                             -6]
    # ties go to the even code (0.0, 1.0, 2.0, 4.0 have even codes)
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6, 0.3: 1, 2.6: 5,
             5.1: 7, 7.0: 7, 1e9: 7, -0.25: 8, -5.0: 14, -7.5: 15}
    for v, c in cases.items():
        assert oracle.f32_to_e2m1(v) == c, v


def _rows(seed, n, H, dtype=torch.bfloat16, spread=3.0):
    g = torch.Generator().manual_seed(seed)
    v = torch.randn((n, H), generator=g) * torch.exp(torch.randn((n, H // 32, 1), generator=g)
                                                     * spread).repeat_interleave(32, 1)[..., 0]
    v = v.to(dtype)
    return v, v.view(torch.int16).numpy().view(np.uint16)


def _e4m3_step(a):
    """Distance between neighbouring E4M3 values at magnitude a (a <= 448)."""
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


def test_fp8_block128_scale_codes_and_error_bound():
    v, words = _rows(1, 16, 1024)
    codes, scales = oracle.quantize_rows(words, oracle.BF16, oracle.WIRE_FP8_BLOCK128)
    vd = v.double().numpy().reshape(16, 8, 128)
    amax = np.abs(vd).max(-1)
    s = scales.astype(np.float64)
    assert np.all(np.abs(s - amax / 448) <= np.spacing(np.float32(amax / 448)))
    dec = torch.from_numpy(codes).view(E4M3).double().numpy().reshape(16, 8, 128)
    # the largest element of every block takes the largest code
    arg = np.abs(vd).argmax(-1)
    assert np.all(np.abs(np.take_along_axis(dec, arg[..., None], -1)) == 448)
    # every element within half a grid step (plus the scale's rounding)
    scaled = vd * (448 / amax)[..., None]
    err = np.abs(dec - scaled)
    assert np.all(err <= _e4m3_step(np.abs(scaled)) / 2 * (1 + 1e-6) + np.abs(scaled) * 2e-7)


def _fp8_block128_torch(v):
    """The FP8 block-128 wire computed in torch, independently of the oracle:
    per block of 128, amax = max |v| in FP32, scale = fl32(amax / 448) and
    r = fl32(448 / amax) (both 1 for an all-zero block), code = E4M3 of the
    FP32 product v * r. Returns (codes uint8 [n, H], scales float32 [n, H/128])."""
    n, H = v.shape
    b = v.float().reshape(n, H // 128, 128)
    amax = b.abs().amax(-1, keepdim=True)
    zero = amax == 0
    f448 = torch.tensor(448.0, dtype=torch.float32)
    s = torch.where(zero, torch.ones_like(amax), amax / f448)
    r = torch.where(zero, torch.ones_like(amax), f448 / amax.clamp(min=torch.finfo(torch.float32).tiny))
    q = (b * r).to(E4M3).view(torch.uint8).reshape(n, H)
    return q.numpy(), s.reshape(n, H // 128).numpy()


@pytest.mark.parametrize("dtype,seed,spread", [(torch.bfloat16, 21, 3.0),
                                               (torch.bfloat16, 22, 8.0),
                                               (torch.float16, 23, 1.5)])
def test_fp8_block128_bit_exact_against_torch(dtype, seed, spread):
    """Codes and scales bit for bit. The blocks mix binades (a factor up to
    e^(3 spread) between 32-element groups), so scaled values fall on E4M3
    normals, subnormals and zero; some blocks are all zero, some hold -0.0,
    and one holds a single nonzero element. A quantizer that divides by the
    scale instead of multiplying by fl32(448 / amax), or that rounds the scale
    differently, changes codes here."""
    v, _ = _rows(seed, 64, 1024, dtype=dtype, spread=spread)
    v = v.clone()
    v[0, :128] = 0.0
    v[1, 128:256] = -0.0
    v[2, 256:384] = 0.0
    v[2, 300] = 3.0
    v[3, 384:512] *= 2.0 ** -20 if dtype == torch.bfloat16 else 1.0
    words = v.view(torch.int16).numpy().view(np.uint16)
    dt = oracle.BF16 if dtype == torch.bfloat16 else oracle.FP16
    codes, scales = oracle.quantize_rows(words, dt, oracle.WIRE_FP8_BLOCK128)
    want_codes, want_scales = _fp8_block128_torch(v)
    assert np.array_equal(scales.view(np.uint32), want_scales.view(np.uint32))
    assert np.array_equal(codes, want_codes)
    assert np.all(codes[1, 128:256] == 0x80)          # -0.0 keeps its sign


def test_fp8_block128_all_zero_block():
    words = np.zeros((2, 256), np.uint16)
    codes, scales = oracle.quantize_rows(words, oracle.BF16, oracle.WIRE_FP8_BLOCK128)
    assert not codes.any() and (scales == 1.0).all()


def test_mxfp4_scale_range_and_grid():
    v, words = _rows(2, 16, 1024)
    codes, scales = oracle.quantize_rows(words, oracle.BF16, oracle.WIRE_MXFP4)
    vd = v.double().numpy().reshape(16, 32, 32)
    amax = np.abs(vd).max(-1)
    X = 2.0 ** (scales.astype(np.float64) - 127)
    assert np.all((amax / X >= 4) & (amax / X < 8))
    lo, hi = codes & 0xF, codes >> 4
    nib = np.stack([lo, hi], -1).reshape(16, 32, 32)
    grid = np.array([oracle.e2m1_to_f32(c) for c in range(16)])
    q = grid[nib]
    u = vd / X[..., None]
    a = np.abs(u)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    inside = a <= 6
    assert np.all(np.abs(q - u)[inside] <= step[inside] / 2)
    assert np.all(np.abs(q[~inside]) == 6)


def test_mxfp4_all_zero_block_and_packing():
    words = np.zeros((1, 64), np.uint16)
    words[0, 33] = 0x3F80                     # 1.0 in the second block, odd element
    codes, scales = oracle.quantize_rows(words, oracle.BF16, oracle.WIRE_MXFP4)
    assert scales[0, 0] == 0                  # all-zero block: E8M0 code 0
    assert scales[0, 1] == 127 - 2            # 1.0 lands at 4.0 = 2^2 * 1.0
    assert codes[0, 16] == 0x60               # element 33: high nibble of byte 16, 4.0
    assert not np.delete(codes[0], 16).any()


def _identity_layout(W, M, k, E, seed):
    import workloads
    wl = workloads.custom(f"wire_ep{W}_t{M}", W, M, 256, k, E, "bf16", seed_index=seed)
    inp = workloads.make_inputs(wl)
    disp = oracle.dispatch(W, M, k, E // W, inp["ntok"], inp["x"].view(torch.uint8).numpy(),
                           inp["idx"].numpy())
    return wl, inp, disp


@pytest.mark.parametrize("wire", [oracle.WIRE_FP8_BLOCK128, oracle.WIRE_MXFP4])
def test_combine_from_wire_equals_combine_of_exact_dequantized_rows(wire):
    W, M, k, E, H = 4, 32, 6, 24, 256
    wl, inp, disp = _identity_layout(W, M, k, E, 700 + wire)
    v, words = _rows(3, W * W * M, H)
    if wire == oracle.WIRE_FP8_BLOCK128:
        # a power-of-two scale: one element per block at 448 * 2^j
        g = torch.Generator().manual_seed(4)
        j = torch.randint(-4, 4, (W * W * M, H // 128), generator=g)
        vv = v.float().reshape(-1, H // 128, 128).clamp(-1, 1) * 0.999 * (448 * 2.0 ** j[..., None])
        vv[..., 0] = 448 * 2.0 ** j
        v = vv.reshape(-1, H).to(torch.bfloat16)
        words = v.view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.quantize_rows(words, oracle.BF16, wire)
    if wire == oracle.WIRE_FP8_BLOCK128:
        dq = torch.from_numpy(codes).view(E4M3).float() * torch.from_numpy(
            scales).repeat_interleave(128, -1)
    else:
        grid = torch.tensor([oracle.e2m1_to_f32(c) for c in range(16)])
        c = torch.from_numpy(codes).long()
        nib = torch.stack([c & 0xF, c >> 4], -1).reshape(codes.shape[0], H)
        dq = grid[nib] * torch.exp2(torch.from_numpy(scales).float() - 127).repeat_interleave(32, -1)
    dq16 = dq.to(torch.bfloat16)
    assert torch.equal(dq16.float(), dq)                  # exact in bf16
    y16 = dq16.view(torch.int16).numpy().view(np.uint16).reshape(W, W * M, H)
    ref, _ = oracle.combine(W, M, k, H, oracle.BF16, inp["ntok"], disp["fwd"], y16)
    got = oracle.combine_wire(W, M, k, H, oracle.BF16, wire, inp["ntok"], disp["fwd"],
                              codes.reshape(W, W * M, -1), scales.reshape(W, W * M, -1))
    assert np.array_equal(got, ref)


E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the MX specification's E2M1 list


def _decoded_wire_rows(rng, n, H, wire):
    """Random wire rows whose values are exact in bf16 (power-of-two scales
    near 1), and those values decoded independently of the oracle: FP8 by
    torch's float8_e4m3fn, MXFP4 by the specification's table."""
    if wire == oracle.WIRE_FP8_BLOCK128:
        codes = rng.integers(0, 256, (n, H), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3C          # no NaN codes
        scales = np.ldexp(1.0, rng.integers(-4, 5, (n, H // 128))).astype(np.float32)
        vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
        vals = vals * np.repeat(scales, 128, axis=1)
        return codes, scales, vals.astype(np.float32)
    codes = rng.integers(0, 256, (n, H // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, (n, H // 32), dtype=np.uint8)
    nib = np.empty((n, H), np.uint8)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    mag = np.array(E2M1_VALUES, np.float32)[nib & 7]
    vals = np.where(nib & 8, -mag, mag) * np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127,
                                                                  32, axis=1))
    return codes, scales, vals.astype(np.float32)


@pytest.mark.parametrize("wire", [oracle.WIRE_FP8_BLOCK128, oracle.WIRE_MXFP4])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("cap", [3, 64])
def test_expert_combine_wire_equals_the_inverse_of_its_decoded_values(wire, weighted, cap):
    """The inverse from wire rows folds each element's exact value: with
    values exact in bf16 it equals the (pinned) inverse of those bf16 rows,
    plain and weighted, with and without capacity drops."""
    W, M, k, Er, H = 3, 20, 5, 4, 256
    rng = np.random.default_rng(17 + wire + 2 * weighted + cap)
    ntok = [20, 7, 13]
    idx = rng.integers(-1, W * Er + 1, (W, M, k)).astype(np.int32)
    w = rng.random((W, M, k)).astype(np.float32)
    x = rng.integers(0, 256, (W, M, 16), dtype=np.uint8)
    ref = oracle.dispatch(W, M, k, Er, ntok, x, idx, w)
    codes, scales, vals = _decoded_wire_rows(rng, W * Er * cap, H, wire)
    words = oracle.f32_to_bf16(vals.reshape(-1)).reshape(W, Er, cap, H)
    assert np.array_equal(oracle.bf16_to_f32(words.reshape(-1)), vals.reshape(-1))  # exact
    wt = ref["out_w"] if weighted else None
    got = oracle.expert_combine_wire(W, M, k, Er, cap, H, oracle.BF16, wire, ref["recv"],
                                     ref["out_idx"], codes.reshape(W, Er, cap, -1),
                                     scales.reshape(W, Er, cap, -1), w=wt)
    want = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, ref["recv"], ref["out_idx"],
                                 words, w=wt)
    assert np.array_equal(got, want)
    assert got.any()
