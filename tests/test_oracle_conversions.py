"""Pins for the oracle's binary32 -> bfloat16 / binary16 casts and widenings.

The combine ends in a round-to-nearest-even cast ("feat(ep): add opt-in
gfx1201 EP2/EP4 support", How the gfx1201 kernels work, Combine: FP32 sum
then BF16/FP16). The oracle writes both casts from the IEEE definitions; here
they are checked against independent library routines (torch's bfloat16
conversion, numpy's float16) over every 16-bit encoding, over random and
tie-heavy binary32 inputs, and at the format boundaries.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _interesting_f32(n=1 << 20, seed=7):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    # force exact ties at the bf16 and fp16 cut points on a quarter each
    bits[: n // 4] = (bits[: n // 4] & 0xFFFF0000) | 0x8000
    bits[n // 4: n // 2] = (bits[n // 4: n // 2] & 0xFFFFE000) | 0x1000
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_widen_all_encodings():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_narrow_roundtrip_all_encodings():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(h)
    back = oracle.f32_to_bf16(f)
    nan = np.isnan(f)
    assert np.array_equal(back[~nan], h[~nan])
    assert np.all(back[nan] == 0x7FC0)


def test_bf16_narrow_matches_torch_rne():
    f = _interesting_f32()
    assert np.array_equal(oracle.f32_to_bf16(f), _torch_bf16_bits(f))


def test_bf16_narrow_boundaries():
    cases = [
        (1.0, 0x3F80), (-0.0, 0x8000), (0.0, 0x0000),
        (float(np.float32(1.0) + np.float32(2.0 ** -8)), 0x3F80),      # tie, even stays
        (float(np.float32(1.0) + np.float32(3 * 2.0 ** -8)), 0x3F82),  # tie, odd rounds up
        (float(np.finfo(np.float32).max), 0x7F80),                     # rounds to +inf
        (float("inf"), 0x7F80), (float("-inf"), 0xFF80),
    ]
    for v, want in cases:
        got = int(oracle.f32_to_bf16(np.array([v], np.float32))[0])
        assert got == want, (v, hex(got), hex(want))
    assert int(oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]) == 0x7FC0


def test_f16_widen_all_encodings():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_narrow_matches_numpy():
    f = _interesting_f32()
    f = np.concatenate([f, (f * np.float32(2.0 ** -20)).astype(np.float32),
                        (f * np.float32(2.0 ** -130)).astype(np.float32)])
    f = f[np.isfinite(f)]
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(f), ref)


def test_f16_narrow_every_f16_midpoint():
    # every exact midpoint between adjacent finite fp16 values, both signs
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # midpoints are exact in fp32
    for s in (1.0, -1.0):
        m = (mid * np.float32(s)).astype(np.float32)
        with np.errstate(over="ignore"):
            ref = m.astype(np.float16).view(np.uint16)
        assert np.array_equal(oracle.f32_to_f16(m), ref)


@pytest.mark.parametrize("v,want", [
    (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (-65520.0, 0xFC00),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -25, 0x0001),
    (3 * 2.0 ** -25, 0x0002), (2.0 ** -14, 0x0400), (-0.0, 0x8000), (1.0, 0x3C00),
])
def test_f16_narrow_boundaries(v, want):
    got = int(oracle.f32_to_f16(np.array([v], np.float32))[0])
    assert got == want, (v, hex(got), hex(want))
