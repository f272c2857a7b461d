"""Pins for the oracle's combine (gather, FP32 sum in fixed order, cast).

"feat(ep): add opt-in gfx1201 EP2/EP4 support", How the gfx1201 kernels
work, Combine: each token's contributions come back through the reverse map,
are summed in FP32 and converted to BF16/FP16; optional FP32 weights are
summed separately and routing weights are not applied.

Pins, none of which calls the oracle through itself:
* closed form of the identity round trip: with identity experts a token comes
  back as RNE(n * v), n = its number of distinct ranks (n * v is exact in
  FP32 for n <= 64), the cast done by torch / numpy, not by the oracle;
* the push formulation (a scatter-add: every received row is added into its
  source token's accumulator through src_pos, with its own accumulation loop
  and its own way of finding a rank's place) equals the gather formulation
  bit for bit, on random expert outputs;
* hand-derived order and seed cases for the payload and for the weights:
  (2^24, 1, -2^24) in the token's rank order sums to 0 and in any other order
  to 1; all -0.0 stays -0.0 only when the sum starts from the first term;
* the relaxed-order bound: |out - exact sum| <= 1 ulp of the output type,
  exact sum in float64;
* weights: n * w exactly for weights with few significant bits;
* a token with no valid rank combines to +0.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

import experts


def _dispatch(wl, seed=None, inp=None):
    inp = inp or workloads.make_inputs(wl, seed)
    xb = inp["x"].view(torch.uint8).numpy()
    sc = None if inp["scales"] is None else inp["scales"].numpy()
    disp = oracle.dispatch(wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank,
                           inp["ntok"], xb, inp["idx"].numpy(), inp["w"].numpy(), sc)
    return inp, disp


def _num_ranks(wl, inp):
    Er, E = wl.experts_per_rank, wl.num_experts
    idx = inp["idx"].numpy()
    n = np.zeros((wl.world_size, wl.max_tokens), np.int64)
    for r in range(wl.world_size):
        for t in range(inp["ntok"][r]):
            n[r, t] = len({int(e) // Er for e in idx[r, t] if 0 <= e < E})
    return n


SMALL = [workloads.WORKLOADS["ep2_t16_h256_bf16_k2"],
         workloads.custom("ep4_t64_h512_fp16_k8", 4, 64, 512, 8, 32, "fp16"),
         workloads.custom("ep3_t40_h256_bf16_k5", 3, 40, 256, 5, 12, "bf16", ragged=True),
         workloads.WORKLOADS["ep4_ragged1024_h2048_fp16_k64"]]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_identity_round_trip_closed_form(wl):
    inp, disp = _dispatch(wl)
    y = experts.identity(wl, disp)
    out, out_w = oracle.combine(wl.world_size, wl.max_tokens, wl.topk, wl.hidden,
                                oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16,
                                inp["ntok"], disp["fwd"], y, disp["out_w"])
    n = torch.from_numpy(_num_ranks(wl, inp)).double()
    v = inp["x"].double()
    want = (v * n.unsqueeze(-1)).to(workloads.TORCH_DTYPE[wl.combine_dtype])
    want = want.view(torch.int16).numpy().view(np.uint16)
    for r in range(wl.world_size):
        T = inp["ntok"][r]
        assert np.array_equal(out[r, :T], want[r, :T])
        assert np.all(out[r, T:] == 0)  # rows of absent tokens untouched


def test_identity_round_trip_fp8_dequant_closed_form():
    """The FP8 workload: y = bf16(dequant(x)), so out = RNE_bf16(n * y)."""
    wl = workloads.custom("ep8_t32_h1024_fp8_k8_zipf", 8, 32, 1024, 8, 256, "fp8", "bf16",
                          scale_dim=8, routing="zipf", expert="dequant")
    inp, disp = _dispatch(wl)
    y = experts.dequant(wl, disp)
    out, _ = oracle.combine(8, 32, 8, 1024, oracle.BF16, inp["ntok"], disp["fwd"], y)
    x = inp["x"].float()
    sc = inp["scales"].repeat_interleave(1024 // 8, dim=-1)
    deq = (x * sc).to(torch.bfloat16).double()
    n = torch.from_numpy(_num_ranks(wl, inp)).double()
    want = (deq * n.unsqueeze(-1)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, want)


def _random_y(wl, seed):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn((wl.world_size, wl.world_size * wl.max_tokens, wl.hidden), generator=g)
    y = y.to(workloads.TORCH_DTYPE[wl.combine_dtype]).view(torch.int16).numpy().view(np.uint16)
    yw = torch.randn((wl.world_size, wl.world_size * wl.max_tokens, wl.topk), generator=g).numpy()
    return y, yw


@pytest.mark.parametrize("wl", SMALL + [workloads.WORKLOADS["ep4_t256_h4096_bf16_k8"]],
                         ids=lambda w: w.name)
def test_push_equals_gather_random_y(wl):
    inp, disp = _dispatch(wl)
    y, yw = _random_y(wl, 11)
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    args = (wl.world_size, wl.max_tokens, wl.topk)
    g_out, g_w = oracle.combine(*args, wl.hidden, dt, inp["ntok"], disp["fwd"], y, yw)
    p_out, p_w = oracle.combine_push(*args, wl.experts_per_rank, wl.hidden, dt, inp["ntok"],
                                     inp["idx"].numpy(), disp["recv"], disp["src_pos"], y, yw)
    assert np.array_equal(g_out, p_out)
    assert np.array_equal(g_w.view(np.uint32), p_w.view(np.uint32))


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_relaxed_order_one_ulp_bound(wl):
    inp, disp = _dispatch(wl)
    y, _ = _random_y(wl, 5)
    dt = workloads.TORCH_DTYPE[wl.combine_dtype]
    out, _ = oracle.combine(wl.world_size, wl.max_tokens, wl.topk, wl.hidden,
                            oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16,
                            inp["ntok"], disp["fwd"], y)
    yt = torch.from_numpy(y.view(np.int16)).view(dt).double().reshape(-1, wl.hidden)
    fwd = disp["fwd"]
    got = torch.from_numpy(out.view(np.int16)).view(dt).double()
    for r in range(wl.world_size):
        for t in range(inp["ntok"][r]):
            g = [int(v) for v in fwd[r, t] if v >= 0]
            exact = yt[g].sum(0)
            ulp = _ulp(torch.maximum(exact.abs(), got[r, t].abs()), dt)
            assert torch.all((got[r, t] - exact).abs() <= ulp), (r, t)


def _ulp(v, dt):
    """Spacing of dt's values at magnitude |v|: 2^(e - mantissa bits), with e
    the binade of |v|, floored at the smallest normal binade."""
    mant, emin = (7, -126) if dt == torch.bfloat16 else (10, -14)
    e = torch.floor(torch.log2(v.abs().clamp(min=2.0 ** emin)))
    return torch.pow(2.0, e - mant)


def test_weights_closed_form():
    wl = workloads.custom("ep4_t32_h64_bf16_k6", 4, 32, 64, 6, 16, "bf16")
    inp = workloads.make_inputs(wl)
    g = torch.Generator().manual_seed(3)
    inp["w"] = (torch.randint(1, 64, inp["w"].shape, generator=g).float() / 64.0).contiguous()
    inp, disp = _dispatch(wl, inp=inp)
    _, out_w = oracle.combine(4, 32, 6, 64, oracle.BF16, inp["ntok"], disp["fwd"],
                              experts.identity(wl, disp), disp["out_w"])
    n = _num_ranks(wl, inp)
    assert np.array_equal(out_w, inp["w"].numpy() * n[:, :, None])


def test_token_without_rank_combines_to_zero():
    W, M, k, Er, H = 2, 2, 2, 2, 8
    idx = np.array([[[-1, 9], [0, 3]], [[1, 2], [-3, -3]]], np.int32)
    x = np.full((W, M, H), 0x3F80, np.uint16)  # bf16 1.0
    disp = oracle.dispatch(W, M, k, Er, [2, 2], x, idx)
    y = disp["out_x"].view(np.uint16).reshape(W, W * M, H)
    out, _ = oracle.combine(W, M, k, H, oracle.BF16, [2, 2], disp["fwd"], y)
    assert np.all(out[0, 0] == 0) and np.all(out[1, 1] == 0)
    assert np.all(out[0, 1] == 0x4000) and np.all(out[1, 0] == 0x4000)  # 2.0


@pytest.mark.parametrize("dtype,big,small,want", [
    # bf16: (2^24 + 1) - 2^24 = 0 in the token's rank order (2^24 + 1 ties to
    # 2^24); ascending-rank or reversed order gives (-2^24 + 1) + 2^24 = 1.
    ("bf16", 0x4B80, 0x3F80, 0x0000),
    # fp16: (1024 + 2^-14) - 1024 = 0 in order (a tie to even in binary32);
    # any other order keeps the 2^-14.
    ("fp16", 0x6400, 0x0400, 0x0000),
])
def test_summation_order_is_token_rank_order(dtype, big, small, want):
    """Hand-derived: a token whose experts sit on ranks [2, 0, 1] in top-k
    order; contributions +big, +small, -big in that order."""
    W, M, k, Er, H = 3, 1, 3, 1, 8
    idx = np.array([[[2, 0, 1]], [[0, 0, 0]], [[0, 0, 0]]], np.int32)
    ntok = [1, 0, 0]
    disp = oracle.dispatch(W, M, k, Er, ntok, np.zeros((W, M, 2 * H), np.uint8), idx)
    y = np.zeros((W, W * M, H), np.uint16)
    y[2, 0] = big
    y[0, 0] = small
    y[1, 0] = big | 0x8000
    out, _ = oracle.combine(W, M, k, H, oracle.BF16 if dtype == "bf16" else oracle.FP16,
                            ntok, disp["fwd"], y)
    assert np.all(out[0, 0] == want), hex(int(out[0, 0, 0]))


def test_sum_is_seeded_with_first_contribution():
    """All contributions -0.0: seeded with the first one the sum stays -0.0
    (an accumulator started at +0.0 would give +0.0)."""
    W, M, k, Er, H = 2, 1, 2, 1, 8
    idx = np.array([[[1, 0]], [[0, 1]]], np.int32)
    disp = oracle.dispatch(W, M, k, Er, [1, 1], np.zeros((W, M, 2 * H), np.uint8), idx)
    y = np.full((W, W * M, H), 0x8000, np.uint16)
    out, _ = oracle.combine(W, M, k, H, oracle.BF16, [1, 1], disp["fwd"], y)
    assert np.all(out == 0x8000)


def _order_case():
    """A token of rank 0 whose experts sit on ranks [2, 0, 1] in top-k order
    (Er = 1, so expert e is on rank e); the other ranks send nothing."""
    W, M, k, Er, H = 3, 1, 3, 1, 8
    idx = np.array([[[2, 0, 1]], [[0, 0, 0]], [[0, 0, 0]]], np.int32)
    ntok = [1, 0, 0]
    disp = oracle.dispatch(W, M, k, Er, ntok, np.zeros((W, M, 2 * H), np.uint8), idx)
    return W, M, k, Er, H, idx, ntok, disp


@pytest.mark.parametrize("form", ["gather", "push"])
def test_weight_sum_order_is_token_rank_order(form):
    """Hand-derived weight fold: the rows received on ranks 2, 0, 1 carry
    weight rows 2^24, 1, -2^24. In the token's rank order (2, 0, 1) the FP32
    sum is (2^24 + 1) - 2^24 = 0, because 2^24 + 1 ties to the even 2^24.
    Ascending ranks (0, 1, 2) give (1 - 2^24) + 2^24 = 1 (1 - 2^24 is exact),
    and the reversed order (1, 0, 2) gives the same 1. A weight that is not
    summed at all, or summed twice, leaves 2^24 or -2^24 in some slot."""
    W, M, k, Er, H, idx, ntok, disp = _order_case()
    y = np.zeros((W, W * M, H), np.uint16)
    yw = np.zeros((W, W * M, k), np.float32)
    yw[2, 0] = [2.0 ** 24, 3.0, -0.5]
    yw[0, 0] = [1.0, 5.0, 0.25]
    yw[1, 0] = [-(2.0 ** 24), 7.0, 0.125]
    if form == "gather":
        _, out_w = oracle.combine(W, M, k, H, oracle.BF16, ntok, disp["fwd"], y, yw)
    else:
        _, out_w = oracle.combine_push(W, M, k, Er, H, oracle.BF16, ntok, idx, disp["recv"],
                                       disp["src_pos"], y, yw)
    # slot 1: 3 + 5 + 7 = 15; slot 2: -0.5 + 0.25 + 0.125 = -0.125 (exact)
    assert out_w[0, 0].tolist() == [0.0, 15.0, -0.125]


@pytest.mark.parametrize("form", ["gather", "push"])
def test_weight_sum_is_seeded_with_first_term(form):
    """All weights -0.0: a sum that starts from the first term stays -0.0
    (-0 + -0 = -0); one started at +0.0 gives +0.0."""
    W, M, k, Er, H, idx, ntok, disp = _order_case()
    y = np.zeros((W, W * M, H), np.uint16)
    yw = np.full((W, W * M, k), -0.0, np.float32)
    if form == "gather":
        _, out_w = oracle.combine(W, M, k, H, oracle.BF16, ntok, disp["fwd"], y, yw)
    else:
        _, out_w = oracle.combine_push(W, M, k, Er, H, oracle.BF16, ntok, idx, disp["recv"],
                                       disp["src_pos"], y, yw)
    assert np.all(out_w[0, 0].view(np.uint32) == 0x80000000)


@pytest.mark.parametrize("dtype,big,small,want", [
    ("bf16", 0x4B80, 0x3F80, 0x0000),
    ("fp16", 0x6400, 0x0400, 0x0000),
])
def test_push_summation_order_and_seed(dtype, big, small, want):
    """The push form on the hand-derived payload cases of the gather form:
    +big, +small, -big on ranks 2, 0, 1 in rank order gives +0; all -0.0
    stays -0.0."""
    W, M, k, Er, H, idx, ntok, disp = _order_case()
    dt = oracle.BF16 if dtype == "bf16" else oracle.FP16
    y = np.zeros((W, W * M, H), np.uint16)
    y[2, 0], y[0, 0], y[1, 0] = big, small, big | 0x8000
    out, _ = oracle.combine_push(W, M, k, Er, H, dt, ntok, idx, disp["recv"], disp["src_pos"], y)
    assert np.all(out[0, 0] == want)
    y[:] = 0x8000
    out, _ = oracle.combine_push(W, M, k, Er, H, dt, ntok, idx, disp["recv"], disp["src_pos"], y)
    assert np.all(out[0, 0] == 0x8000)


def test_push_rejects_a_missing_row():
    """The scatter-add checks that every token got one row per distinct rank:
    a reverse map that sends a token's row twice (and so drops another)
    fails instead of summing the wrong rows."""
    wl = workloads.custom("ep3_t8_h64_bf16_k3", 3, 8, 64, 3, 9, "bf16")
    inp, disp = _dispatch(wl)
    y, yw = _random_y(wl, 2)
    sp = disp["src_pos"].copy()
    d = int(np.argmax(disp["recv"] >= 2))
    sp[d, 1] = sp[d, 0]
    with pytest.raises(RuntimeError):
        oracle.combine_push(3, 8, 3, 3, 64, oracle.BF16, inp["ntok"], inp["idx"].numpy(),
                            disp["recv"], sp, y, yw)
