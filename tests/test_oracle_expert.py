"""Pins for the oracle's expert-major layout and its inverse.

"MORI-EP User Guide", section 4 "Standard MoE Compatibility (DeepEP)":
convert_dispatch_output() turns a rank's received rows into packed rows per
local expert with counts, source info and layout ranges, and
convert_combine_input() turns the experts' outputs back into one combine row
per received row. The section names the calls and their outputs only; the
readings the oracle takes are listed in its header.

Pins, none of which calls the oracle through itself:
* a hand-worked example (tests/golden/expert_layout_tiny.json), with a row of
  three local experts whose fold gives another result in id order;
* a sort formulation: every (rank, local expert, received row) triple from
  numpy's unique over each row's local ids, ordered by numpy's lexsort; the
  p-th triple of a (rank, expert) group is the expert's p-th row;
* layout ranges from numpy's searchsorted over each list's source ranks;
* capacity: a smaller capacity keeps a prefix of a larger one's lists and
  clips its ranges;
* the inverse: integer-valued outputs sum exactly (numpy add.at in float64),
  identity experts give RNE(n * x) with the cast done by torch, and rows whose
  outputs are (2^24, 1, -2^24) in first-occurrence order fold to +0;
* the round trip dispatch -> layout -> identity experts -> inverse -> combine
  gives K * x for integer payloads, K = the token's distinct valid experts;
* the weighted inverse: a hand-worked case where one fused multiply-add per
  term gives 2^-24 and a separate multiply and add gives +0; a repeated
  expert's weights add up; dyadic weights over integer outputs are exact
  (float64 reference); and the weighted round trip through dispatch and
  combine equals the mixture-of-experts sum over the token's valid slots of
  w_i * x.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _words(a):
    return np.array([[int(h, 16) for h in row] for row in a], np.uint16)


def test_golden_hand_worked_example():
    with open(os.path.join(GOLDEN, "expert_layout_tiny.json")) as f:
        g = json.load(f)
    W, M, k, Er, cap = g["W"], g["M"], g["k"], g["Er"], g["cap"]
    WM = W * M
    src_pos = np.full((W, WM), -1, np.int32)
    idx = np.full((W, WM, k), -3, np.int32)
    for d, rows in enumerate(g["rows"]):
        for q, (s, t, ids) in enumerate(rows):
            src_pos[d, q] = s * WM + t
            idx[d, q] = ids
    x = np.zeros((W, WM, 2), np.uint8)
    for d in range(W):
        for q in range(WM):
            x[d, q] = [12 * d + 2 * q, 12 * d + 2 * q + 1]
    o = oracle.expert_layout(W, M, k, Er, cap, g["recv"], src_pos, x, idx, fill=g["fill"])
    assert o["count"].tolist() == g["count"]
    assert o["src_info"].tolist() == g["src_info"]
    assert (o["layout_range"] >> 32).tolist() == g["layout_lo"]
    assert (o["layout_range"] & 0xFFFFFFFF).tolist() == g["layout_n"]
    assert o["px"].tolist() == g["px"]

    py = np.stack([np.stack([_words(slot) for slot in expert]) for expert in g["py_bf16"]])
    y = oracle.expert_combine(W, M, k, Er, cap, 2, oracle.BF16, g["recv"], idx, py)
    for d in range(W):
        want = _words(g["y_bf16"][d])
        assert np.array_equal(y[d, :len(want)], want), d
        assert not y[d, len(want):].any()


# --------------------------------------------------------------------------
# second formulation: sort of (rank, expert, row) triples
# --------------------------------------------------------------------------

def _local_lists(W, k, Er, recv, idx):
    """Per received row, its distinct local experts in first-occurrence order
    (numpy unique with return_index, re-sorted by index)."""
    out = {}
    for d in range(W):
        for q in range(int(recv[d])):
            ids = idx[d, q].astype(np.int64)
            loc = ids[(ids >= d * Er) & (ids < (d + 1) * Er)] - d * Er
            u, first = np.unique(loc, return_index=True)
            out[(d, q)] = u[np.argsort(first)]
    return out


def _sorted_triples(W, Er, lists):
    D, J, Q = [], [], []
    for (d, q), js in lists.items():
        for j in js:
            D.append(d)
            J.append(int(j))
            Q.append(q)
    D, J, Q = (np.array(v, np.int64) for v in (D, J, Q))
    order = np.lexsort((Q, J, D))
    D, J, Q = D[order], J[order], Q[order]
    groups = {}
    for d, j, q in zip(D, J, Q):
        groups.setdefault((int(d), int(j)), []).append(int(q))
    return groups


def _dispatched(wl, seed=None, integer_payload=False):
    inp = workloads.make_inputs(wl, seed)
    x = inp["x"]
    if integer_payload:
        g = torch.Generator().manual_seed(7)
        x = torch.randint(-4, 5, x.shape, generator=g).to(x.dtype)
    sc = None if inp["scales"] is None else inp["scales"].numpy()
    disp = oracle.dispatch(wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank,
                           inp["ntok"], x.view(torch.uint8).numpy(), inp["idx"].numpy(),
                           inp["w"].numpy(), sc)
    return inp, x, disp


CASES = [
    workloads.custom("ep2_t64_h64_bf16_k8", 2, 64, 64, 8, 16, "bf16"),
    workloads.custom("ep4_t48_h128_fp16_k6", 4, 48, 128, 6, 24, "fp16", ragged=True),
    workloads.custom("ep3_t40_h256_fp8_k5_s2", 3, 40, 256, 5, 12, "fp8", scale_dim=2),
    workloads.custom("ep4_t32_h64_bf16_k16_zipf", 4, 32, 64, 16, 64, "bf16", routing="zipf"),
    workloads.custom("ep1_t50_h64_bf16_k4", 1, 50, 64, 4, 8, "bf16"),
    workloads.WORKLOADS["ep2_t16_h256_bf16_k2"],
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_layout_equals_sort_formulation(wl):
    W, M, k, Er = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank
    WM = W * M
    inp, x, disp = _dispatched(wl)
    lists = _local_lists(W, k, Er, disp["recv"], disp["out_idx"])
    groups = _sorted_triples(W, Er, lists)
    cap = max([len(v) for v in groups.values()] + [1])
    o = oracle.expert_layout(W, M, k, Er, cap, disp["recv"], disp["src_pos"], disp["out_x"],
                             disp["out_idx"], disp["out_scales"], fill=-9)
    for d in range(W):
        for j in range(Er):
            rows = groups.get((d, j), [])
            assert o["count"][d, j] == len(rows)
            n = len(rows)
            assert np.array_equal(o["px"][d, j, :n], disp["out_x"][d, rows])
            assert not o["px"][d, j, n:].any()
            if disp["out_scales"] is not None:
                assert np.array_equal(o["psc"][d, j, :n], disp["out_scales"][d, rows])
            assert np.array_equal(o["src_info"][d, j, :n], disp["src_pos"][d, rows] % WM)
            assert (o["src_info"][d, j, n:] == -9).all()
            # ranges: searchsorted over the list's (non-decreasing) source ranks
            srcs = disp["src_pos"][d, rows] // WM
            assert (np.diff(srcs) >= 0).all()
            lo = np.searchsorted(srcs, np.arange(W), side="left")
            hi = np.searchsorted(srcs, np.arange(W), side="right")
            assert np.array_equal(o["layout_range"][d, j] >> 32, lo)
            assert np.array_equal(o["layout_range"][d, j] & 0xFFFFFFFF, hi - lo)


@pytest.mark.parametrize("wl", CASES[:4], ids=lambda w: w.name)
def test_smaller_capacity_keeps_a_prefix(wl):
    W, M, k, Er = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank
    inp, x, disp = _dispatched(wl)
    args = (disp["recv"], disp["src_pos"], disp["out_x"], disp["out_idx"], disp["out_scales"])
    big = oracle.expert_layout(W, M, k, Er, int(W * M), *args)
    top = int(big["count"].max())
    for cap in sorted({1, max(1, top // 3), max(1, top - 1)}):
        small = oracle.expert_layout(W, M, k, Er, cap, *args)
        assert np.array_equal(small["count"], big["count"])
        assert np.array_equal(small["px"], big["px"][:, :, :cap])
        assert np.array_equal(small["src_info"], big["src_info"][:, :, :cap])
        if small["psc"] is not None:
            assert np.array_equal(small["psc"], big["psc"][:, :, :cap])
        lo_b = big["layout_range"] >> 32
        hi_b = lo_b + (big["layout_range"] & 0xFFFFFFFF)
        lo, hi = np.minimum(lo_b, cap), np.minimum(hi_b, cap)
        assert np.array_equal(small["layout_range"], (lo << 32) | (hi - lo))


def test_no_rows_and_no_local_expert():
    W, M, k, Er = 2, 4, 2, 2
    WM = W * M
    idx = np.full((W, WM, k), 3, np.int32)        # expert 3: rank 1 only
    idx[1, :, :] = [0, 7]                         # rank 1's rows name rank 0's and invalid ids
    src_pos = np.tile(np.arange(WM, dtype=np.int32), (W, 1))
    x = np.arange(W * WM * 4, dtype=np.uint8).reshape(W, WM, 4)
    o = oracle.expert_layout(W, M, k, Er, 3, [0, 5], src_pos, x, idx, fill=-1)
    assert not o["count"].any()
    assert not o["px"].any()
    assert (o["src_info"] == -1).all()
    assert not o["layout_range"].any()
    y = oracle.expert_combine(W, M, k, Er, 3, 8, oracle.BF16, [0, 5], idx,
                              np.full((W, Er, 3, 8), 0x3F80, np.uint16))
    assert not y.any()                            # +0 rows for rank 1, nothing for rank 0


# --------------------------------------------------------------------------
# the inverse
# --------------------------------------------------------------------------

def _positions(W, Er, groups):
    pos = {}
    for (d, j), rows in groups.items():
        for p, q in enumerate(rows):
            pos[(d, j, q)] = p
    return pos


@pytest.mark.parametrize("wl", [CASES[0], CASES[1], CASES[3]], ids=lambda w: w.name)
@pytest.mark.parametrize("cap_div", [1, 2])
def test_inverse_integer_outputs_sum_exactly(wl, cap_div):
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    inp, x, disp = _dispatched(wl)
    lists = _local_lists(W, k, Er, disp["recv"], disp["out_idx"])
    groups = _sorted_triples(W, Er, lists)
    cap = max(1, max(len(v) for v in groups.values()) // cap_div)
    g = torch.Generator().manual_seed(11)
    vals = torch.randint(-50, 51, (W, Er, cap, H), generator=g)
    tdt = torch.bfloat16 if wl.combine_dtype == "bf16" else torch.float16
    py = vals.to(tdt).view(torch.int16).numpy().view(np.uint16)
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    y = oracle.expert_combine(W, M, k, Er, cap, H, dt, disp["recv"], disp["out_idx"], py)
    want = np.zeros((W, W * M, H), np.float64)
    pos = _positions(W, Er, groups)
    for (d, q), js in lists.items():
        for j in js:
            p = pos[(d, int(j), q)]
            if p < cap:
                np.add.at(want, (d, q), vals[d, j, p].numpy().astype(np.float64))
    got = torch.from_numpy(y.view(np.int16)).view(tdt).double().numpy()
    for d in range(W):
        R = int(disp["recv"][d])
        assert np.array_equal(got[d, :R], want[d, :R])
        assert not y[d, R:].any()


@pytest.mark.parametrize("wl", [CASES[0], CASES[1]], ids=lambda w: w.name)
def test_inverse_identity_closed_form(wl):
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    inp, x, disp = _dispatched(wl)
    lists = _local_lists(W, k, Er, disp["recv"], disp["out_idx"])
    cap = W * M
    o = oracle.expert_layout(W, M, k, Er, cap, disp["recv"], disp["src_pos"], disp["out_x"],
                             disp["out_idx"])
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    tdt = torch.bfloat16 if wl.combine_dtype == "bf16" else torch.float16
    y = oracle.expert_combine(W, M, k, Er, cap, H, dt, disp["recv"], disp["out_idx"],
                              o["px"].view(np.uint16))
    rows = torch.from_numpy(disp["out_x"].view(np.int16).reshape(W, W * M, H)).view(tdt)
    for (d, q), js in lists.items():
        want = (rows[d, q].double() * len(js)).to(tdt)     # n * v exact in fp64; torch rounds
        got = torch.from_numpy(y[d, q].view(np.int16)).view(tdt)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (d, q)


def test_inverse_folds_in_first_occurrence_order():
    wl = CASES[0]
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, 4
    inp, x, disp = _dispatched(wl)
    lists = _local_lists(W, k, Er, disp["recv"], disp["out_idx"])
    groups = _sorted_triples(W, Er, lists)
    pos = _positions(W, Er, groups)
    cap = W * M
    py = np.zeros((W, Er, cap, H), np.uint16)
    three = 0
    for (d, q), js in lists.items():
        if len(js) < 3 or list(js) == sorted(js):
            continue
        three += 1
        for j, v in zip(js[:3], (0x4B80, 0x3F80, 0xCB80)):   # 2^24, 1, -2^24
            py[d, j, pos[(d, int(j), q)]] = v
    assert three > 20
    y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, disp["recv"], disp["out_idx"], py)
    for (d, q), js in lists.items():
        if len(js) >= 3 and list(js) != sorted(js):
            # 2^24 + 1 rounds back to 2^24 in binary32, so this order gives +0;
            # summing in expert-id order would put 1 elsewhere and, in most
            # rows, give 1.
            assert not y[d, q].any(), (d, q, js)


@pytest.mark.parametrize("wl", [CASES[0], CASES[1], CASES[3], CASES[4]], ids=lambda w: w.name)
def test_round_trip_through_dispatch_and_combine(wl):
    W, M, k, Er, H, E = (wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden,
                         wl.num_experts)
    inp, x, disp = _dispatched(wl, integer_payload=True)
    cap = W * M
    o = oracle.expert_layout(W, M, k, Er, cap, disp["recv"], disp["src_pos"], disp["out_x"],
                             disp["out_idx"])
    dt = oracle.BF16 if wl.combine_dtype == "bf16" else oracle.FP16
    y = oracle.expert_combine(W, M, k, Er, cap, H, dt, disp["recv"], disp["out_idx"],
                              o["px"].view(np.uint16))
    out, _ = oracle.combine(W, M, k, H, dt, inp["ntok"], disp["fwd"], y)
    tdt = torch.bfloat16 if wl.combine_dtype == "bf16" else torch.float16
    got = torch.from_numpy(out.view(np.int16)).view(tdt).double()
    ids = inp["idx"].numpy()
    for r in range(W):
        for t in range(inp["ntok"][r]):
            K = len({int(e) for e in ids[r, t] if 0 <= e < E})
            assert torch.equal(got[r, t], x[r, t].double() * K), (r, t)


# --------------------------------------------------------------------------
# the weighted inverse ("MORI-EP User Guide", section 3: combine weights are
# for a weighted combination)
# --------------------------------------------------------------------------

def _one_row_case(ids, weights, outputs, k, Er=2):
    """One rank, one received row naming `ids`, the given weights, and the
    expert outputs (bf16 words, H = 1) in slot p = 0 of each local expert."""
    W, M, cap = 1, 2, 2
    idx = np.full((W, W * M, k), -1, np.int32)
    idx[0, 0] = ids
    w = np.zeros((W, W * M, k), np.float32)
    w[0, 0] = weights
    py = np.zeros((W, Er, cap, 1), np.uint16)
    for j, v in outputs.items():
        py[0, j, 0, 0] = v
    return oracle.expert_combine(W, M, k, Er, cap, 1, oracle.BF16, [1], idx, py, w=w)[0, 0, 0]


def test_weighted_inverse_uses_one_fused_multiply_add_per_term():
    # c0 = -(1 + 2^-17), c1 = 1 + 2^-17, both outputs 1 + 2^-7 (bf16 0x3F81).
    # c0 * v rounds the exact -(1 + 2^-7 + 2^-17 + 2^-24) (a tie) to
    # -(1 + 2^-7 + 2^-17); fma(c1, v, acc) then leaves exactly 2^-24 (bf16
    # 0x3380). A separate multiply and add would give +0.
    c = np.float32(1 + 2.0 ** -17)
    got = _one_row_case([0, 1], [-c, c], {0: 0x3F81, 1: 0x3F81}, k=2)
    assert got == 0x3380


def test_weighted_inverse_sums_the_weights_of_a_repeated_expert():
    # ids [1, 1]: expert 1 processes the row once, weight 0.5 + 0.25; output 2
    got = _one_row_case([1, 1], [0.5, 0.25], {1: 0x4000}, k=2)
    assert got == 0x3FC0                                    # 1.5


def test_weighted_inverse_exact_closed_form():
    wl = CASES[1]
    W, M, k, Er, H = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden
    inp, x, disp = _dispatched(wl)
    lists = _local_lists(W, k, Er, disp["recv"], disp["out_idx"])
    groups = _sorted_triples(W, Er, lists)
    pos = _positions(W, Er, groups)
    cap = max(len(v) for v in groups.values())
    g = torch.Generator().manual_seed(21)
    wts = np.array([0.25, 0.5, 1.0, 2.0, -1.0, -0.5], np.float32)
    w = wts[torch.randint(0, len(wts), (W, W * M, k), generator=g).numpy()]
    vals = torch.randint(-8, 9, (W, Er, cap, H), generator=g)
    py = vals.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.FP16, disp["recv"], disp["out_idx"],
                              py, w=w)
    got = torch.from_numpy(y.view(np.int16)).view(torch.float16).double().numpy()
    # every product and partial sum is a small dyadic number: exact in binary32
    for (d, q), js in lists.items():
        want = np.zeros(H)
        ids = disp["out_idx"][d, q]
        for j in js:
            c = sum(float(w[d, q, s]) for s in range(k) if ids[s] == d * Er + j)
            want += c * vals[d, j, pos[(d, int(j), q)]].numpy().astype(np.float64)
        assert np.array_equal(got[d, q], want), (d, q)


@pytest.mark.parametrize("wl", [CASES[0], CASES[3], CASES[4]], ids=lambda w: w.name)
def test_weighted_round_trip_is_the_moe_sum(wl):
    """dispatch -> layout -> identity experts -> weighted inverse -> combine
    gives sum over the token's valid slots of w_i * x, the mixture-of-experts
    output, for integer payloads and dyadic weights (all exact)."""
    W, M, k, Er, H, E = (wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, wl.hidden,
                         wl.num_experts)
    inp, x, disp = _dispatched(wl, integer_payload=True)
    g = torch.Generator().manual_seed(22)
    wts = np.array([0.25, 0.5, 1.0, 2.0], np.float32)
    w_tok = wts[torch.randint(0, 4, (W, M, k), generator=g).numpy()]
    disp = oracle.dispatch(W, M, k, Er, inp["ntok"], x.view(torch.uint8).numpy(),
                           inp["idx"].numpy(), w_tok)
    cap = W * M
    o = oracle.expert_layout(W, M, k, Er, cap, disp["recv"], disp["src_pos"], disp["out_x"],
                             disp["out_idx"])
    y = oracle.expert_combine(W, M, k, Er, cap, H, oracle.BF16, disp["recv"], disp["out_idx"],
                              o["px"].view(np.uint16), w=disp["out_w"])
    out, _ = oracle.combine(W, M, k, H, oracle.BF16, inp["ntok"], disp["fwd"], y)
    got = torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).double()
    ids = inp["idx"].numpy()
    for r in range(W):
        for t in range(inp["ntok"][r]):
            c = sum(float(w_tok[r, t, s]) for s in range(k) if 0 <= ids[r, t, s] < E)
            want = (x[r, t].double() * c).to(torch.bfloat16).double()
            assert torch.equal(got[r, t], want), (r, t)
