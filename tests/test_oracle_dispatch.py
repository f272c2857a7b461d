"""Pins for the oracle's dispatch (routing, dedup, receive layout, copies).

What the pages fix ("feat(ep): add opt-in gfx1201 EP2/EP4 support", How the
gfx1201 kernels work, Dispatch; "MORI-EP User Guide", section 3):
one receive row per (token, distinct destination rank); experts on one rank
share the payload; each received row carries the token's payload, expert ids,
weights and scales and its source, encoded src_rank * (W * M) + src_token.
"gfx1250 EPv2 ..." (PR 726) bounds a token's rows by min(W, k); the staging
refactor (PR 703, Motivation) puts a rank's receive capacity at W * M.

Pins, none of which calls the oracle through itself:
* brute force over every top-k row of tiny shapes, written as a per-rank
  filter and list search rather than the oracle's counting walk;
* a hand-worked example stored under tests/golden/;
* the second formulation (qsort of (d, r, t) triples) at every workload shape;
* invariants: each (token, rank) pair sent once, src_pos a bijection onto the
  received rows, rows copied verbatim, |D| within [1, min(W, k)];
* the expected number of distinct ranks per token against its closed form.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def brute_layout(W, M, k, Er, ntok, idx):
    """For every destination d: the list of source tokens (r, t), in (r, t)
    order, whose top-k row names an expert on d. A token's ranks in order of
    first appearance. Independent of the oracle's walk."""
    E = W * Er
    rows = {d: [] for d in range(W)}
    ranks_of = {}
    for r in range(W):
        for t in range(ntok[r]):
            row = [int(e) for e in idx[r, t]]
            valid = [e for e in row if 0 <= e < E]
            ranks = []
            for e in valid:
                if e // Er not in ranks:
                    ranks.append(e // Er)
            ranks_of[(r, t)] = ranks
    for d in range(W):
        for r in range(W):
            for t in range(ntok[r]):
                if any(0 <= int(e) < E and int(e) // Er == d for e in idx[r, t]):
                    rows[d].append((r, t))
    return rows, ranks_of


def check_against_brute(W, M, k, Er, ntok, idx, x=None, w=None):
    if x is None:
        x = np.arange(W * M * 16, dtype=np.uint32).astype(np.uint8).reshape(W, M, 16)
    out = oracle.dispatch(W, M, k, Er, ntok, x, idx, w)
    rows, ranks_of = brute_layout(W, M, k, Er, ntok, idx)
    WM = W * M
    P = min(W, k)
    for d in range(W):
        assert out["recv"][d] == len(rows[d])
        for s, (r, t) in enumerate(rows[d]):
            assert out["src_pos"][d, s] == r * WM + t
            assert np.array_equal(out["out_x"][d, s], x[r, t])
            assert np.array_equal(out["out_idx"][d, s], idx[r, t])
    for (r, t), ranks in ranks_of.items():
        want = [d * WM + rows[d].index((r, t)) for d in ranks] + [-1] * (P - len(ranks))
        assert list(out["fwd"][r, t]) == want


@pytest.mark.parametrize("W,Er,k", [(1, 1, 1), (1, 3, 2), (2, 1, 2), (2, 2, 3), (3, 1, 3),
                                    (3, 2, 2), (2, 3, 3)])
def test_exhaustive_single_token_rows(W, Er, k):
    """Every top-k row over E = W * Er experts (repeats included) as the only
    token on rank 0, and as token 1 of rank W-1 behind a fixed token."""
    E = W * Er
    for row in itertools.product(range(E), repeat=k):
        M = 2
        idx = np.zeros((W, M, k), np.int32)
        ntok = [0] * W
        idx[0, 0] = row
        ntok[0] = 1
        check_against_brute(W, M, k, Er, ntok, idx)
        idx2 = np.zeros((W, M, k), np.int32)
        ntok2 = [0] * W
        idx2[W - 1, 0] = [(j * Er) % E for j in range(k)]
        idx2[W - 1, 1] = row
        ntok2[W - 1] = 2
        check_against_brute(W, M, k, Er, ntok2, idx2)


@pytest.mark.parametrize("seed", range(6))
def test_random_tiny_against_brute(seed):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(1, 5))
    Er = int(rng.integers(1, 4))
    k = int(rng.integers(1, 7))
    M = int(rng.integers(1, 9))
    E = W * Er
    ntok = [int(v) for v in rng.integers(0, M + 1, size=W)]
    idx = rng.integers(-1, E + 1, size=(W, M, k)).astype(np.int32)  # includes invalid ids
    w = rng.standard_normal((W, M, k)).astype(np.float32)
    x = rng.integers(0, 256, size=(W, M, 32)).astype(np.uint8)
    check_against_brute(W, M, k, Er, ntok, idx, x=x, w=w)


def test_golden_hand_worked_example():
    with open(os.path.join(GOLDEN, "dispatch_tiny.json")) as f:
        g = json.load(f)
    W, M, k, Er = g["W"], g["M"], g["k"], g["Er"]
    idx = np.array(g["idx"], np.int32)
    x = np.arange(W * M * 16, dtype=np.uint8).reshape(W, M, 16)
    out = oracle.dispatch(W, M, k, Er, g["ntok"], x, idx)
    assert out["recv"].tolist() == g["recv"]
    for d in range(W):
        assert out["src_pos"][d, : g["recv"][d]].tolist() == g["src_pos"][d]
    assert out["fwd"].tolist() == g["fwd"]


def test_invalid_ids_select_no_rank():
    W, M, k, Er = 2, 3, 3, 2
    idx = np.array([[[-1, 4, 1], [7, -5, 99], [3, 3, 0]],
                    [[0, 0, 0], [2, -1, 2], [1, 1, 1]]], np.int32)
    out = oracle.dispatch(W, M, k, Er, [3, 3], np.zeros((W, M, 16), np.uint8), idx)
    # rank 0: t0 -> [0]; t1 -> []; t2 -> [1, 0]; rank 1: t0 -> [0]; t1 -> [1]; t2 -> [0]
    assert out["recv"].tolist() == [4, 2]
    assert out["fwd"][0, 1].tolist() == [-1, -1]


def _dispatch_workload(wl, M_cap=None):
    inp = workloads.make_inputs(wl)
    ntok = inp["ntok"]
    idx = inp["idx"].numpy()
    xb = inp["x"].view(torch.uint8).numpy()
    sc = None if inp["scales"] is None else inp["scales"].numpy()
    out = oracle.dispatch(wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank, ntok,
                          xb, idx, inp["w"].numpy(), sc)
    return inp, xb, out


def _check_invariants(wl, inp, xb, out):
    W, M, k = wl.world_size, wl.max_tokens, wl.topk
    WM = W * M
    ntok = inp["ntok"]
    idx = inp["idx"].numpy()
    w = inp["w"].numpy()
    sc = None if inp["scales"] is None else inp["scales"].numpy().view(np.uint8).reshape(W, M, -1)
    Er = wl.experts_per_rank
    # receive capacity and bijection of src_pos onto the received rows
    seen = set()
    for d in range(W):
        R = int(out["recv"][d])
        assert 0 <= R <= WM
        sp = out["src_pos"][d, :R]
        r, t = sp // WM, sp % WM
        assert np.all(t < np.array(ntok)[r])
        # rows copied verbatim, row by row
        assert np.array_equal(out["out_x"][d, :R], xb[r, t])
        assert np.array_equal(out["out_idx"][d, :R], idx[r, t])
        assert np.array_equal(out["out_w"][d, :R].view(np.uint32), w[r, t].view(np.uint32))
        if sc is not None:
            assert np.array_equal(out["out_scales"][d, :R], sc[r, t])
        # each received token really routes to d
        assert np.all(np.any(idx[r, t] // Er == d, axis=1))
        # rows of one destination are in (source rank, source token) order
        assert np.all(np.diff(sp.astype(np.int64)) > 0)
        for p in sp.tolist():
            assert (d, p) not in seen
            seen.add((d, p))
    # every (token, distinct rank) pair was sent exactly once
    total = 0
    for r in range(W):
        ranks = idx[r, : ntok[r]] // Er
        nd = np.array([len(set(row.tolist())) for row in ranks])
        assert np.all(nd >= 1) and np.all(nd <= min(W, k))
        total += int(nd.sum())
        # fwd points back to rows that name this token
        fw = out["fwd"][r, : ntok[r]]
        for t in range(ntok[r]):
            g = fw[t][fw[t] >= 0]
            assert len(g) == nd[t]
            assert np.all(out["src_pos"].reshape(-1)[g] == r * WM + t)
            assert [int(v) // WM for v in g] == list(dict.fromkeys((ranks[t]).tolist()))
    assert total == int(out["recv"].sum()) == len(seen)


@pytest.mark.parametrize("name", [n for n in workloads.WORKLOADS if n != workloads.HEADLINE])
def test_workload_invariants_and_sort_formulation(name):
    wl = workloads.WORKLOADS[name]
    inp, xb, out = _dispatch_workload(wl)
    _check_invariants(wl, inp, xb, out)
    recv, src_pos = oracle.layout_by_sort(wl.world_size, wl.max_tokens, wl.topk,
                                          wl.experts_per_rank, inp["ntok"], inp["idx"].numpy())
    assert np.array_equal(recv, out["recv"])
    for d in range(wl.world_size):
        assert np.array_equal(src_pos[d, : recv[d]], out["src_pos"][d, : recv[d]])


def test_headline_layout_sort_formulation():
    """The 8-rank x 4096-token routing, layout only (no payload copy)."""
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    ntok = workloads.token_counts(wl)
    idx = workloads.expert_ids(wl).numpy()
    W, M, k, Er = wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank
    x = np.zeros((W, M, 16), np.uint8)
    out = oracle.dispatch(W, M, k, Er, ntok, x, idx)
    recv, src_pos = oracle.layout_by_sort(W, M, k, Er, ntok, idx)
    assert np.array_equal(recv, out["recv"])
    for d in range(W):
        assert np.array_equal(src_pos[d, : recv[d]], out["src_pos"][d, : recv[d]])


def expected_distinct_ranks(W, E, Er, k):
    """E|D| = W * (1 - C(E - Er, k) / C(E, k)) for k distinct uniform ids."""
    return W * (1 - math.comb(E - Er, k) / math.comb(E, k))


@pytest.mark.parametrize("name,closed", [
    ("ep2_t16_h256_bf16_k2", 1.5714), ("ep4_t256_h4096_bf16_k8", 3.6142),
    ("ep8_t4096_h7168_bf16_k8", 5.2947), ("ep4_ragged1024_h2048_fp16_k64", 4.0000)])
def test_mean_distinct_ranks_closed_form(name, closed):
    wl = workloads.WORKLOADS[name]
    val = expected_distinct_ranks(wl.world_size, wl.num_experts, wl.experts_per_rank, wl.topk)
    assert abs(val - closed) < 1e-4
    ntok = workloads.token_counts(wl)
    idx = workloads.expert_ids(wl).numpy()
    W, M = wl.world_size, wl.max_tokens
    out = oracle.dispatch(W, M, wl.topk, wl.experts_per_rank, ntok, np.zeros((W, M, 16), np.uint8), idx)
    n = sum(ntok)
    mean = out["recv"].sum() / n
    # binomial-ish spread: allow 4 standard errors (|D| <= W, var <= W^2/4)
    tol = 4 * (W / 2) / math.sqrt(n) if n < 4096 else 0.01 * val
    assert abs(mean - val) <= max(tol, 1e-9), (mean, val)
