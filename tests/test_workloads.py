"""The seeded input generators: shapes, ranges, determinism and the
distributions the workloads name."""
import numpy as np
import pytest
import torch

import workloads

SMALL = [n for n in workloads.WORKLOADS if n != workloads.HEADLINE]


@pytest.mark.parametrize("name", SMALL)
def test_shapes_ranges_and_determinism(name):
    wl = workloads.WORKLOADS[name]
    a = workloads.make_inputs(wl)
    b = workloads.make_inputs(wl)
    W, M, k, E = wl.world_size, wl.max_tokens, wl.topk, wl.num_experts
    assert a["x"].shape == (W, M, wl.hidden) and a["x"].dtype == workloads.TORCH_DTYPE[wl.dispatch_dtype]
    assert a["idx"].shape == (W, M, k) and a["idx"].dtype == torch.int32
    assert a["w"].shape == (W, M, k) and a["w"].dtype == torch.float32
    assert torch.equal(a["x"].view(torch.uint8), b["x"].view(torch.uint8))
    assert torch.equal(a["idx"], b["idx"]) and torch.equal(a["w"], b["w"])
    assert a["ntok"] == b["ntok"]
    assert all(0 <= t <= M for t in a["ntok"])
    idx = a["idx"].reshape(-1, k)
    assert int(idx.min()) >= 0 and int(idx.max()) < E
    # distinct ids in every row
    s, _ = idx.sort(dim=1)
    assert bool((s[:, 1:] != s[:, :-1]).all())
    assert torch.allclose(a["w"].sum(-1), torch.ones(W, M), atol=1e-5)
    if wl.scale_dim:
        sc = a["scales"]
        assert sc.shape == (W, M, wl.scale_dim)
        assert float(sc.min()) >= 0.01 and float(sc.max()) <= 1.0
        assert wl.hidden == 128 * wl.scale_dim


def test_other_seed_changes_bytes():
    wl = workloads.WORKLOADS["ep2_t16_h256_bf16_k2"]
    a = workloads.make_inputs(wl)
    b = workloads.make_inputs(wl, seed=1)
    assert not torch.equal(a["idx"], b["idx"])


def test_uniform_ids_are_uniform():
    wl = workloads.WORKLOADS["ep4_t256_h4096_bf16_k8"]
    ids = workloads.expert_ids(wl).reshape(-1).numpy()
    cnt = np.bincount(ids, minlength=wl.num_experts)
    mean = ids.size / wl.num_experts
    # chi-square with 255 dof: mean 255, sd ~22.6; 6 sd margin
    chi2 = float(((cnt - mean) ** 2 / mean).sum())
    assert chi2 < 255 + 6 * 22.6


def test_zipf_ids_are_skewed_by_popularity():
    wl = workloads.WORKLOADS["ep8_t128_h7168_fp8_k8_zipf"]
    ids = workloads.expert_ids(wl).reshape(-1).numpy()
    cnt = np.bincount(ids, minlength=wl.num_experts)
    g = torch.Generator()
    g.manual_seed(workloads.BASE_SEED + 1000 * 5 + wl.seed_index)
    perm = torch.randperm(wl.num_experts, generator=g).numpy()
    by_rank = cnt[perm]  # counts in popularity-rank order
    assert by_rank[0] == cnt.max()
    assert by_rank[:8].sum() > by_rank[-64:].sum()


def test_ragged_counts_cover_zero_to_max():
    wl = workloads.WORKLOADS["ep4_ragged1024_h2048_fp16_k64"]
    ntok = workloads.token_counts(wl)
    assert len(ntok) == 4 and all(0 <= t <= 1024 for t in ntok)
    many = [workloads.token_counts(wl, seed=s)[0] for s in range(200)]
    assert min(many) < 64 and max(many) > 960
