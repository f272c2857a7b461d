"""Seeded synthetic inputs for MoE expert-parallel dispatch/combine.

This module only draws inputs: token counts, payload rows, top-k expert ids,
routing weights, scale rows and per-expert scalars. It holds none of the
method's arithmetic (no routing, no layout, no sums, no casts of results) and
is shared by the tests, the smoke check and the benchmark, which feed the
same bytes to the CPU oracle and to the GPU library.

Workload shapes follow the pages' own setups: uniform distinct top-8 over 256
experts ("feat(ep): add opt-in gfx1201 EP2/EP4 support", measurement setup),
the DeepSeek-V3 shape of 7168 hidden, 256 experts over 8 ranks, top-8
("MORI-EP User Guide", section 2), FP8 payloads with FP32 per-128 block scales
("MORI (ROCm/mori) — L2 Distillation", section 11). Every draw is from a
seeded torch CPU generator; the base seed 20261225 is the one the gfx1201
benchmark instructions use. Each workload and each input stream gets its own
generator, so a stream's bytes do not depend on the others.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

BASE_SEED = 20261225

# input stream ids: independent generators per stream
_S_NTOK, _S_X, _S_IDX, _S_W, _S_SCALES, _S_PERM, _S_EXPERT = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    world_size: int            # W virtual ranks on the one GPU
    max_tokens: int            # M = max_num_inp_token_per_rank
    hidden: int                # H
    dispatch_dtype: str        # "bf16" | "fp16" | "fp8"
    combine_dtype: str         # "bf16" | "fp16"
    num_experts: int           # E (experts per rank = E / W)
    topk: int                  # k
    scale_dim: int = 0         # S fp32 scales per token (0: none)
    routing: str = "uniform"   # "uniform" distinct ids | "zipf" (s = 1.2)
    ragged: bool = False       # token counts ~ U{0..M} per rank
    expert: str = "identity"   # simulated expert: "identity" | "scalar" | "dequant"
    seed_index: int = 0

    @property
    def experts_per_rank(self) -> int:
        return self.num_experts // self.world_size


WORKLOADS = {
    w.name: w for w in [
        Workload("ep2_t16_h256_bf16_k2", 2, 16, 256, "bf16", "bf16", 8, 2, seed_index=0),
        Workload("ep4_t256_h4096_bf16_k8", 4, 256, 4096, "bf16", "bf16", 256, 8,
                 expert="scalar", seed_index=1),
        Workload("ep8_t4096_h7168_bf16_k8", 8, 4096, 7168, "bf16", "bf16", 256, 8, seed_index=2),
        Workload("ep8_t128_h7168_fp8_k8_zipf", 8, 128, 7168, "fp8", "bf16", 256, 8,
                 scale_dim=56, routing="zipf", expert="dequant", seed_index=3),
        Workload("ep4_ragged1024_h2048_fp16_k64", 4, 1024, 2048, "fp16", "fp16", 256, 64,
                 ragged=True, seed_index=4),
    ]
}

# the throughput case the benchmark times
HEADLINE = "ep8_t4096_h7168_bf16_k8"

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp8": torch.float8_e4m3fn}
ELEM_BYTES = {"bf16": 2, "fp16": 2, "fp8": 1}


def _gen(wl: Workload, stream: int, seed: Optional[int]) -> torch.Generator:
    g = torch.Generator()
    base = BASE_SEED if seed is None else seed
    g.manual_seed(base + 1000 * stream + wl.seed_index)
    return g


def token_counts(wl: Workload, seed: Optional[int] = None) -> list:
    if not wl.ragged:
        return [wl.max_tokens] * wl.world_size
    g = _gen(wl, _S_NTOK, seed)
    return [int(v) for v in torch.randint(0, wl.max_tokens + 1, (wl.world_size,), generator=g)]


def payload(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """[W, M, H] rows ~ N(0,1) in the dispatch dtype (fp8: OCP e4m3fn after
    clamping to its finite range). Every row of M is drawn, also rows past a
    rank's token count, so a kernel that read them would change results."""
    g = _gen(wl, _S_X, seed)
    W, M, H = wl.world_size, wl.max_tokens, wl.hidden
    out = torch.empty((W, M, H), dtype=TORCH_DTYPE[wl.dispatch_dtype])
    for r in range(W):  # per rank, to bound the fp32 temporary
        v = torch.randn((M, H), generator=g, dtype=torch.float32)
        if wl.dispatch_dtype == "fp8":
            v = v.clamp_(-448.0, 448.0)
        out[r] = v.to(out.dtype)
    return out


def expert_ids(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """[W, M, k] int32 expert ids. "uniform": k distinct ids, uniform over the
    E experts and in random order. "zipf": k distinct ids drawn one after
    another without replacement with p(i) ~ i^-1.2 over popularity ranks
    i = 1..E, mapped through a seeded permutation of the experts."""
    W, M, k, E = wl.world_size, wl.max_tokens, wl.topk, wl.num_experts
    g = _gen(wl, _S_IDX, seed)
    if wl.routing == "uniform":
        keys = torch.rand((W * M, E), generator=g)
        ids = keys.argsort(dim=1)[:, :k]
    elif wl.routing == "zipf":
        gp = _gen(wl, _S_PERM, seed)
        perm = torch.randperm(E, generator=gp)
        p = torch.arange(1, E + 1, dtype=torch.float64).pow(-1.2)
        ranks = torch.multinomial(p.expand(W * M, E), k, replacement=False, generator=g)
        ids = perm[ranks]
    else:
        raise ValueError(wl.routing)
    return ids.to(torch.int32).reshape(W, M, k).contiguous()


def routing_weights(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """[W, M, k] fp32 softmax of N(0,1) logits."""
    g = _gen(wl, _S_W, seed)
    logits = torch.randn((wl.world_size, wl.max_tokens, wl.topk), generator=g)
    return torch.softmax(logits, dim=-1).contiguous()


def scales(wl: Workload, seed: Optional[int] = None) -> Optional[torch.Tensor]:
    """[W, M, S] fp32 ~ U(0.01, 1), one per 128-element block, or None."""
    if wl.scale_dim == 0:
        return None
    g = _gen(wl, _S_SCALES, seed)
    u = torch.rand((wl.world_size, wl.max_tokens, wl.scale_dim), generator=g)
    return (0.01 + 0.99 * u).contiguous()


def expert_scalars(wl: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """[E] fp32 ~ U(0.5, 2): the per-expert factor of the "scalar" expert."""
    g = _gen(wl, _S_EXPERT, seed)
    return (0.5 + 1.5 * torch.rand((wl.num_experts,), generator=g)).contiguous()


def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """All inputs of one call, as CPU tensors."""
    return dict(
        ntok=token_counts(wl, seed),
        x=payload(wl, seed),
        idx=expert_ids(wl, seed),
        w=routing_weights(wl, seed),
        scales=scales(wl, seed),
        expert_scalars=expert_scalars(wl, seed) if wl.expert == "scalar" else None,
    )


def custom(name: str, W: int, M: int, H: int, k: int, E: int, dispatch_dtype: str = "bf16",
           combine_dtype: Optional[str] = None, scale_dim: int = 0, routing: str = "uniform",
           ragged: bool = False, expert: str = "identity", seed_index: int = 100) -> Workload:
    """A workload of any shape, for sweeps and edge cases."""
    if combine_dtype is None:
        combine_dtype = "fp16" if dispatch_dtype == "fp16" else "bf16"
    return Workload(name, W, M, H, dispatch_dtype, combine_dtype, E, k, scale_dim, routing,
                    ragged, expert, seed_index)
