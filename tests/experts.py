"""Simulated experts: what a caller would run between dispatch and combine.

The pages leave the expert computation to the caller; the workloads name a
few stand-ins, computed here on the CPU with plain torch ops from the
oracle's dispatch outputs, and fed identically to the oracle's and the GPU
library's combine.

* identity: the expert returns its input row ("MORI-EP User Guide", section 7,
  uses the dispatched rows as the expert output).
* scalar:   row times the sum of the per-expert scalars s_e of the token's
  experts that live on the receiving rank, c = sum in top-k order, then
  y = bf16(f32(row) * c).
* dequant:  an FP8 row times its per-128 block FP32 scales, rounded to bf16
  (identity expert on the dequantized row).
"""
import numpy as np
import torch

from workloads import TORCH_DTYPE


def _rows_as(out_x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(out_x))
    return t.view(TORCH_DTYPE[dtype])


def identity(wl, disp) -> np.ndarray:
    """y = the received rows, as 16-bit words [W, W*M, H]."""
    assert wl.dispatch_dtype == wl.combine_dtype
    return disp["out_x"].view(np.uint16).reshape(wl.world_size, -1, wl.hidden)


def scalar(wl, disp, expert_scalars: torch.Tensor) -> np.ndarray:
    W, Er = wl.world_size, wl.experts_per_rank
    x = _rows_as(disp["out_x"], wl.dispatch_dtype).float()          # [W, WM, H]
    idx = torch.from_numpy(disp["out_idx"]).long()                   # [W, WM, k]
    s = expert_scalars.float()
    c = torch.zeros(idx.shape[:2], dtype=torch.float32)
    d_of_row = torch.arange(W).view(W, 1)
    for j in range(wl.topk):  # top-k order
        e = idx[:, :, j]
        valid = (e >= 0) & (e < wl.num_experts)
        local = valid & (e.clamp(0, wl.num_experts - 1) // Er == d_of_row)
        c = c + torch.where(local, s[e.clamp(0, wl.num_experts - 1)], torch.zeros(()))
    y = (x * c.unsqueeze(-1)).to(TORCH_DTYPE[wl.combine_dtype])
    return y.view(torch.int16).numpy().view(np.uint16)


def dequant(wl, disp) -> np.ndarray:
    x = _rows_as(disp["out_x"], "fp8").float()                       # [W, WM, H]
    sc = torch.from_numpy(disp["out_scales"]).view(torch.float32)    # [W, WM, S]
    blk = wl.hidden // wl.scale_dim
    sc_full = sc.repeat_interleave(blk, dim=-1)
    y = (x * sc_full).to(TORCH_DTYPE[wl.combine_dtype])
    return y.view(torch.int16).numpy().view(np.uint16)


def expert_output(wl, disp, inputs) -> np.ndarray:
    if wl.expert == "identity":
        return identity(wl, disp)
    if wl.expert == "scalar":
        return scalar(wl, disp, inputs["expert_scalars"])
    if wl.expert == "dequant":
        return dequant(wl, disp)
    raise ValueError(wl.expert)
