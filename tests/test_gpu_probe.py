"""The access-pattern probes (include/ep_probe.h) move the bytes they claim
to: a probe whose result were wrong would time the wrong pattern. The
fan-out through the dispatch's forward map writes exactly the rows the
dispatch writes; the gather-sum through it gives the combine's result (on
rows that are not all -0.0); the copy and write probes fill what they cover
and nothing past it. Shapes span several tiles with a ragged row tail and
several row pieces."""
import numpy as np
import pytest
import torch

import combine_route_amd as cra
import workloads

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _op_after_dispatch(W, M, H, k, E, seed):
    wl = workloads.custom(f"probe_ep{W}_t{M}_h{H}_k{k}", W, M, H, k, E, "bf16", seed_index=seed)
    inp = workloads.make_inputs(wl)
    cfg = cra.make_config(W, H, M, E // W, k, "bf16", "bf16")
    op = cra.EpDispatchCombineOp(cfg)
    x = inp["x"].cuda()
    op.dispatch(inp["ntok"], x, inp["idx"].cuda(), inp["w"].cuda())
    torch.cuda.synchronize()
    return wl, inp, op, x


@pytest.mark.parametrize("W,M,H,k,E,pieces,waves", [(4, 96, 1032, 8, 64, 1, 8),
                                                    (8, 200, 7168, 8, 256, 2, 8),
                                                    (3, 70, 520, 5, 12, 3, 4)])
def test_fanout_and_gather_equal_dispatch_and_combine(W, M, H, k, E, pieces, waves):
    _say(f"[case] probe fanout/gather W={W} M={M} H={H} k={k} pieces={pieces}")
    wl, inp, op, x = _op_after_dispatch(W, M, H, k, E, 700 + W)
    WM, row = W * M, H * 2
    recv = op.recv_num_token.cpu().numpy()
    want_x = op.out_x.clone()
    out, _ = op.combine(op.out_x)
    torch.cuda.synchronize()
    want_out = out.clone()
    fmap, stride = cra.ep_probe_forward_map(op.plan)
    assert stride == min(W, k)
    dst = torch.zeros_like(op.out_x)
    cra.ep_probe_pattern(cra.EP_PROBE_FANOUT, row, W * M, x, dst, fmap, W * WM, stride,
                         pieces, waves)
    torch.cuda.synchronize()
    for d in range(W):
        R = int(recv[d])
        assert torch.equal(dst[d, :R].view(torch.int16), want_x[d, :R].view(torch.int16)), d
        assert not dst[d, R:].view(torch.int16).any(), d      # nothing past the received rows
    g = torch.full_like(op.combine_out, 7.0)
    cra.ep_probe_pattern(cra.EP_PROBE_GATHER, row, W * M, want_x, g, fmap, W * WM, stride,
                         pieces, waves)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), want_out.view(torch.int16))
    op.close()


def test_copy_write_read_cover_their_rows():
    _say("[case] probe copy/write/read")
    rows, row = 37, 7168 * 2
    src = torch.randint(-30000, 30000, (rows + 3, row // 2), dtype=torch.int16,
                        device="cuda").view(torch.bfloat16)
    dst = torch.zeros_like(src)
    cra.ep_probe_pattern(cra.EP_PROBE_COPY, row, rows, src, dst, pieces=2, waves=4)
    torch.cuda.synchronize()
    assert torch.equal(dst[:rows].view(torch.int16), src[:rows].view(torch.int16))
    assert not dst[rows:].view(torch.int16).any()
    w = torch.zeros((rows + 1, row), dtype=torch.uint8, device="cuda")
    cra.ep_probe_pattern(cra.EP_PROBE_WRITE, row, rows, None, w, pieces=3, waves=8)
    torch.cuda.synchronize()
    words = w[:rows].view(torch.int32).view(rows, row // 16, 4).cpu().numpy()
    assert np.array_equal(words[:, :, 0], np.repeat(np.arange(rows)[:, None], row // 16, 1))
    assert np.array_equal(words[:, :, 1], np.repeat(np.arange(row // 16)[None, :], rows, 0))
    assert not w[rows:].any()
    sink = torch.zeros(rows * 2, dtype=torch.int32, device="cuda")
    cra.ep_probe_pattern(cra.EP_PROBE_READ, row, rows, src, sink, pieces=2, waves=8)
    torch.cuda.synchronize()
    # each wave's word is the XOR of its piece's 32-bit words
    s32 = src[:rows].view(torch.int32).view(rows, 2, -1).cpu().numpy()
    want = np.bitwise_xor.reduce(s32, axis=2).reshape(-1)
    assert np.array_equal(sink.cpu().numpy(), want)
