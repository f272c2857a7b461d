"""Host-side checks of the C ABI (no GPU needed, no kernel is ever launched).

The library must load, export every function include/ep.h declares, size the
workspace from one function, and reject every bad argument on the host with
a message naming it before anything is enqueued (the staging refactor's
caller contract: "refactor(EPv2): replace per-module __device__ staging with
shared buffer", Caller contract). Every call below fails validation before a
launch, so these tests are safe on a machine with a GPU too; pointers are
fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import combine_route_amd as cra
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_WS = 0x7F0000000000          # 256-byte aligned, never dereferenced
FAKE = 0x7F1000000000             # 16-byte aligned device-looking address


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cra.LIB_PATH):
        import combine_route_amd.build as b
        b.build()
    return cra.load()


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            with open(os.path.join(ROOT, "include", h)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) == 22
    assert sorted(cra.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def wl_config(wl):
    return cra.make_config(wl.world_size, wl.hidden, wl.max_tokens, wl.experts_per_rank,
                           wl.topk, wl.dispatch_dtype, wl.combine_dtype,
                           scale_dim=wl.scale_dim, scale_type_size=4)


def expected_workspace(W, M, k):
    """Layout: tile counts and tile bases (W x W*ceil(M/16) int32 each),
    src_pos (W x W*M int32), forward map (W x M x min(W,k) int32), each
    rounded up to 256 bytes."""
    up = lambda v: (v + 255) // 256 * 256
    tiles = W * ((M + 15) // 16)
    return 2 * up(4 * W * tiles) + up(4 * W * W * M) + up(4 * W * M * min(W, k))


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workspace_bytes_golden(lib, name):
    wl = workloads.WORKLOADS[name]
    cfg = wl_config(wl)
    assert cra.ep_workspace_bytes(cfg) == expected_workspace(wl.world_size, wl.max_tokens, wl.topk)


def test_workspace_bytes_headline_value(lib):
    # 8 ranks x 4096 tokens, top-8: 2 x 32 KiB tiles + 1 MiB src_pos + 1 MiB fwd
    cfg = wl_config(workloads.WORKLOADS[workloads.HEADLINE])
    assert cra.ep_workspace_bytes(cfg) == 2 * 8 * 8 * 256 * 4 + 8 * 8 * 4096 * 4 + 8 * 4096 * 8 * 4


BAD_CONFIGS = [
    (dict(world_size=0), "world_size"), (dict(world_size=65), "world_size"),
    (dict(max_num_inp_token_per_rank=0), "max_num_inp_token_per_rank"),
    (dict(num_experts_per_token=0), "num_experts_per_token"),
    (dict(num_experts_per_token=65), "num_experts_per_token"),
    (dict(num_experts_per_rank=0), "num_experts_per_rank"),
    (dict(hidden_dim=0), "hidden_dim"), (dict(hidden_dim=260), "hidden_dim"),
    (dict(dispatch_dtype=7), "dispatch_dtype"), (dict(combine_dtype=2), "combine_dtype"),
    (dict(scale_dim=-1), "scale_dim"), (dict(scale_dim=3, scale_type_size=3), "scale_type_size"),
    (dict(scale_dim=3, scale_type_size=2), "scale_dim * cfg.scale_type_size"),
    (dict(world_size=64, max_num_inp_token_per_rank=600000), "2^31"),
    (dict(combine_wire=3), "combine_wire"), (dict(combine_wire=-1), "combine_wire"),
    (dict(combine_wire=1, hidden_dim=7168 + 64), "EP_WIRE_FP8_BLOCK128"),
    (dict(combine_wire=2, hidden_dim=7168 + 16), "EP_WIRE_MXFP4"),
    (dict(dispatch_cast=3), "dispatch_cast"), (dict(dispatch_cast=-1), "dispatch_cast"),
    (dict(dispatch_cast=1), "EP_FP8_E4M3"),
]


@pytest.mark.parametrize("change,word", BAD_CONFIGS)
def test_bad_config_rejected(lib, change, word):
    base = dict(world_size=8, hidden_dim=7168, scale_dim=0, scale_type_size=0,
                max_num_inp_token_per_rank=4096, num_experts_per_rank=32,
                num_experts_per_token=8, dispatch_dtype=0, combine_dtype=0)
    base.update(change)
    cfg = cra.EpConfig(**base)
    assert lib.ep_workspace_bytes(ctypes.byref(cfg)) == 0
    assert word in cra.ep_last_error()
    out = ctypes.c_void_p(0)
    rc = lib.ep_plan_create(ctypes.byref(cfg), FAKE_WS, 1 << 40, ctypes.byref(out))
    assert rc in (cra.EP_ERR_ARG, cra.EP_ERR_SIZE) and out.value is None


def test_fp8_hidden_must_fill_16_bytes(lib):
    cfg = cra.make_config(8, 7160, 128, 32, 8, "fp8", "bf16", scale_dim=56)
    assert lib.ep_workspace_bytes(ctypes.byref(cfg)) == 0


def make_plan(lib, cfg, ws=FAKE_WS, nbytes=None):
    out = ctypes.c_void_p(0)
    n = cra.ep_workspace_bytes(cfg) if nbytes is None else nbytes
    rc = lib.ep_plan_create(ctypes.byref(cfg), ws, n, ctypes.byref(out))
    return rc, out.value


def test_plan_create_errors(lib):
    cfg = cra.make_config(4, 4096, 256, 64, 8)
    need = cra.ep_workspace_bytes(cfg)
    out = ctypes.c_void_p(0)
    assert lib.ep_plan_create(None, FAKE_WS, need, ctypes.byref(out)) == cra.EP_ERR_NULL
    assert lib.ep_plan_create(ctypes.byref(cfg), None, need, ctypes.byref(out)) == cra.EP_ERR_NULL
    assert "workspace" in cra.ep_last_error()
    assert lib.ep_plan_create(ctypes.byref(cfg), FAKE_WS, need, None) == cra.EP_ERR_NULL
    assert make_plan(lib, cfg, ws=FAKE_WS + 16)[0] == cra.EP_ERR_ALIGN
    assert "256" in cra.ep_last_error()
    assert make_plan(lib, cfg, nbytes=need - 1)[0] == cra.EP_ERR_SIZE
    assert str(need) in cra.ep_last_error()
    rc, plan = make_plan(lib, cfg)
    assert rc == cra.EP_OK and plan
    assert lib.ep_plan_destroy(plan) == cra.EP_OK
    assert lib.ep_plan_destroy(None) == cra.EP_OK


def test_src_token_pos_pointer_and_rank_check(lib):
    W, M, k = 4, 256, 8
    cfg = cra.make_config(W, 4096, M, 64, k)
    rc, plan = make_plan(lib, cfg)
    assert rc == 0
    p = ctypes.c_void_p()
    up = lambda v: (v + 255) // 256 * 256
    off = 2 * up(4 * W * W * ((M + 15) // 16))
    for r in range(W):
        assert lib.ep_get_src_token_pos(plan, r, ctypes.byref(p)) == 0
        assert p.value == FAKE_WS + off + r * W * M * 4
    assert lib.ep_get_src_token_pos(plan, W, ctypes.byref(p)) == cra.EP_ERR_ARG
    assert lib.ep_get_src_token_pos(plan, -1, ctypes.byref(p)) == cra.EP_ERR_ARG
    assert lib.ep_get_src_token_pos(plan, 0, None) == cra.EP_ERR_NULL
    lib.ep_plan_destroy(plan)


def dispatch_args(W, **over):
    nt = (ctypes.c_int32 * W)(*([4] * W))
    a = dict(num_tokens=ctypes.cast(nt, ctypes.c_void_p).value, x=FAKE, indices=FAKE + 0x1000,
             weights=None, scales=None, out_x=FAKE + 0x2000, out_indices=FAKE + 0x3000,
             out_weights=None, out_scales=None, recv_num_token=FAKE + 0x4000)
    a.update(over)
    return cra.EpDispatchArgs(**a), nt


@pytest.mark.parametrize("over,code,word", [
    (dict(num_tokens=None), cra.EP_ERR_NULL, "num_tokens"),
    (dict(x=None), cra.EP_ERR_NULL, "args.x"),
    (dict(indices=None), cra.EP_ERR_NULL, "args.indices"),
    (dict(out_x=None), cra.EP_ERR_NULL, "args.out_x"),
    (dict(out_indices=None), cra.EP_ERR_NULL, "args.out_indices"),
    (dict(recv_num_token=None), cra.EP_ERR_NULL, "recv_num_token"),
    (dict(x=FAKE + 8), cra.EP_ERR_ALIGN, "args.x"),
    (dict(out_x=FAKE + 4), cra.EP_ERR_ALIGN, "args.out_x"),
    (dict(weights=FAKE + 0x5000), cra.EP_ERR_ARG, "weights"),
    (dict(out_weights=FAKE + 0x5000), cra.EP_ERR_ARG, "weights"),
    (dict(scales=FAKE + 0x6000, out_scales=FAKE + 0x7000), cra.EP_ERR_ARG, "scale_dim = 0"),
])
def test_dispatch_rejects_before_launch(lib, over, code, word):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    a, keep = dispatch_args(2, **over)
    assert lib.ep_dispatch(plan, ctypes.byref(a), None) == code
    assert word in cra.ep_last_error()
    lib.ep_plan_destroy(plan)


def test_dispatch_rejects_token_counts(lib):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    for bad in ([17, 0], [0, -1]):
        nt = (ctypes.c_int32 * 2)(*bad)
        a, _ = dispatch_args(2, num_tokens=ctypes.cast(nt, ctypes.c_void_p).value, x=None)
        # T_r is checked before any pointer
        assert lib.ep_dispatch(plan, ctypes.byref(a), None) == cra.EP_ERR_ARG
        assert "num_tokens" in cra.ep_last_error()
    lib.ep_plan_destroy(plan)


def test_dispatch_rejects_a_copy_grid_past_32_bits(lib):
    # 8 x 4096 tokens in 16-token tiles: 2048 tiles x 16 shares x 896 row
    # pieces x 1024 work-items a block is past 2^32; checked before any launch
    cfg = cra.make_config(8, 7168, 4096, 32, 8)
    rc, plan = make_plan(lib, cfg)
    cra.ep_plan_set_launch(plan, dict(tile_tokens=16, dispatch_waves=16, dispatch_row_split=896,
                                      dispatch_token_split=16))
    nt = (ctypes.c_int32 * 8)(*([4096] * 8))
    a, _ = dispatch_args(8, num_tokens=ctypes.cast(nt, ctypes.c_void_p).value)
    assert lib.ep_dispatch(plan, ctypes.byref(a), None) == cra.EP_ERR_ARG
    assert "2^32" in cra.ep_last_error()
    lib.ep_plan_destroy(plan)


def test_dispatch_requires_scales_when_configured(lib):
    cfg = cra.make_config(8, 7168, 128, 32, 8, "fp8", "bf16", scale_dim=56)
    rc, plan = make_plan(lib, cfg)
    a, _ = dispatch_args(8, scales=FAKE + 0x6000)
    assert lib.ep_dispatch(plan, ctypes.byref(a), None) == cra.EP_ERR_NULL
    assert "scales" in cra.ep_last_error()
    a, _ = dispatch_args(8, scales=FAKE + 0x6004, out_scales=FAKE + 0x7000)
    assert lib.ep_dispatch(plan, ctypes.byref(a), None) == cra.EP_ERR_ALIGN
    lib.ep_plan_destroy(plan)


def test_combine_errors_and_state(lib):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    ok = dict(y=FAKE, y_weights=None, out=FAKE + 0x1000, out_weights=None, y_scales=None)
    cases = [(dict(y=None), cra.EP_ERR_NULL, "args.y"), (dict(out=None), cra.EP_ERR_NULL, "args.out"),
             (dict(y=FAKE + 2), cra.EP_ERR_ALIGN, "aligned"),
             (dict(y_weights=FAKE + 0x2000), cra.EP_ERR_ARG, "weights"),
             (dict(y_scales=FAKE + 0x3000), cra.EP_ERR_ARG, "y_scales"),
             ({}, cra.EP_ERR_STATE, "before any dispatch")]
    for over, code, word in cases:
        a = cra.EpCombineArgs(**{**ok, **over})
        assert lib.ep_combine(plan, ctypes.byref(a), None) == code
        assert word in cra.ep_last_error()
    assert lib.ep_combine(None, ctypes.byref(cra.EpCombineArgs(**ok)), None) == cra.EP_ERR_NULL
    lib.ep_plan_destroy(plan)


def test_launch_override_limits_and_auto_geometry(lib):
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    cfg = wl_config(wl)
    rc, plan = make_plan(lib, cfg)
    auto = cra.ep_plan_get_launch(plan, [4096] * 8)
    assert auto["tile_tokens"] in (16, 32, 64)
    assert 1 <= auto["dispatch_row_split"] <= 7168 * 2 // 16
    # 512 tiles of 64 tokens: 14 KB rows in two 7 KB pieces, each tile shared
    # by blocks of 4 waves, one token a wave
    assert (auto["tile_tokens"], auto["dispatch_waves"], auto["dispatch_token_split"],
            auto["dispatch_row_split"]) == (64, 4, 16, 2)
    # and the combines fold 1 KB pieces, 16 waves a block
    assert (auto["combine_waves"], auto["combine_row_split"]) == (16, 14)
    assert (auto["expert_combine_waves"], auto["expert_combine_row_split"]) == (16, 14)
    for bad in (dict(tile_tokens=8), dict(dispatch_waves=17), dict(combine_waves=17),
                dict(dispatch_row_split=7168 * 2 // 16 + 1), dict(combine_row_split=897),
                dict(cache_policy=3), dict(cache_policy=-1), dict(layout=4), dict(layout=-2)):
        with pytest.raises(cra.EpError):
            cra.ep_plan_set_launch(plan, bad)
    cra.ep_plan_set_launch(plan, dict(tile_tokens=32, dispatch_waves=2))
    got = cra.ep_plan_get_launch(plan, [4096] * 8)
    assert got["tile_tokens"] == 32 and got["dispatch_waves"] == 2
    assert got["dispatch_token_split"] == 16  # still one token a wave
    cra.ep_plan_set_launch(plan, None)
    assert cra.ep_plan_get_launch(plan, [4096] * 8) == auto
    small = cra.ep_plan_get_launch(plan, [1] + [0] * 7)
    assert small["tile_tokens"] == 16
    # rows of the full call far exceed the last-level cache: streaming moves;
    # one token's rows fit: cached moves
    assert auto["cache_policy"] == cra.EP_CACHE_STREAM
    assert small["cache_policy"] == cra.EP_CACHE_KEEP
    # 32768 tokens in 512 tiles: routing and scan kernels; one token: the copy
    # blocks work out the layout alone
    assert auto["layout"] == cra.EP_LAYOUT_KERNELS
    assert small["layout"] == cra.EP_LAYOUT_IN_COPY
    assert cra.ep_plan_get_launch(plan, [200, 56] + [0] * 6)["layout"] == cra.EP_LAYOUT_IN_COPY
    assert cra.ep_plan_get_launch(plan, [200, 57] + [0] * 6)["layout"] == \
        cra.EP_LAYOUT_SCAN_IN_COPY
    assert cra.ep_plan_get_launch(plan, [4096, 1024] + [0] * 6)["layout"] == \
        cra.EP_LAYOUT_KERNELS
    with pytest.raises(cra.EpError):
        cra.ep_plan_get_launch(plan, [4097] + [0] * 7)
    # the expert-major copy (tiles of 64 of the most rows a rank can hold):
    # 8 x 512 tiles, and 8 x 16 tiles x 14 row pieces, reach 1024 blocks
    # without sharing a tile, and share each tile among blocks of one row a
    # wave; 8 x 2 tiles x 14 pieces do not, so small calls share each tile
    # first, at most one row a wave
    assert auto["expert_token_split"] == 64 // auto["expert_waves"]
    assert auto["expert_row_split"] == 1
    mid = cra.ep_plan_get_launch(plan, [128] * 8)
    assert mid["expert_token_split"] == 64 // mid["expert_waves"]
    assert mid["expert_row_split"] == 8
    for few in ([16] * 8, [1] + [0] * 7):
        dec = cra.ep_plan_get_launch(plan, few)
        assert dec["expert_token_split"] == 64 // dec["expert_waves"]
    for bad in (dict(expert_token_split=65),):
        with pytest.raises(cra.EpError):
            cra.ep_plan_set_launch(plan, bad)
    cra.ep_plan_set_launch(plan, dict(expert_token_split=64))
    assert cra.ep_plan_get_launch(plan, [4096] * 8)["expert_token_split"] == 64
    cra.ep_plan_set_launch(plan, None)
    # small calls share no tile
    assert cra.ep_plan_get_launch(plan, [16] * 8)["dispatch_token_split"] == 1
    with pytest.raises(cra.EpError):
        cra.ep_plan_set_launch(plan, dict(dispatch_token_split=65))
    cra.ep_plan_set_launch(plan, dict(dispatch_token_split=8))
    assert cra.ep_plan_get_launch(plan, [4096] * 8)["dispatch_token_split"] == 8
    cra.ep_plan_set_launch(plan, None)
    lib.ep_plan_destroy(plan)
    # k > 16: the copy blocks cannot route the whole call; few tiles: they scan
    wl = workloads.WORKLOADS["ep4_ragged1024_h2048_fp16_k64"]
    rc, plan = make_plan(lib, wl_config(wl))
    got = cra.ep_plan_get_launch(plan, workloads.token_counts(wl))
    assert got["layout"] == cra.EP_LAYOUT_SCAN_IN_COPY
    with pytest.raises(cra.EpError):
        cra.ep_plan_set_launch(plan, dict(layout=cra.EP_LAYOUT_IN_COPY))
    lib.ep_plan_destroy(plan)
    # a large top-64 call: one block a tile, rows in one 4 KB piece
    rc, plan = make_plan(lib, cra.make_config(4, 2048, 4096, 64, 64, "fp16", "fp16"))
    big = cra.ep_plan_get_launch(plan, [4096] * 4)
    assert (big["tile_tokens"], big["dispatch_token_split"], big["dispatch_row_split"]) == \
        (32, 1, 1)
    lib.ep_plan_destroy(plan)
    # a cast dispatch: as the plain one, 4 waves a block, one token a wave
    rc, plan = make_plan(lib, cra.make_config(8, 7168, 4096, 32, 8, "fp8", "bf16",
                                              dispatch_cast="bf16"))
    cast = cra.ep_plan_get_launch(plan, [4096] * 8)
    assert (cast["dispatch_waves"], cast["dispatch_token_split"], cast["dispatch_row_split"]) == \
        (4, 16, 2)
    lib.ep_plan_destroy(plan)


def test_kernel_time_argument_checks(lib):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    c, ms = ctypes.c_int32(), ctypes.c_double()
    assert lib.ep_plan_kernel_time(plan, 12, ctypes.byref(c), ctypes.byref(ms)) == cra.EP_ERR_ARG
    assert lib.ep_plan_kernel_time(plan, -1, ctypes.byref(c), ctypes.byref(ms)) == cra.EP_ERR_ARG
    assert lib.ep_plan_kernel_time(plan, 0, ctypes.byref(c), ctypes.byref(ms)) == 0
    assert lib.ep_plan_kernel_time(plan, cra.EP_KERNEL_STANDARD_COMBINE, ctypes.byref(c),
                                   ctypes.byref(ms)) == 0
    assert c.value == 0 and ms.value == 0.0
    lib.ep_plan_destroy(plan)


# ---------------------------------------------------------------------------
# expert plans ("MORI-EP User Guide", section 4: convert_dispatch_output and
# convert_combine_input)
# ---------------------------------------------------------------------------

def expected_expert_workspace(W, M, k, Er):
    """Layout: tile counts and bases (W*Er x max(ceil(W*M/64), W*ceil(M/64)),
    at least 1, int32 each: the convert path's tiles of received rows or the
    fused path's tiles of source tokens), source starts (W x W int32),
    in-tile prefixes (W*Er x W int32), the inverse's map (W x W*M x min(k, Er)
    int32, or the fused path's per-slot map W x M x k, whichever is larger)
    and its weights (W x W*M x min(k, Er) float), each rounded up to 256
    bytes."""
    up = lambda v: (v + 255) // 256 * 256
    T = max(1, (W * M + 63) // 64)
    tiles = max(T, W * max(1, (M + 63) // 64))
    return (2 * up(4 * W * Er * tiles) + up(4 * W * W) + up(4 * W * Er * W)
            + up(4 * max(W * W * M * min(k, Er), W * M * k)) + up(4 * W * W * M * min(k, Er)))


def make_expert(lib, plan, cap, ws=FAKE_WS + (1 << 30), nbytes=None):
    out = ctypes.c_void_p(0)
    n = lib.ep_expert_workspace_bytes(plan, cap) if nbytes is None else nbytes
    rc = lib.ep_expert_plan_create(plan, cap, ws, n, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_expert_workspace_bytes_golden(lib, name):
    wl = workloads.WORKLOADS[name]
    rc, plan = make_plan(lib, wl_config(wl))
    for cap in (1, 7, wl.world_size * wl.max_tokens):
        assert lib.ep_expert_workspace_bytes(plan, cap) == expected_expert_workspace(
            wl.world_size, wl.max_tokens, wl.topk, wl.experts_per_rank)
    lib.ep_plan_destroy(plan)


def test_expert_plan_create_errors_and_lifetime(lib):
    W, M, Er = 4, 64, 16
    cfg = cra.make_config(W, 512, M, Er, 8)
    rc, plan = make_plan(lib, cfg)
    for cap, code, word in ((0, cra.EP_ERR_ARG, "cap"), (W * M + 1, cra.EP_ERR_ARG, "cap")):
        assert lib.ep_expert_workspace_bytes(plan, cap) == 0
        assert word in cra.ep_last_error()
        assert make_expert(lib, plan, cap, nbytes=1 << 30)[0] == code
    assert lib.ep_expert_workspace_bytes(None, 4) == 0
    need = lib.ep_expert_workspace_bytes(plan, 8)
    out = ctypes.c_void_p(0)
    assert lib.ep_expert_plan_create(None, 8, FAKE_WS, need, ctypes.byref(out)) == cra.EP_ERR_NULL
    assert lib.ep_expert_plan_create(plan, 8, None, need, ctypes.byref(out)) == cra.EP_ERR_NULL
    assert lib.ep_expert_plan_create(plan, 8, FAKE_WS, need, None) == cra.EP_ERR_NULL
    assert make_expert(lib, plan, 8, ws=FAKE_WS + 64)[0] == cra.EP_ERR_ALIGN
    assert make_expert(lib, plan, 8, nbytes=need - 1)[0] == cra.EP_ERR_SIZE
    assert str(need) in cra.ep_last_error()
    rc, ex = make_expert(lib, plan, 8)
    assert rc == cra.EP_OK and ex
    # the plan outlives its expert plans
    assert lib.ep_plan_destroy(plan) == cra.EP_ERR_STATE
    assert "expert plan" in cra.ep_last_error()
    assert lib.ep_expert_plan_destroy(ex) == cra.EP_OK
    assert lib.ep_expert_plan_destroy(None) == cra.EP_OK
    assert lib.ep_plan_destroy(plan) == cra.EP_OK


def test_expert_capacity_limit_is_int32(lib):
    # W * Er * cap must stay below 2^31: packed rows are int32 in the map
    cfg = cra.make_config(8, 256, 65536, 4096, 8)
    rc, plan = make_plan(lib, cfg)
    assert rc == 0
    assert lib.ep_expert_workspace_bytes(plan, 65536) == 0
    assert "2^31" in cra.ep_last_error()
    assert lib.ep_expert_workspace_bytes(plan, 65535) > 0
    lib.ep_plan_destroy(plan)


def convert_args(**over):
    a = dict(x=FAKE, indices=FAKE + 0x1000, weights=None, scales=None,
             recv_num_token=FAKE + 0x2000,
             packed_x=FAKE + 0x3000, packed_scales=None, packed_count=FAKE + 0x4000,
             packed_src_info=FAKE + 0x5000, packed_layout_range=FAKE + 0x6000)
    a.update(over)
    return cra.EpConvertDispatchArgs(**a)


@pytest.mark.parametrize("over,code,word", [
    (dict(x=None), cra.EP_ERR_NULL, "args.x"),
    (dict(indices=None), cra.EP_ERR_NULL, "args.indices"),
    (dict(recv_num_token=None), cra.EP_ERR_NULL, "recv_num_token"),
    (dict(packed_x=None), cra.EP_ERR_NULL, "packed_x"),
    (dict(packed_count=None), cra.EP_ERR_NULL, "packed_count"),
    (dict(packed_src_info=None), cra.EP_ERR_NULL, "packed_src_info"),
    (dict(packed_layout_range=None), cra.EP_ERR_NULL, "packed_layout_range"),
    (dict(x=FAKE + 8), cra.EP_ERR_ALIGN, "args.x"),
    (dict(packed_x=FAKE + 0x3004), cra.EP_ERR_ALIGN, "packed_x"),
    (dict(packed_layout_range=FAKE + 0x6004), cra.EP_ERR_ALIGN, "packed_layout_range"),
    (dict(indices=FAKE + 0x1002), cra.EP_ERR_ALIGN, "indices"),
    (dict(weights=FAKE + 0x9002), cra.EP_ERR_ALIGN, "weights"),
    (dict(scales=FAKE + 0x7000, packed_scales=FAKE + 0x8000), cra.EP_ERR_ARG, "scale_dim = 0"),
    ({}, cra.EP_ERR_STATE, "before any dispatch"),
])
def test_convert_dispatch_output_rejects_before_launch(lib, over, code, word):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 8)
    a = convert_args(**over)
    assert lib.ep_convert_dispatch_output(ex, ctypes.byref(a), None) == code
    assert word in cra.ep_last_error()
    assert lib.ep_convert_dispatch_output(None, ctypes.byref(a), None) == cra.EP_ERR_NULL
    assert lib.ep_convert_dispatch_output(ex, None, None) == cra.EP_ERR_NULL
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def test_convert_requires_scales_when_configured(lib):
    cfg = cra.make_config(8, 7168, 128, 32, 8, "fp8", "bf16", scale_dim=56)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 64)
    a = convert_args(scales=FAKE + 0x7000)
    assert lib.ep_convert_dispatch_output(ex, ctypes.byref(a), None) == cra.EP_ERR_NULL
    assert "scales" in cra.ep_last_error()
    a = convert_args(scales=FAKE + 0x7002, packed_scales=FAKE + 0x8000)
    assert lib.ep_convert_dispatch_output(ex, ctypes.byref(a), None) == cra.EP_ERR_ALIGN
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def test_convert_combine_input_errors_and_state(lib):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 8)
    ok = dict(packed_y=FAKE, y=FAKE + 0x1000, apply_weights=0)
    for over, code, word in [(dict(packed_y=None), cra.EP_ERR_NULL, "packed_y"),
                             (dict(y=None), cra.EP_ERR_NULL, "args.y"),
                             (dict(y=FAKE + 8), cra.EP_ERR_ALIGN, "aligned"),
                             (dict(apply_weights=2), cra.EP_ERR_ARG, "apply_weights"),
                             (dict(apply_weights=-1), cra.EP_ERR_ARG, "apply_weights"),
                             ({}, cra.EP_ERR_STATE, "before any convert_dispatch_output")]:
        a = cra.EpConvertCombineArgs(**{**ok, **over})
        assert lib.ep_convert_combine_input(ex, ctypes.byref(a), None) == code
        assert word in cra.ep_last_error()
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def standard_args(**over):
    a = dict(num_tokens=None, x=FAKE, indices=FAKE + 0x1000, scales=None,
             packed_x=FAKE + 0x3000, packed_scales=None, packed_count=FAKE + 0x4000,
             packed_src_info=FAKE + 0x5000, packed_layout_range=FAKE + 0x6000)
    a.update(over)
    return a


@pytest.mark.parametrize("over,code,word", [
    (dict(x=None), cra.EP_ERR_NULL, "args.x"),
    (dict(indices=None), cra.EP_ERR_NULL, "args.indices"),
    (dict(packed_x=None), cra.EP_ERR_NULL, "packed_x"),
    (dict(packed_count=None), cra.EP_ERR_NULL, "packed_count"),
    (dict(packed_src_info=None), cra.EP_ERR_NULL, "packed_src_info"),
    (dict(packed_layout_range=None), cra.EP_ERR_NULL, "packed_layout_range"),
    (dict(x=FAKE + 8), cra.EP_ERR_ALIGN, "args.x"),
    (dict(packed_x=FAKE + 0x3004), cra.EP_ERR_ALIGN, "packed_x"),
    (dict(packed_layout_range=FAKE + 0x6004), cra.EP_ERR_ALIGN, "packed_layout_range"),
    (dict(indices=FAKE + 0x1002), cra.EP_ERR_ALIGN, "indices"),
    (dict(scales=FAKE + 0x7000, packed_scales=FAKE + 0x8000), cra.EP_ERR_ARG, "scale_dim = 0"),
    (dict(ntok=(17, 0)), cra.EP_ERR_ARG, "num_tokens[0]"),
    (dict(ntok=(3, -1)), cra.EP_ERR_ARG, "num_tokens[1]"),
])
def test_dispatch_standard_rejects_before_launch(lib, over, code, word):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 8)
    ntok = (ctypes.c_int32 * 2)(*over.pop("ntok", (16, 5)))
    a = cra.EpDispatchStandardArgs(**standard_args(num_tokens=ctypes.addressof(ntok), **over))
    assert lib.ep_dispatch_standard_moe(ex, ctypes.byref(a), None) == code
    assert word in cra.ep_last_error()
    assert lib.ep_dispatch_standard_moe(None, ctypes.byref(a), None) == cra.EP_ERR_NULL
    assert lib.ep_dispatch_standard_moe(ex, None, None) == cra.EP_ERR_NULL
    a.num_tokens = None
    assert lib.ep_dispatch_standard_moe(ex, ctypes.byref(a), None) == cra.EP_ERR_NULL
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def test_combine_standard_scales_pairing(lib):
    """A combine wire needs the packed outputs' scale rows; no wire, none."""
    cfg = cra.make_config(8, 7168, 128, 32, 8, combine_wire="mxfp4")
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 64)
    c = cra.EpCombineStandardArgs(packed_y=FAKE, indices=FAKE + 0x1000, weights=None,
                                  out=FAKE + 0x2000, packed_y_scales=None)
    assert lib.ep_combine_standard_moe(ex, ctypes.byref(c), None) == cra.EP_ERR_NULL
    assert "packed_y_scales" in cra.ep_last_error()
    c.packed_y_scales = FAKE + 0x3002
    assert lib.ep_combine_standard_moe(ex, ctypes.byref(c), None) == cra.EP_ERR_ALIGN
    c.packed_y_scales = FAKE + 0x3000
    assert lib.ep_combine_standard_moe(ex, ctypes.byref(c), None) == cra.EP_ERR_STATE
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)
    cfg = cra.make_config(8, 7168, 128, 32, 8)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 64)
    assert lib.ep_combine_standard_moe(ex, ctypes.byref(c), None) == cra.EP_ERR_ARG
    assert "packed_y_scales" in cra.ep_last_error()
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def test_combine_standard_errors_and_state(lib):
    cfg = cra.make_config(2, 256, 16, 4, 2)
    rc, plan = make_plan(lib, cfg)
    rc, ex = make_expert(lib, plan, 8)
    ok = dict(packed_y=FAKE, indices=FAKE + 0x1000, weights=None, out=FAKE + 0x2000)
    for over, code, word in [(dict(packed_y=None), cra.EP_ERR_NULL, "packed_y"),
                             (dict(indices=None), cra.EP_ERR_NULL, "indices"),
                             (dict(out=None), cra.EP_ERR_NULL, "args.out"),
                             (dict(out=FAKE + 0x2008), cra.EP_ERR_ALIGN, "aligned"),
                             (dict(weights=FAKE + 0x3002), cra.EP_ERR_ALIGN, "weights"),
                             ({}, cra.EP_ERR_STATE, "before any dispatch_standard_moe")]:
        a = cra.EpCombineStandardArgs(**{**ok, **over})
        assert lib.ep_combine_standard_moe(ex, ctypes.byref(a), None) == code
        assert word in cra.ep_last_error()
    assert lib.ep_combine_standard_moe(None, ctypes.byref(a), None) == cra.EP_ERR_NULL
    assert lib.ep_combine_standard_moe(ex, None, None) == cra.EP_ERR_NULL
    lib.ep_expert_plan_destroy(ex)
    lib.ep_plan_destroy(plan)


def test_expert_launch_overrides(lib):
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    rc, plan = make_plan(lib, wl_config(wl))
    auto = cra.ep_plan_get_launch(plan, [4096] * 8)
    assert auto["expert_waves"] >= 1 and auto["expert_combine_waves"] >= 1
    assert 1 <= auto["expert_row_split"] <= 7168 * 2 // 16
    assert 1 <= auto["expert_combine_row_split"] <= 7168 * 2 // 16
    for bad in (dict(expert_waves=17), dict(expert_combine_waves=17),
                dict(expert_row_split=897), dict(expert_combine_row_split=897),
                dict(expert_row_split=70000), dict(expert_cache_policy=3),
                dict(expert_cache_policy=-1)):
        with pytest.raises(cra.EpError):
            cra.ep_plan_set_launch(plan, bad)
    cra.ep_plan_set_launch(plan, dict(expert_waves=2, expert_combine_row_split=3))
    got = cra.ep_plan_get_launch(plan, [4096] * 8)
    assert got["expert_waves"] == 2 and got["expert_combine_row_split"] == 3
    # a small call splits rows to fill the chip
    small = cra.ep_plan_get_launch(plan, [16] + [0] * 7)
    assert small["expert_combine_row_split"] > 1
    # the expert calls' own footprint decides their cache policy
    assert auto["expert_cache_policy"] == cra.EP_CACHE_STREAM
    assert small["expert_cache_policy"] == cra.EP_CACHE_KEEP
    lib.ep_plan_destroy(plan)


# ---------------------------------------------------------------------------
# quantized combine wire
# ---------------------------------------------------------------------------

def test_wire_combine_requires_scales(lib):
    for wire in (cra.EP_WIRE_FP8_BLOCK128, cra.EP_WIRE_MXFP4):
        cfg = cra.make_config(2, 256, 16, 4, 2, combine_wire=wire)
        rc, plan = make_plan(lib, cfg)
        assert rc == 0
        a = cra.EpCombineArgs(y=FAKE, y_weights=None, out=FAKE + 0x1000, out_weights=None,
                              y_scales=None)
        assert lib.ep_combine(plan, ctypes.byref(a), None) == cra.EP_ERR_NULL
        assert "y_scales" in cra.ep_last_error()
        a.y_scales = FAKE + 0x2002
        assert lib.ep_combine(plan, ctypes.byref(a), None) == cra.EP_ERR_ALIGN
        a.y_scales = FAKE + 0x2000
        assert lib.ep_combine(plan, ctypes.byref(a), None) == cra.EP_ERR_STATE
        lib.ep_plan_destroy(plan)


@pytest.mark.parametrize("args,code,word", [
    ((None, 4, 256, 0, 1, FAKE, FAKE + 0x1000), cra.EP_ERR_NULL, "required"),
    ((FAKE, 4, 256, 0, 1, FAKE, None), cra.EP_ERR_NULL, "required"),
    ((FAKE + 8, 4, 256, 0, 1, FAKE, FAKE + 0x1000), cra.EP_ERR_ALIGN, "aligned"),
    ((FAKE, 4, 256, 0, 1, FAKE, FAKE + 0x1002), cra.EP_ERR_ALIGN, "aligned"),
    ((FAKE, 4, 256, 2, 1, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "in_dtype"),
    ((FAKE, 4, 256, 0, 0, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "wire"),
    ((FAKE, 4, 256, 0, 3, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "wire"),
    ((FAKE, -1, 256, 0, 1, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "rows"),
    ((FAKE, 4, 192, 0, 1, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "multiple of 128"),
    ((FAKE, 4, 48, 1, 2, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "multiple of 32"),
    ((FAKE, 4, 0, 0, 2, FAKE, FAKE + 0x1000), cra.EP_ERR_ARG, "multiple of 32"),
])
def test_quantize_rows_rejects_before_launch(lib, args, code, word):
    src, rows, H, dt, wire, out, sc = args
    assert lib.ep_quantize_rows(src, rows, H, dt, wire, out, sc, None, 0, None) == code
    assert word in cra.ep_last_error()


@pytest.mark.parametrize("counts,group,code,word", [
    (FAKE + 0x3002, 2, cra.EP_ERR_ALIGN, "row_counts"),
    (FAKE + 0x3000, 0, cra.EP_ERR_ARG, "group_rows"),
    (FAKE + 0x3000, -4, cra.EP_ERR_ARG, "group_rows"),
    (FAKE + 0x3000, 3, cra.EP_ERR_ARG, "divide rows"),
    (FAKE + 0x3000, 5, cra.EP_ERR_ARG, "divide rows"),
])
def test_quantize_row_counts_checked_before_launch(lib, counts, group, code, word):
    assert lib.ep_quantize_rows(FAKE, 4, 256, 0, 1, FAKE, FAKE + 0x1000, counts, group,
                                None) == code
    assert word in cra.ep_last_error()


def test_quantize_zero_rows_is_a_no_op(lib):
    assert lib.ep_quantize_rows(FAKE, 0, 256, 0, 1, FAKE, FAKE + 0x1000, None, 0,
                                None) == cra.EP_OK
    assert lib.ep_quantize_rows(FAKE, 0, 256, 0, 2, FAKE, FAKE + 0x1000, FAKE + 0x3000, 4,
                                None) == cra.EP_OK


def test_dispatch_cast_layout_and_sizes(lib):
    cfg = cra.make_config(8, 7168, 128, 32, 8, "fp8", "bf16", dispatch_cast="bf16")
    rc, plan = make_plan(lib, cfg)
    assert rc == 0
    # a cast never runs in the all-in-copy layout
    small = cra.ep_plan_get_launch(plan, [1] + [0] * 7)
    assert small["layout"] != cra.EP_LAYOUT_IN_COPY
    with pytest.raises(cra.EpError):
        cra.ep_plan_set_launch(plan, dict(layout=cra.EP_LAYOUT_IN_COPY))
    # row pieces are counted in 16-byte vectors of the bf16 input row
    cra.ep_plan_set_launch(plan, dict(dispatch_row_split=7168 * 2 // 16))
    with pytest.raises(cra.EpError):
        cra.ep_plan_set_launch(plan, dict(dispatch_row_split=7168 * 2 // 16 + 1))
    lib.ep_plan_destroy(plan)


def test_argument_cache_keeps_no_tensor_alive():
    """The binding's argument cache holds weak references: a cached tensor
    the caller drops is freed, and a later call with a new tensor misses."""
    import gc
    import weakref

    import torch

    a, b = torch.zeros(8), torch.zeros(8)
    held = cra._hold((a, None, b))
    assert cra._same_tensors(held, (a, None, b))
    assert not cra._same_tensors(held, (b, None, a))
    assert not cra._same_tensors(held, (a, b, None))
    alive = weakref.ref(a)
    del a
    gc.collect()
    assert alive() is None
    assert not cra._same_tensors(held, (torch.zeros(8), None, b))


def test_argument_cache_misses_on_a_tensor_changed_in_place():
    """A cached tensor resized, retyped or transposed in place keeps its object
    (and maybe its address) but must be checked again."""
    import torch

    a = torch.zeros(64)
    held = cra._hold((a,))
    assert cra._same_tensors(held, (a,))
    a.resize_(32)                       # same storage, same address, fewer bytes
    assert not cra._same_tensors(held, (a,))
    b = torch.zeros(8, 8)
    held = cra._hold((b,))
    b.t_()                              # same bytes, no longer contiguous
    assert not cra._same_tensors(held, (b,))
    c = torch.zeros(16, dtype=torch.int32)
    held = cra._hold((c,))
    c.data = c.data.view(torch.float32)  # same bytes, another element type
    assert not cra._same_tensors(held, (c,))


def _headline_cfg(**kw):
    return cra.make_config(8, 7168, 64, 32, 8, kw.pop("dtype", "bf16"), **kw)


@pytest.mark.parametrize("arg,bad,word", [
    ("indices", "int64", "indices must be torch.int32"),
    ("weights", "float64", "weights must be torch.float32"),
    ("weights", "float16", "weights must be torch.float32"),
    ("x", "float32", "x must be torch.bfloat16 or torch.uint8"),
    ("recv_num_token", "int64", "recv_num_token must be torch.int32"),
])
def test_dispatch_rejects_wrong_element_types(arg, bad, word):
    """The element type is checked before anything else: int64 ids (what
    torch.topk returns) hold twice the bytes the int32 ids need, so a size
    check alone would pass them and the kernel would read every id as a pair
    of int32 words."""
    import torch

    cfg = _headline_cfg()
    args = dict(x=None, indices=None, weights=None, scales=None, out_x=None, out_indices=None,
                out_weights=None, out_scales=None, recv_num_token=None)
    args[arg] = torch.zeros(4, dtype=getattr(torch, bad))
    with pytest.raises(ValueError, match=word):
        cra._dispatch_args(cfg, [64] * 8, **args)


def test_dispatch_cast_takes_its_source_type():
    import torch

    cfg = _headline_cfg(dtype="fp8", dispatch_cast="fp16")
    with pytest.raises(ValueError, match="x must be torch.float16 or torch.uint8"):
        cra._dispatch_args(cfg, [64] * 8, torch.zeros(4, dtype=torch.bfloat16), *[None] * 8)


@pytest.mark.parametrize("wire,arg,bad", [
    (None, "y", "float32"), (None, "y_weights", "float64"), (None, "out", "float16"),
    ("fp8_block128", "y", "bfloat16"), ("fp8_block128", "y_scales", "float64"),
    ("mxfp4", "y_scales", "float32"),
])
def test_combine_rejects_wrong_element_types(wire, arg, bad):
    import torch

    cfg = _headline_cfg(combine_wire=wire)
    args = dict(y=None, y_weights=None, out=None, out_weights=None, y_scales=None)
    args[arg] = torch.zeros(4, dtype=getattr(torch, bad))
    with pytest.raises(ValueError, match=f"{arg} must be"):
        cra._combine_args(cfg, **args)


def test_expert_calls_reject_wrong_element_types():
    import torch

    cfg = _headline_cfg()
    with pytest.raises(ValueError, match="packed_layout_range must be torch.int64"):
        cra._convert_dispatch_args(cfg, 64, *[None] * 9, torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="indices must be torch.int32"):
        cra._combine_standard_args(cfg, 64, None, torch.zeros(4, dtype=torch.int64), None, None)
    with pytest.raises(ValueError, match="packed_y must be torch.bfloat16"):
        cra._convert_combine_args(cfg, 64, torch.zeros(4, dtype=torch.float16), None)


def test_device_code_has_no_packed_fp32(lib):
    """The gfx950 code of the built library holds no packed FP32 arithmetic
    (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the build turns the feature
    off for the device pass, and this reads the code object back."""
    import combine_route_amd.build as b

    if not os.path.exists("/opt/rocm/llvm/bin/clang-offload-bundler"):
        pytest.skip("ROCm LLVM tools not installed")
    counts = b.device_packed_fp32(cra.LIB_PATH)
    assert counts == {m: 0 for m in b.PACKED_FP32}, counts


def test_probe_rejects_before_launch(lib):
    """ep_probe_pattern checks every field on the host; nothing is launched."""
    def args(**kw):
        a = dict(kind=cra.EP_PROBE_FANOUT, row_bytes=1024, rows=4, src=FAKE, dst=FAKE + 0x10000,
                 map=FAKE + 0x20000, map_rows=8, stride=4, pieces=1, waves=8)
        a.update(kw)
        return cra.EpProbeArgs(**a)
    for kw, code in [(dict(kind=7), cra.EP_ERR_ARG), (dict(row_bytes=24), cra.EP_ERR_ARG),
                     (dict(rows=-1), cra.EP_ERR_ARG), (dict(pieces=0), cra.EP_ERR_ARG),
                     (dict(waves=17), cra.EP_ERR_ARG), (dict(src=None), cra.EP_ERR_NULL),
                     (dict(dst=None), cra.EP_ERR_NULL), (dict(map=None), cra.EP_ERR_NULL),
                     (dict(stride=65), cra.EP_ERR_ARG), (dict(map=FAKE + 2), cra.EP_ERR_ALIGN),
                     (dict(src=FAKE + 8), cra.EP_ERR_ALIGN),
                     (dict(rows=1 << 31), cra.EP_ERR_ARG)]:
        assert lib.ep_probe_pattern(ctypes.byref(args(**kw)), None) == code, kw
        assert cra.ep_last_error()
    assert lib.ep_probe_pattern(None, None) == cra.EP_ERR_NULL
    p = ctypes.c_void_p()
    s = ctypes.c_int32()
    assert lib.ep_probe_forward_map(None, ctypes.byref(p), ctypes.byref(s)) == cra.EP_ERR_NULL


def test_static_plan_rejects_what_does_not_fit(lib):
    """ep_plan_static checks the configuration and the static scratch's size
    before any HIP call: a workspace past EP_STATIC_SCRATCH_BYTES is refused
    with EP_ERR_SIZE, an invalid configuration with EP_ERR_ARG."""
    big = cra.make_config(8, 7168, 16384, 32, 8, "bf16")
    assert cra.ep_workspace_bytes(big) > cra.EP_STATIC_SCRATCH_BYTES
    out = ctypes.c_void_p()
    assert lib.ep_plan_static(ctypes.byref(big), ctypes.byref(out)) == cra.EP_ERR_SIZE
    assert "static scratch" in cra.ep_last_error()
    assert out.value is None
    bad = cra.make_config(0, 7168, 64, 32, 8, "bf16")
    assert lib.ep_plan_static(ctypes.byref(bad), ctypes.byref(out)) == cra.EP_ERR_ARG
    assert lib.ep_plan_static(None, ctypes.byref(out)) == cra.EP_ERR_NULL
    ok = cra.make_config(8, 7168, 4096, 32, 8, "bf16")
    assert cra.ep_workspace_bytes(ok) <= cra.EP_STATIC_SCRATCH_BYTES
    assert lib.ep_plan_static(ctypes.byref(ok), None) == cra.EP_ERR_NULL
