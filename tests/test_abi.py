"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-only calls (validation, workspace sizing, error text)
behave as documented.  No call here touches a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_moe_topk_amd as moe
from combine_moe_topk_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_topk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_topk_gate", "moe_dispatch_layout", "moe_dispatch_pack",
              "moe_combine", "moe_dispatch_combine", "moe_workspace_bytes",
              "moe_validate_cfg", "moe_read_device_error", "moe_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", libbuild.LIB],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (moe_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_struct_layout_matches_header():
    # the header's moe_cfg: ten 4-byte fields; moe_layout: eleven pointers
    assert ctypes.sizeof(moe.moe_cfg) == 40
    assert ctypes.sizeof(moe.moe_layout) == 11 * 8


def cfg(**kw):
    base = dict(T=16384, H=7168, E=256, K=8, R=64, N=8)
    base.update(kw)
    return moe.make_cfg(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, moe.MOE_OK),
    ({"T": 0}, moe.MOE_OK),
    ({"T": -1}, moe.MOE_EINVAL),
    ({"H": 0}, moe.MOE_EINVAL),
    ({"E": 0}, moe.MOE_EINVAL),
    ({"K": 0}, moe.MOE_EINVAL),
    ({"K": 257}, moe.MOE_EINVAL),
    ({"K": 33, "E": 512, "R": 64}, moe.MOE_EINVAL),
    ({"E": 250}, moe.MOE_EINVAL),          # E % R != 0
    ({"R": 64, "N": 3}, moe.MOE_EINVAL),   # R % N != 0
    ({"E": 8192, "R": 64}, moe.MOE_EINVAL),
    ({"E": 128, "R": 128, "N": 128}, moe.MOE_EINVAL),  # N > 64
    ({"T": 1 << 28, "K": 8}, moe.MOE_EINVAL),  # T*K overflows int32
    ({"H": 7164}, moe.MOE_EUNSUPPORTED),   # not a multiple of 8
    ({"x_dtype": "f32", "out_dtype": "bf16"}, moe.MOE_OK),
    ({"layout_tile": 1024}, moe.MOE_OK),
    ({"T": 2**31 - 4097, "K": 1}, moe.MOE_OK),
    ({"T": 2**31 - 4096, "K": 1}, moe.MOE_EINVAL),  # no tile headroom
])
def test_validate_cfg(kw, code):
    assert moe.moe_validate_cfg(cfg(**kw)) == code


def test_validate_rejects_bad_tile_flags_dtype():
    c = cfg()
    c.layout_tile = 100
    assert moe.moe_validate_cfg(c) == moe.MOE_EINVAL
    c = cfg()
    c.flags = 0x80
    assert moe.moe_validate_cfg(c) == moe.MOE_EINVAL
    c = cfg()
    c.x_dtype = 7
    assert moe.moe_validate_cfg(c) == moe.MOE_EUNSUPPORTED
    assert moe.lib().moe_validate_cfg(None) == moe.MOE_EINVAL


def test_workspace_bytes():
    def ws(T, tile, cols=256 + 64 + 8):
        # 256-byte header + (ceil(T/tile) + 1) rows of (E + R + N) int32
        rows = -(-T // tile) + 1
        return 256 + ((rows * cols * 4 + 255) // 256) * 256

    n = moe.moe_workspace_bytes(cfg(layout_tile=256))
    assert n == ws(16384, 256)
    assert n % 256 == 0
    assert moe.moe_workspace_bytes(cfg(T=-1)) == 0
    # smaller tiles need more rows; results do not depend on the tile
    assert moe.moe_workspace_bytes(cfg(layout_tile=64)) > n
    # default tile: 256 halved (to 64 at least) while under 91 tiles and a
    # table of at most 256 KiB; one 256-token tile up to 256 tokens
    assert moe.moe_workspace_bytes(cfg()) == ws(16384, 128)
    assert moe.moe_workspace_bytes(cfg(T=32768)) == ws(32768, 256)
    assert moe.moe_workspace_bytes(cfg(T=8192)) == ws(8192, 64)
    assert moe.moe_workspace_bytes(cfg(T=200)) == ws(200, 256)
    assert moe.moe_workspace_bytes(cfg(T=300)) == ws(300, 64)
    # E = 896, R = 128, N = 16 at 8192 tokens: tile 128 would need a
    # 65-row table of 1040 columns (> 256 KiB), so 256 stays
    wide = cfg(T=8192, E=896, K=16, R=128, N=16)
    assert moe.moe_workspace_bytes(wide) == ws(8192, 256, 896 + 128 + 16)
    # empty input still needs the header and the offsets row
    assert moe.moe_workspace_bytes(cfg(T=0)) > 256


def test_strerror_and_version():
    assert moe.moe_strerror(0) == "success"
    for c in (moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED, moe.MOE_EWORKSPACE,
              moe.MOE_ELAUNCH):
        assert moe.moe_strerror(c) != "unknown error code"
    assert moe.moe_strerror(12345) == "unknown error code"
    assert moe.moe_version() >= 10000


def test_host_validation_before_any_device_work():
    # invalid arguments are rejected on the host, so these calls return
    # before touching HIP even on a machine without a GPU
    lib = moe.lib()
    c = cfg()
    assert lib.moe_topk_gate(ctypes.byref(c), None, None, None, None) == moe.MOE_EINVAL
    bad = cfg(E=250)
    assert lib.moe_dispatch_pack(ctypes.byref(bad), None, None, None, None) == moe.MOE_EINVAL
    lay = moe.moe_layout()
    assert lib.moe_dispatch_layout(ctypes.byref(c), None, ctypes.byref(lay),
                                   None, 0, None) == moe.MOE_EINVAL
    assert lib.moe_workspace_init(None, 0, None) == moe.MOE_EWORKSPACE
    assert lib.moe_read_device_error(None, None, None, 0) == moe.MOE_EINVAL


def test_node_entry_points_declared_and_validated():
    names = declared_functions()
    for n in ("moe_node_rows_max", "moe_dispatch_pack_nodes",
              "moe_dispatch_forward", "moe_combine_partial",
              "moe_combine_nodes", "moe_dispatch_combine_nodes"):
        assert n in names
    c = cfg()
    assert moe.moe_node_rows_max(c) == 16384 * 8          # T * min(K, N)
    assert moe.moe_node_rows_max(cfg(K=2, N=1, R=8, E=8)) == 16384
    assert moe.moe_node_rows_max(cfg(E=250)) == 0
    lib = moe.lib()
    assert lib.moe_dispatch_pack_nodes(ctypes.byref(c), None, None, None,
                                       None) == moe.MOE_EINVAL
    assert lib.moe_dispatch_forward(ctypes.byref(c), None, None, None, None,
                                    None, None) == moe.MOE_EINVAL
    # a partial type other than f32/bf16 is refused before any pointer check
    assert lib.moe_combine_partial(ctypes.byref(c), None, None, None, None,
                                   None, None, 5, None, None) == moe.MOE_EUNSUPPORTED
    assert lib.moe_combine_nodes(ctypes.byref(c), None, 5, None, None,
                                 None) == moe.MOE_EUNSUPPORTED
    assert lib.moe_combine_nodes(ctypes.byref(c), None, moe.MOE_BF16, None,
                                 None, None) == moe.MOE_EINVAL
    lay = moe.moe_layout()
    assert lib.moe_dispatch_combine_nodes(
        ctypes.byref(c), None, None, None, None, None, ctypes.byref(lay),
        None, None, moe.MOE_BF16, None, None, None, 0, None) == moe.MOE_EINVAL


def test_capacity_entry_points_validate_on_host():
    names = declared_functions()
    for n in ("moe_capacity_workspace_bytes", "moe_dispatch_layout_capacity",
              "moe_dispatch_pack_capacity", "moe_combine_capacity",
              "moe_dispatch_combine_capacity", "moe_fp8_row_bytes",
              "moe_dispatch_pack_fp8", "moe_combine_fp8",
              "moe_dispatch_combine_fp8"):
        assert n in names
    assert ctypes.sizeof(moe.moe_capacity_layout) == 6 * 8
    c = cfg()
    ws = moe.lib().moe_capacity_workspace_bytes(ctypes.byref(c))
    assert ws > moe.moe_workspace_bytes(c) + 16384 * 8 * 4
    lib = moe.lib()
    lay = moe.moe_capacity_layout()
    lv = (ctypes.c_int32 * 3)(64, 32, 128)           # not increasing
    assert lib.moe_dispatch_layout_capacity(ctypes.byref(c), None, lv, 3,
                                            ctypes.byref(lay), None, 0,
                                            None) == moe.MOE_EINVAL
    lv = (ctypes.c_int32 * 9)(*range(1, 10))          # too many levels
    assert lib.moe_dispatch_layout_capacity(ctypes.byref(c), None, lv, 9,
                                            ctypes.byref(lay), None, 0,
                                            None) == moe.MOE_EINVAL
    assert moe.moe_fp8_row_bytes(7168, 128) == 7424     # 7168 + 224, to 128
    assert moe.moe_fp8_row_bytes(256, 128) == 384      # 256 + 8, to 128
    assert moe.moe_fp8_row_bytes(7168, 32) == 8064     # 7168 + 896, exact
    assert moe.moe_fp8_row_bytes(100, 32) == 0
    # the FP8 pack holds each row's scale-and-padding tail in LDS: a tail
    # above 16 KiB (H/B scales of 4 bytes) is refused on the host
    for H, B, code in ((7168, 32, moe.MOE_EINVAL), (131072, 32, moe.MOE_EINVAL),
                       (131200, 32, moe.MOE_EUNSUPPORTED)):
        c = cfg(T=4, H=H)
        assert lib.moe_dispatch_pack_fp8(ctypes.byref(c), None, None, B, None,
                                         None) == code, (H, B)


def test_assign_entry_point_validates_on_host():
    assert "moe_assign_tasks" in declared_functions()
    c = cfg()
    assert moe.lib().moe_assign_workspace_bytes(ctypes.byref(c)) == \
        256 + 256 * 8 + 256 * 8 * 8
    lib = moe.lib()
    assert lib.moe_assign_tasks(ctypes.byref(c), None, None, None, None, None,
                                None, None, None, 0, None) == moe.MOE_EINVAL


def test_assign_refuses_more_than_24_nodes_on_host():
    # the cover search tests up to 2^(N-1) node subsets per token ("Cobalt",
    # Section 3.3): above 24 nodes the call is refused on the host, before
    # any pointer is looked at or anything is enqueued
    lib = moe.lib()
    for N, R, ok in ((24, 48, True), (25, 50, False), (32, 64, False),
                     (64, 64, False)):
        c = cfg(E=R * 4, R=R, N=N)
        assert moe.moe_validate_cfg(c) == moe.MOE_OK
        ws = lib.moe_assign_workspace_bytes(ctypes.byref(c))
        rc = lib.moe_assign_tasks(ctypes.byref(c), None, None, None, None,
                                  None, None, None, None, 0, None)
        if ok:
            assert ws > 0
            assert rc == moe.MOE_EINVAL  # past the node bound: null holds
        else:
            assert ws == 0
            assert rc == moe.MOE_EUNSUPPORTED
    with pytest.raises(moe.MoeError):
        moe.alloc_assign_workspace(cfg(E=256, R=64, N=32), device="cpu")


def _host(n, dtype):
    import torch
    return torch.zeros(n, dtype=dtype)


def test_binding_refuses_undersized_buffers_before_any_call():
    # every wrapper checks each buffer's element count against cfg before
    # the device check and before the C call; host tensors suffice here
    import torch
    c = moe.make_cfg(T=100, H=64, E=16, K=4, R=4, N=2)
    TK, TH = 400, 100 * 64
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32

    def refused(fn, name):
        with pytest.raises(ValueError, match=name):
            fn()

    refused(lambda: moe.moe_topk_gate(c, _host(100 * 16 - 1, f32),
                                      _host(TK, i32), _host(TK, f32)),
            "logits")
    refused(lambda: moe.moe_topk_gate(c, _host(1600, f32), _host(TK - 1, i32),
                                      _host(TK, f32)), "topk_idx")
    refused(lambda: moe.moe_dispatch_pack(c, _host(TH, bf), _host(TK, i32),
                                          _host(TK * 64 - 8, bf)), "send")
    refused(lambda: moe.moe_dispatch_pack(c, _host(TH - 64, bf),
                                          _host(TK, i32), _host(TK * 64, bf)),
            "x")
    refused(lambda: moe.moe_combine(c, _host(TK * 64, bf), _host(TK, i32),
                                    _host(TK, f32), None, None,
                                    _host(TH - 1, bf)), "out")
    refused(lambda: moe.moe_combine(c, _host(TK * 64, bf), _host(TK, i32),
                                    _host(TK, f32), _host(TK, i32),
                                    _host(15, f32), _host(TH, bf)),
            "expert_scale")
    lay = moe.alloc_layout(c, device="cpu")
    lay.slot_pos = _host(TK - 1, i32)
    refused(lambda: moe.moe_dispatch_layout(c, _host(TK, i32), lay,
                                            _host(1 << 16, torch.uint8)),
            "slot_pos")
    lay = moe.alloc_layout(c, device="cpu")
    lay.node_slot = _host(100 * 2 - 1, i32)
    refused(lambda: moe.moe_dispatch_combine(
        c, _host(TH, bf), _host(1600, f32), None, _host(TK, i32),
        _host(TK, f32), lay, _host(TK * 64, bf), _host(TH, bf),
        _host(1 << 16, torch.uint8)), "node_slot")
    refused(lambda: moe.moe_dispatch_combine(
        c, _host(TH, bf), _host(1600, f32), None, _host(TK, i32),
        _host(TK, f32), moe.alloc_layout(c, device="cpu"),
        _host(TK * 64 - 1, bf), _host(TH, bf), _host(1 << 16, torch.uint8)),
        "send")
    # node-level buffers hold T * min(K, N) rows
    refused(lambda: moe.moe_dispatch_pack_nodes(
        c, _host(TH, bf), _host(200, i32), _host(200 * 64 - 1, bf)),
        "node_send")
    refused(lambda: moe.moe_combine_nodes(
        c, _host(200 * 64, f32), _host(200, i32), _host(TH - 1, bf)), "out")
    # FP8 rows: round_up(H + 4 H / B, 128) bytes each (256 for H = 64)
    rb = moe.moe_fp8_row_bytes(64, 32)
    assert rb == 128
    refused(lambda: moe.moe_dispatch_pack_fp8(
        c, _host(TH, bf), _host(TK, i32), _host(TK * rb - 1, torch.uint8),
        qblock=32), "send")
    # capacity: row_src needs one entry per send row
    refused(lambda: moe.moe_dispatch_pack_capacity(
        c, _host(TH, bf), _host(TK, i32), _host(99, i32),
        torch.zeros((100, 64), dtype=bf)), "row_src")
    refused(lambda: moe.moe_combine_capacity(
        c, torch.zeros((100, 63), dtype=bf), _host(TK, i32), _host(TK, f32),
        None, None, _host(TH, bf)), "y")
    # assignment
    refused(lambda: moe.moe_assign_tasks(
        c, _host(TK, i32), _host(99, i32), torch.zeros(64, dtype=torch.uint8),
        _host(TK, i32), _host(TK, i32), _host(TK, i32),
        _host(100, torch.int64), _host(1 << 16, torch.uint8)), "src_rank")
    # correctly sized host tensors pass the size checks and stop at the
    # device check, still before the C call
    with pytest.raises(ValueError, match="device tensor"):
        moe.moe_dispatch_pack(c, _host(TH, bf), _host(TK, i32),
                              _host(TK * 64, bf))
