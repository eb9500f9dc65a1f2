"""ctypes binding of ``libmoe_topk.so`` (the C ABI in ``include/moe_topk.h``).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C calls.  PyTorch provides device memory and the HIP stream.  The
library is loaded on first use; if it is missing the call raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

from . import build as _build

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EWORKSPACE = -3
MOE_ELAUNCH = -4
MOE_ESCRATCH = -5
MOE_SCRATCH_BYTES = 1 << 20

MOE_DEVERR_EXPERT_RANGE = 0x1
MOE_DEVERR_DUP_EXPERT = 0x2
MOE_DEVERR_NO_REPLICA = 0x4
MOE_DEVERR_SRC_RANK = 0x8

MOE_F32 = 0
MOE_BF16 = 1
MOE_F_NO_RENORM = 0x1

DTYPE_CODE = {"f32": MOE_F32, "bf16": MOE_BF16}
TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {moe_strerror(code)} (code {code})")


class moe_cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("R", ctypes.c_int32), ("N", ctypes.c_int32),
                ("x_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("layout_tile", ctypes.c_int32)]


class moe_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_count", "expert_off", "rank_count", "rank_off",
        "rank_token_count", "node_mask", "node_count", "node_off",
        "node_slot", "slot_pos", "row_src")]


LAYOUT_FIELDS = [n for n, _ in moe_layout._fields_]

MOE_MAX_LEVELS = 8


class moe_capacity_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_count", "expert_cap", "expert_off", "slot_pos", "row_src",
        "dropped")]


CAP_FIELDS = [n for n, _ in moe_capacity_layout._fields_]

_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_CFG = ctypes.POINTER(moe_cfg)
_LAY = ctypes.POINTER(moe_layout)
_CAP = ctypes.POINTER(moe_capacity_layout)
_I32P = ctypes.POINTER(ctypes.c_int32)


def lib() -> ctypes.CDLL:
    """Load the HIP library (once); raise if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(
                f"{_build.LIB} is missing: build it first with "
                "`python -m combine_moe_topk_amd.build` (there is no "
                "fallback implementation)")
        L = ctypes.CDLL(_build.LIB)
        sig = {
            "moe_validate_cfg": (ctypes.c_int, [_CFG]),
            "moe_workspace_bytes": (ctypes.c_size_t, [_CFG]),
            "moe_workspace_init": (ctypes.c_int, [_P, ctypes.c_size_t, _P]),
            "moe_topk_gate": (ctypes.c_int, [_CFG, _P, _P, _P, _P]),
            "moe_dispatch_layout": (ctypes.c_int, [_CFG, _P, _LAY, _P,
                                                   ctypes.c_size_t, _P]),
            "moe_dispatch_pack": (ctypes.c_int, [_CFG, _P, _P, _P, _P]),
            "moe_combine": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P]),
            "moe_dispatch_combine": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P,
                                                    _LAY, _P, _P, _P,
                                                    ctypes.c_size_t, _P]),
            "moe_dispatch_combine_noalloc": (ctypes.c_int, [
                _CFG, _P, _P, _P, _P, _P, _LAY, _P, _P, _P]),
            "moe_node_rows_max": (ctypes.c_size_t, [_CFG]),
            "moe_dispatch_pack_nodes": (ctypes.c_int, [_CFG, _P, _P, _P, _P]),
            "moe_dispatch_forward": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P,
                                                    _P]),
            "moe_combine_partial": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P,
                                                   _P, ctypes.c_int32, _P,
                                                   _P]),
            "moe_combine_nodes": (ctypes.c_int, [_CFG, _P, ctypes.c_int32, _P,
                                                 _P, _P]),
            "moe_dispatch_combine_nodes": (ctypes.c_int, [
                _CFG, _P, _P, _P, _P, _P, _LAY, _P, _P, ctypes.c_int32, _P,
                _P, _P, ctypes.c_size_t, _P]),
            "moe_fp8_row_bytes": (ctypes.c_size_t, [ctypes.c_int32,
                                                    ctypes.c_int32]),
            "moe_dispatch_pack_fp8": (ctypes.c_int, [_CFG, _P, _P,
                                                     ctypes.c_int32, _P, _P]),
            "moe_combine_fp8": (ctypes.c_int, [_CFG, _P, ctypes.c_int32, _P,
                                               _P, _P, _P, _P, _P]),
            "moe_dispatch_combine_fp8": (ctypes.c_int, [
                _CFG, _P, _P, _P, _P, _P, _LAY, ctypes.c_int32, _P, _P, _P,
                ctypes.c_size_t, _P]),
            "moe_capacity_workspace_bytes": (ctypes.c_size_t, [_CFG]),
            "moe_dispatch_layout_capacity": (ctypes.c_int, [
                _CFG, _P, _I32P, ctypes.c_int32, _CAP, _P, ctypes.c_size_t,
                _P]),
            "moe_dispatch_pack_capacity": (ctypes.c_int, [
                _CFG, _P, _P, _P, ctypes.c_int32, _P, _P]),
            "moe_combine_capacity": (ctypes.c_int, [
                _CFG, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
            "moe_dispatch_combine_capacity": (ctypes.c_int, [
                _CFG, _P, _P, _P, _P, _P, _I32P, ctypes.c_int32, _CAP, _P, _P,
                _P, ctypes.c_size_t, _P]),
            "moe_assign_workspace_bytes": (ctypes.c_size_t, [_CFG]),
            "moe_assign_tasks": (ctypes.c_int, [
                _CFG, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
            "moe_read_device_error": (ctypes.c_int, [_P, _P,
                                                     ctypes.POINTER(ctypes.c_int32),
                                                     ctypes.c_int]),
            "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_version": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def make_cfg(T: int, H: int, E: int, K: int, R: int, N: int,
             x_dtype: str = "bf16", out_dtype: str = "bf16",
             renorm: bool = True, layout_tile: int = 0) -> moe_cfg:
    return moe_cfg(T, H, E, K, R, N, DTYPE_CODE[x_dtype],
                   DTYPE_CODE[out_dtype], 0 if renorm else MOE_F_NO_RENORM,
                   layout_tile)


# torch's current-stream handle without building a Stream object (about
# 0.3 instead of 2.8 us a call); the public route where it is missing
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, what: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _need(t: Optional[torch.Tensor], n: int, what: str) -> None:
    """Refuse a buffer smaller than the n elements cfg says a call touches.

    The kernels index buffers by cfg alone, so an undersized tensor would be
    an out-of-bounds device access; this raises before anything is enqueued
    (and before the device check, so it also holds for host tensors)."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{what}: {t.numel()} elements, the call needs "
                         f"at least {n}")


def _need_rows(t: torch.Tensor, H: int, what: str) -> int:
    """A [rows, H] buffer whose row count the call takes from its shape."""
    if t.dim() != 2 or t.shape[1] != H:
        raise ValueError(f"{what}: expected shape [rows, {H}], got "
                         f"{list(t.shape)}")
    return t.shape[0]


def _check(rc: int, what: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, what)


def moe_strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def moe_version() -> int:
    return lib().moe_version()


def moe_validate_cfg(cfg: moe_cfg) -> int:
    return lib().moe_validate_cfg(ctypes.byref(cfg))


def moe_workspace_bytes(cfg: moe_cfg) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(cfg))


def moe_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check(lib().moe_workspace_init(_ptr(ws, torch.uint8, "ws"), ws.numel(),
                                    _stream(stream)), "moe_workspace_init")


def moe_topk_gate(cfg: moe_cfg, logits: torch.Tensor, topk_idx: torch.Tensor,
                  topk_w: torch.Tensor, stream=None) -> None:
    TK = cfg.T * cfg.K
    _need(logits, cfg.T * cfg.E, "logits")
    _need(topk_idx, TK, "topk_idx")
    _need(topk_w, TK, "topk_w")
    _check(lib().moe_topk_gate(
        ctypes.byref(cfg), _ptr(logits, torch.float32, "logits"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), _stream(stream)),
        "moe_topk_gate")


@dataclasses.dataclass
class Layout:
    """Device tensors receiving the dispatch layout (see ``moe_layout``)."""

    expert_count: torch.Tensor
    expert_off: torch.Tensor
    rank_count: torch.Tensor
    rank_off: torch.Tensor
    rank_token_count: Optional[torch.Tensor]
    node_mask: Optional[torch.Tensor]
    node_count: Optional[torch.Tensor]
    node_off: Optional[torch.Tensor]
    node_slot: Optional[torch.Tensor]
    slot_pos: torch.Tensor
    row_src: torch.Tensor
    _key: Optional[tuple] = dataclasses.field(default=None, init=False,
                                              repr=False, compare=False)
    _cs: Optional[moe_layout] = dataclasses.field(default=None, init=False,
                                                  repr=False, compare=False)

    def c_struct(self, cfg: moe_cfg) -> moe_layout:
        """The C struct of these tensors, checked (type, device, size for
        cfg) and built again only when a field holds another tensor or other
        memory than last time, or cfg's sizes changed."""
        ts = [getattr(self, name) for name in LAYOUT_FIELDS]
        sizes = layout_sizes(cfg)
        key = (sizes,) + tuple(None if t is None else (id(t), t.data_ptr())
                               for t in ts)
        if key != self._key:
            for name, t, n in zip(LAYOUT_FIELDS, ts, sizes):
                _need(t, n, name)
            vals = []
            for name, t in zip(LAYOUT_FIELDS, ts):
                want = torch.int64 if name == "node_mask" else torch.int32
                vals.append(_ptr(t, want, name))
            self._cs, self._key = moe_layout(*vals), key
        return self._cs


def layout_sizes(cfg: moe_cfg) -> tuple:
    """Elements each moe_layout field must hold, in LAYOUT_FIELDS order."""
    T, E, K, R, N = cfg.T, cfg.E, cfg.K, cfg.R, cfg.N
    return (E, E + 1, R, R + 1, R, T, N, N + 1, T * N, T * K, T * K)


def alloc_layout(cfg: moe_cfg, device="cuda", optional: bool = True) -> Layout:
    """Allocate layout outputs with torch (``node_mask`` as int64 bits)."""
    def i32(n):
        return torch.empty(max(n, 0), dtype=torch.int32, device=device)
    T, E, K, R, N = cfg.T, cfg.E, cfg.K, cfg.R, cfg.N
    return Layout(
        expert_count=i32(E), expert_off=i32(E + 1), rank_count=i32(R),
        rank_off=i32(R + 1),
        rank_token_count=i32(R) if optional else None,
        node_mask=(torch.empty(T, dtype=torch.int64, device=device)
                   if optional else None),
        node_count=i32(N) if optional else None,
        node_off=i32(N + 1) if optional else None,
        node_slot=i32(T * N) if optional else None,
        slot_pos=i32(T * K), row_src=i32(T * K))


def alloc_workspace(cfg: moe_cfg, device="cuda", init: bool = True,
                    stream=None) -> torch.Tensor:
    n = moe_workspace_bytes(cfg)
    if n == 0:
        raise MoeError(moe_validate_cfg(cfg), "moe_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace not aligned to 256 B")
    if init:
        moe_workspace_init(ws, stream)
    return ws


def moe_dispatch_layout(cfg: moe_cfg, topk_idx: torch.Tensor, layout: Layout,
                        ws: torch.Tensor, stream=None) -> None:
    _need(topk_idx, cfg.T * cfg.K, "topk_idx")
    lay = layout.c_struct(cfg)
    _check(lib().moe_dispatch_layout(
        ctypes.byref(cfg), _ptr(topk_idx, torch.int32, "topk_idx"),
        ctypes.byref(lay), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_dispatch_layout")


def _row_dtype(cfg: moe_cfg):
    return TORCH_DTYPE[cfg.x_dtype]


def moe_dispatch_pack(cfg: moe_cfg, x: torch.Tensor, slot_pos: torch.Tensor,
                      send: torch.Tensor, stream=None) -> None:
    TK = cfg.T * cfg.K
    _need(x, cfg.T * cfg.H, "x")
    _need(slot_pos, TK, "slot_pos")
    _need(send, TK * cfg.H, "send")
    _check(lib().moe_dispatch_pack(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(send, _row_dtype(cfg), "send"), _stream(stream)),
        "moe_dispatch_pack")


def _need_routing(cfg: moe_cfg, slot_pos, topk_w, topk_idx, expert_scale):
    TK = cfg.T * cfg.K
    _need(slot_pos, TK, "slot_pos")
    _need(topk_w, TK, "topk_w")
    _need(topk_idx, TK, "topk_idx")
    _need(expert_scale, cfg.E, "expert_scale")


def _need_front(cfg: moe_cfg, x, logits, expert_scale, topk_idx, topk_w):
    """Sizes of the inputs and gate outputs of the fused calls."""
    TK = cfg.T * cfg.K
    _need(x, cfg.T * cfg.H, "x")
    _need(logits, cfg.T * cfg.E, "logits")
    _need(expert_scale, cfg.E, "expert_scale")
    _need(topk_idx, TK, "topk_idx")
    _need(topk_w, TK, "topk_w")


def moe_combine(cfg: moe_cfg, y: torch.Tensor, slot_pos: torch.Tensor,
                topk_w: torch.Tensor, topk_idx: Optional[torch.Tensor],
                expert_scale: Optional[torch.Tensor], out: torch.Tensor,
                stream=None) -> None:
    _need_routing(cfg, slot_pos, topk_w, topk_idx, expert_scale)
    _need(y, cfg.T * cfg.K * cfg.H, "y")
    _need(out, cfg.T * cfg.H, "out")
    _check(lib().moe_combine(
        ctypes.byref(cfg), _ptr(y, _row_dtype(cfg), "y"),
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"), _stream(stream)),
        "moe_combine")


def moe_dispatch_combine(cfg: moe_cfg, x: torch.Tensor, logits: torch.Tensor,
                         expert_scale: Optional[torch.Tensor],
                         topk_idx: torch.Tensor, topk_w: torch.Tensor,
                         layout: Layout, send: torch.Tensor, out: torch.Tensor,
                         ws: torch.Tensor, stream=None) -> None:
    _need_front(cfg, x, logits, expert_scale, topk_idx, topk_w)
    _need(send, cfg.T * cfg.K * cfg.H, "send")
    _need(out, cfg.T * cfg.H, "out")
    lay = layout.c_struct(cfg)
    _check(lib().moe_dispatch_combine(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(lay),
        _ptr(send, _row_dtype(cfg), "send"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_dispatch_combine")


def moe_dispatch_combine_noalloc(cfg: moe_cfg, x: torch.Tensor,
                                 logits: torch.Tensor,
                                 expert_scale: Optional[torch.Tensor],
                                 topk_idx: torch.Tensor, topk_w: torch.Tensor,
                                 layout: Layout, send: torch.Tensor,
                                 out: torch.Tensor, stream=None) -> None:
    """moe_dispatch_combine with the layout workspace in the library's
    static device scratch (MOE_SCRATCH_BYTES): nothing is allocated."""
    _need_front(cfg, x, logits, expert_scale, topk_idx, topk_w)
    _need(send, cfg.T * cfg.K * cfg.H, "send")
    _need(out, cfg.T * cfg.H, "out")
    lay = layout.c_struct(cfg)
    _check(lib().moe_dispatch_combine_noalloc(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(lay),
        _ptr(send, _row_dtype(cfg), "send"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"), _stream(stream)),
        "moe_dispatch_combine_noalloc")


# ---- node-level two-leg dispatch and hierarchical combine -----------------

def moe_node_rows_max(cfg: moe_cfg) -> int:
    """Rows of the leg-1 (node_send) and partial buffers: T * min(K, N)."""
    return lib().moe_node_rows_max(ctypes.byref(cfg))


def _part_code(part: torch.Tensor) -> int:
    if part.dtype == torch.float32:
        return MOE_F32
    if part.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"part: expected float32 or bfloat16, got {part.dtype}")


def _node_rows(cfg: moe_cfg) -> int:
    return cfg.T * min(cfg.K, cfg.N)


def moe_dispatch_pack_nodes(cfg: moe_cfg, x: torch.Tensor,
                            node_slot: torch.Tensor, node_send: torch.Tensor,
                            stream=None) -> None:
    _need(x, cfg.T * cfg.H, "x")
    _need(node_slot, cfg.T * cfg.N, "node_slot")
    _need(node_send, _node_rows(cfg) * cfg.H, "node_send")
    _check(lib().moe_dispatch_pack_nodes(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(node_slot, torch.int32, "node_slot"),
        _ptr(node_send, _row_dtype(cfg), "node_send"), _stream(stream)),
        "moe_dispatch_pack_nodes")


def moe_dispatch_forward(cfg: moe_cfg, node_send: torch.Tensor,
                         node_slot: torch.Tensor, topk_idx: torch.Tensor,
                         slot_pos: torch.Tensor, send: torch.Tensor,
                         stream=None) -> None:
    TK = cfg.T * cfg.K
    _need(node_send, _node_rows(cfg) * cfg.H, "node_send")
    _need(node_slot, cfg.T * cfg.N, "node_slot")
    _need(topk_idx, TK, "topk_idx")
    _need(slot_pos, TK, "slot_pos")
    _need(send, TK * cfg.H, "send")
    _check(lib().moe_dispatch_forward(
        ctypes.byref(cfg), _ptr(node_send, _row_dtype(cfg), "node_send"),
        _ptr(node_slot, torch.int32, "node_slot"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(send, _row_dtype(cfg), "send"), _stream(stream)),
        "moe_dispatch_forward")


def moe_combine_partial(cfg: moe_cfg, y: torch.Tensor, slot_pos: torch.Tensor,
                        topk_w: torch.Tensor, topk_idx: torch.Tensor,
                        expert_scale: Optional[torch.Tensor],
                        node_slot: torch.Tensor, part: torch.Tensor,
                        stream=None) -> None:
    _need_routing(cfg, slot_pos, topk_w, topk_idx, expert_scale)
    _need(y, cfg.T * cfg.K * cfg.H, "y")
    _need(node_slot, cfg.T * cfg.N, "node_slot")
    _need(part, _node_rows(cfg) * cfg.H, "part")
    _check(lib().moe_combine_partial(
        ctypes.byref(cfg), _ptr(y, _row_dtype(cfg), "y"),
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(node_slot, torch.int32, "node_slot"), _part_code(part),
        _ptr(part, None, "part"), _stream(stream)), "moe_combine_partial")


def moe_combine_nodes(cfg: moe_cfg, part: torch.Tensor,
                      node_slot: torch.Tensor, out: torch.Tensor,
                      stream=None) -> None:
    _need(part, _node_rows(cfg) * cfg.H, "part")
    _need(node_slot, cfg.T * cfg.N, "node_slot")
    _need(out, cfg.T * cfg.H, "out")
    _check(lib().moe_combine_nodes(
        ctypes.byref(cfg), _ptr(part, None, "part"), _part_code(part),
        _ptr(node_slot, torch.int32, "node_slot"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"), _stream(stream)),
        "moe_combine_nodes")


def moe_dispatch_combine_nodes(cfg: moe_cfg, x: torch.Tensor,
                               logits: torch.Tensor,
                               expert_scale: Optional[torch.Tensor],
                               topk_idx: torch.Tensor, topk_w: torch.Tensor,
                               layout: Layout, node_send: torch.Tensor,
                               send: torch.Tensor, part: torch.Tensor,
                               out: torch.Tensor, ws: torch.Tensor,
                               stream=None) -> None:
    _need_front(cfg, x, logits, expert_scale, topk_idx, topk_w)
    _need(node_send, _node_rows(cfg) * cfg.H, "node_send")
    _need(send, cfg.T * cfg.K * cfg.H, "send")
    _need(part, _node_rows(cfg) * cfg.H, "part")
    _need(out, cfg.T * cfg.H, "out")
    lay = layout.c_struct(cfg)
    _check(lib().moe_dispatch_combine_nodes(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(lay),
        _ptr(node_send, _row_dtype(cfg), "node_send"),
        _ptr(send, _row_dtype(cfg), "send"), _part_code(part),
        _ptr(part, None, "part"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_dispatch_combine_nodes")


# ---- FP8 dispatch with per-block scales -----------------------------------

def moe_fp8_row_bytes(H: int, qblock: int = 128) -> int:
    """Stride of a packed FP8 row (codes, scales, padding); 0 if unsupported."""
    return lib().moe_fp8_row_bytes(H, qblock)


def _fp8_rb(cfg: moe_cfg, qblock: int) -> int:
    # 0 for an unsupported (H, qblock): the C call then refuses it
    return moe_fp8_row_bytes(cfg.H, qblock)


def moe_dispatch_pack_fp8(cfg: moe_cfg, x: torch.Tensor,
                          slot_pos: torch.Tensor, send: torch.Tensor,
                          qblock: int = 128, stream=None) -> None:
    _need(x, cfg.T * cfg.H, "x")
    _need(slot_pos, cfg.T * cfg.K, "slot_pos")
    _need(send, cfg.T * cfg.K * _fp8_rb(cfg, qblock), "send")
    _check(lib().moe_dispatch_pack_fp8(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(slot_pos, torch.int32, "slot_pos"), qblock,
        _ptr(send, torch.uint8, "send"), _stream(stream)),
        "moe_dispatch_pack_fp8")


def moe_combine_fp8(cfg: moe_cfg, y: torch.Tensor, slot_pos: torch.Tensor,
                    topk_w: torch.Tensor, topk_idx: Optional[torch.Tensor],
                    expert_scale: Optional[torch.Tensor], out: torch.Tensor,
                    qblock: int = 128, stream=None) -> None:
    _need_routing(cfg, slot_pos, topk_w, topk_idx, expert_scale)
    _need(y, cfg.T * cfg.K * _fp8_rb(cfg, qblock), "y")
    _need(out, cfg.T * cfg.H, "out")
    _check(lib().moe_combine_fp8(
        ctypes.byref(cfg), _ptr(y, torch.uint8, "y"), qblock,
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"), _stream(stream)),
        "moe_combine_fp8")


def moe_dispatch_combine_fp8(cfg: moe_cfg, x: torch.Tensor,
                             logits: torch.Tensor,
                             expert_scale: Optional[torch.Tensor],
                             topk_idx: torch.Tensor, topk_w: torch.Tensor,
                             layout: Layout, send: torch.Tensor,
                             out: torch.Tensor, ws: torch.Tensor,
                             qblock: int = 128, stream=None) -> None:
    _need_front(cfg, x, logits, expert_scale, topk_idx, topk_w)
    _need(send, cfg.T * cfg.K * _fp8_rb(cfg, qblock), "send")
    _need(out, cfg.T * cfg.H, "out")
    lay = layout.c_struct(cfg)
    _check(lib().moe_dispatch_combine_fp8(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), ctypes.byref(lay), qblock,
        _ptr(send, torch.uint8, "send"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_dispatch_combine_fp8")


# ---- capacity-padded and bucketed layout ----------------------------------

@dataclasses.dataclass
class CapacityLayout:
    """Device tensors receiving the capacity layout (``moe_capacity_layout``)."""

    expert_count: torch.Tensor
    expert_cap: torch.Tensor
    expert_off: torch.Tensor
    slot_pos: torch.Tensor
    row_src: torch.Tensor
    dropped: torch.Tensor

    def c_struct(self, cfg: moe_cfg, levels) -> moe_capacity_layout:
        E = cfg.E
        sizes = (E, E, E + 1, cfg.T * cfg.K, E * int(levels[-1]), 1)
        for n, k in zip(CAP_FIELDS, sizes):
            _need(getattr(self, n), k, n)
        return moe_capacity_layout(*[_ptr(getattr(self, n), torch.int32, n)
                                     for n in CAP_FIELDS])


def alloc_capacity_layout(cfg: moe_cfg, levels, device="cuda") -> CapacityLayout:
    def i32(n):
        return torch.empty(max(n, 0), dtype=torch.int32, device=device)
    cmax = int(levels[-1])
    return CapacityLayout(expert_count=i32(cfg.E), expert_cap=i32(cfg.E),
                          expert_off=i32(cfg.E + 1),
                          slot_pos=i32(cfg.T * cfg.K),
                          row_src=i32(cfg.E * cmax), dropped=i32(1))


def alloc_capacity_workspace(cfg: moe_cfg, device="cuda",
                             stream=None) -> torch.Tensor:
    n = lib().moe_capacity_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(moe_validate_cfg(cfg), "moe_capacity_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def _levels(levels):
    arr = (ctypes.c_int32 * len(levels))(*[int(v) for v in levels])
    return arr, len(levels)


def moe_dispatch_layout_capacity(cfg: moe_cfg, topk_idx: torch.Tensor, levels,
                                 layout: CapacityLayout, ws: torch.Tensor,
                                 stream=None) -> None:
    lv, q = _levels(levels)
    _need(topk_idx, cfg.T * cfg.K, "topk_idx")
    lay = layout.c_struct(cfg, levels)
    _check(lib().moe_dispatch_layout_capacity(
        ctypes.byref(cfg), _ptr(topk_idx, torch.int32, "topk_idx"), lv, q,
        ctypes.byref(lay), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)), "moe_dispatch_layout_capacity")


def moe_dispatch_pack_capacity(cfg: moe_cfg, x: torch.Tensor,
                               slot_pos: torch.Tensor, row_src: torch.Tensor,
                               send: torch.Tensor, stream=None) -> None:
    n_rows = _need_rows(send, cfg.H, "send")
    _need(row_src, n_rows, "row_src")
    _need(x, cfg.T * cfg.H, "x")
    _need(slot_pos, cfg.T * cfg.K, "slot_pos")
    _check(lib().moe_dispatch_pack_capacity(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(row_src, torch.int32, "row_src"), send.shape[0],
        _ptr(send, _row_dtype(cfg), "send"), _stream(stream)),
        "moe_dispatch_pack_capacity")


def moe_combine_capacity(cfg: moe_cfg, y: torch.Tensor, slot_pos: torch.Tensor,
                         topk_w: torch.Tensor, topk_idx: Optional[torch.Tensor],
                         expert_scale: Optional[torch.Tensor],
                         out: torch.Tensor, stream=None) -> None:
    _need_rows(y, cfg.H, "y")
    _need_routing(cfg, slot_pos, topk_w, topk_idx, expert_scale)
    _need(out, cfg.T * cfg.H, "out")
    _check(lib().moe_combine_capacity(
        ctypes.byref(cfg), _ptr(y, _row_dtype(cfg), "y"), y.shape[0],
        _ptr(slot_pos, torch.int32, "slot_pos"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"), _stream(stream)),
        "moe_combine_capacity")


def moe_dispatch_combine_capacity(cfg: moe_cfg, x: torch.Tensor,
                                  logits: torch.Tensor,
                                  expert_scale: Optional[torch.Tensor],
                                  topk_idx: torch.Tensor, topk_w: torch.Tensor,
                                  levels, layout: CapacityLayout,
                                  send: torch.Tensor, out: torch.Tensor,
                                  ws: torch.Tensor, stream=None) -> None:
    lv, q = _levels(levels)
    if _need_rows(send, cfg.H, "send") != cfg.E * int(levels[-1]):
        raise ValueError("send must have E * levels[-1] rows")
    _need_front(cfg, x, logits, expert_scale, topk_idx, topk_w)
    _need(out, cfg.T * cfg.H, "out")
    lay = layout.c_struct(cfg, levels)
    _check(lib().moe_dispatch_combine_capacity(
        ctypes.byref(cfg), _ptr(x, _row_dtype(cfg), "x"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(expert_scale, torch.float32, "expert_scale"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), lv, q, ctypes.byref(lay),
        _ptr(send, _row_dtype(cfg), "send"),
        _ptr(out, TORCH_DTYPE[cfg.out_dtype], "out"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_dispatch_combine_capacity")


# ---- communication-aware task assignment -----------------------------------

def alloc_assign_workspace(cfg: moe_cfg, device="cuda",
                           stream=None) -> torch.Tensor:
    n = lib().moe_assign_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(moe_validate_cfg(cfg), "moe_assign_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def moe_assign_tasks(cfg: moe_cfg, topk_idx: torch.Tensor,
                     src_rank: torch.Tensor, holds: torch.Tensor,
                     u_node: torch.Tensor, u_rank: torch.Tensor,
                     assign_rank: torch.Tensor, remote_mask: torch.Tensor,
                     ws: torch.Tensor, stream=None) -> None:
    """holds: uint8 [R, E]; u_node/u_rank: int32 views of uint32 draws;
    remote_mask: int64 (bit n = node n)."""
    if holds.numel() != cfg.R * cfg.E:
        raise ValueError("holds must be [R, E]")
    TK = cfg.T * cfg.K
    for t, n, what in ((topk_idx, TK, "topk_idx"), (src_rank, cfg.T, "src_rank"),
                       (u_node, TK, "u_node"), (u_rank, TK, "u_rank"),
                       (assign_rank, TK, "assign_rank"),
                       (remote_mask, cfg.T, "remote_mask")):
        _need(t, n, what)
    _check(lib().moe_assign_tasks(
        ctypes.byref(cfg), _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(src_rank, torch.int32, "src_rank"),
        _ptr(holds, torch.uint8, "holds"), _ptr(u_node, torch.int32, "u_node"),
        _ptr(u_rank, torch.int32, "u_rank"),
        _ptr(assign_rank, torch.int32, "assign_rank"),
        _ptr(remote_mask, torch.int64, "remote_mask"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
        "moe_assign_tasks")


def moe_read_device_error(ws: torch.Tensor, clear: bool = True,
                          stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().moe_read_device_error(_ptr(ws, torch.uint8, "ws"),
                                       _stream(stream), ctypes.byref(code),
                                       int(bool(clear))),
           "moe_read_device_error")
    return code.value
