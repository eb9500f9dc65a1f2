"""CPU oracle for the MoE dispatch/combine path (ctypes over ``moe_ref.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the HIP path; both are fed from ``moe_inputs``.

Each function follows the definition stated in ``moe_ref.c`` (gate:
"Efficient and portable mixture-of-experts communication", "Introdución";
layout: the same page's "Envío (Dispatch)" section, Cobalt Section 1 for node-level
deduplication and the OCS decode paper's "Variable MoE Traffic and
Regularization" for per-destination row counts; pack and combine: the same
blog's "Envío (Dispatch)" and "Combinación (Combine)" sections; the two-leg
node-level dispatch and the per-node partial combine: Cobalt Section 1 and
"MoX: Efficient MoE Routing on Direct-Connect Topologies" Section 2.5; the
FP8 dispatch with block scales: the blog's "Envío (Dispatch)" and the OCS
decode paper's "Communication precision"; the capacity-padded and bucketed
layout: the decode paper's "Variable MoE Traffic and Regularization"; the task
assignment: Cobalt Section 3.3).  All are pinned by the CPU tests.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

_LIB: Optional[ctypes.CDLL] = None

DT_F32 = 0
DT_BF16 = 1

_P = ctypes.c_void_p


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.moe_ref_gate.argtypes = [ctypes.c_int] * 4 + [_P, _P, _P]
        lib.moe_ref_layout.argtypes = [ctypes.c_int] * 5 + [_P] * 12
        lib.moe_ref_pack.argtypes = [ctypes.c_int, ctypes.c_int,
                                     ctypes.c_size_t, _P, _P, _P]
        lib.moe_ref_combine.argtypes = ([ctypes.c_int] * 4 + [_P] * 5 +
                                        [ctypes.c_int, _P, _P])
        lib.moe_ref_combine_tokens.argtypes = (
            [ctypes.c_int, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int] +
            [_P] * 6)
        lib.moe_ref_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.moe_ref_f64_to_bf16.restype = ctypes.c_uint16
        lib.moe_ref_pack_nodes.argtypes = [ctypes.c_int, ctypes.c_int,
                                           ctypes.c_size_t, _P, _P,
                                           ctypes.c_int, _P]
        lib.moe_ref_forward.argtypes = ([ctypes.c_int] * 5 +
                                        [ctypes.c_size_t, _P, ctypes.c_int] +
                                        [_P] * 4)
        lib.moe_ref_combine_partial.argtypes = (
            [ctypes.c_int] * 7 + [_P] * 6 + [ctypes.c_int, ctypes.c_int,
                                            _P, _P])
        lib.moe_ref_combine_partial_f32.argtypes = (
            [ctypes.c_int] * 7 + [_P] * 6 + [ctypes.c_int, ctypes.c_int,
                                            _P, _P])
        lib.moe_ref_combine_nodes.argtypes = (
            [ctypes.c_int] * 4 + [_P, ctypes.c_int, _P, ctypes.c_int, _P,
                                  _P])
        lib.moe_ref_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.moe_ref_e4m3_value.restype = ctypes.c_double
        lib.moe_ref_e4m3_code.argtypes = [ctypes.c_double]
        lib.moe_ref_e4m3_code.restype = ctypes.c_uint8
        lib.moe_ref_fp8_row_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.moe_ref_fp8_row_bytes.restype = ctypes.c_size_t
        lib.moe_ref_pack_fp8.argtypes = [ctypes.c_int] * 5 + [_P] * 3
        lib.moe_ref_combine_fp8.argtypes = ([ctypes.c_int] * 4 + [_P] * 5 +
                                            [ctypes.c_int, _P, _P])
        lib.moe_ref_layout_capacity.argtypes = ([ctypes.c_int] * 3 +
                                                [_P, _P, ctypes.c_int] +
                                                [_P] * 6)
        lib.moe_ref_pack_capacity.argtypes = [ctypes.c_int, ctypes.c_int,
                                              ctypes.c_size_t, _P, _P,
                                              ctypes.c_int, _P]
        lib.moe_ref_assign.argtypes = [ctypes.c_int] * 5 + [_P] * 7
        lib.moe_ref_assign.restype = ctypes.c_int
        for f in ("moe_ref_pack_fp8", "moe_ref_combine_fp8",
                  "moe_ref_layout_capacity", "moe_ref_pack_capacity"):
            getattr(lib, f).restype = ctypes.c_int
        for f in ("moe_ref_gate", "moe_ref_layout", "moe_ref_pack",
                  "moe_ref_combine", "moe_ref_combine_tokens",
                  "moe_ref_pack_nodes", "moe_ref_forward",
                  "moe_ref_combine_partial", "moe_ref_combine_partial_f32",
                  "moe_ref_combine_nodes"):
            getattr(lib, f).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (code {rc})")


def gate(logits: np.ndarray, K: int, renorm: bool = True):
    """Top-K experts per token and their gate weights.

    Returns ``(topk_idx int32 [T,K], topk_w fp32 [T,K])``.
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, K), dtype=np.int32)
    w = np.empty((T, K), dtype=np.float32)
    _check(_lib().moe_ref_gate(T, E, K, int(bool(renorm)), _ptr(logits),
                               _ptr(idx), _ptr(w)), "gate")
    return idx, w


def layout(topk_idx: np.ndarray, E: int, R: int, N: int,
           with_node_slot: bool = True) -> dict:
    """Dispatch layout of ``topk_idx`` (int32 [T,K]); see ``moe_ref.c``."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = topk_idx.shape
    o = {
        "expert_count": np.empty(E, np.int32),
        "expert_off": np.empty(E + 1, np.int32),
        "rank_count": np.empty(R, np.int32),
        "rank_off": np.empty(R + 1, np.int32),
        "rank_token_count": np.empty(R, np.int32),
        "node_mask": np.empty(T, np.uint64),
        "node_count": np.empty(N, np.int32),
        "node_off": np.empty(N + 1, np.int32),
        "node_slot": np.empty((T, N), np.int32) if with_node_slot else None,
        "slot_pos": np.empty((T, K), np.int32),
        "row_src": np.empty(T * K, np.int32),
    }
    _check(_lib().moe_ref_layout(
        T, E, K, R, N, _ptr(topk_idx), _ptr(o["expert_count"]),
        _ptr(o["expert_off"]), _ptr(o["rank_count"]), _ptr(o["rank_off"]),
        _ptr(o["rank_token_count"]), _ptr(o["node_mask"]),
        _ptr(o["node_count"]), _ptr(o["node_off"]), _ptr(o["node_slot"]),
        _ptr(o["slot_pos"]), _ptr(o["row_src"])), "layout")
    if not with_node_slot:
        del o["node_slot"]
    return o


def pack(x: np.ndarray, slot_pos: np.ndarray) -> np.ndarray:
    """``send[slot_pos[t,k]] = x[t]`` bit for bit; returns send [T*K, H]."""
    x = np.ascontiguousarray(x)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    T, K = slot_pos.shape
    assert x.shape[0] == T
    send = np.empty((T * K,) + x.shape[1:], dtype=x.dtype)
    row_bytes = x[0].nbytes if T > 0 else 0
    _check(_lib().moe_ref_pack(T, K, row_bytes, _ptr(x), _ptr(slot_pos),
                               _ptr(send)), "pack")
    return send


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    raise TypeError(f"rows must be fp32 or bf16 bits (uint16), got {a.dtype}")


def combine(y: np.ndarray, slot_pos: np.ndarray, topk_w: np.ndarray,
            topk_idx: Optional[np.ndarray] = None,
            expert_scale: Optional[np.ndarray] = None,
            out_dtype: str = "bf16"):
    """Gate-weighted sum of each token's K expert rows.

    Returns ``(out, exact)``: ``out`` rounded to nearest-even in ``out_dtype``
    (fp32, or bf16 bits as uint16) and ``exact`` the unrounded fp64 sums.
    """
    y = np.ascontiguousarray(y)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, K = slot_pos.shape
    H = y.shape[1]
    if expert_scale is not None:
        expert_scale = np.ascontiguousarray(expert_scale, dtype=np.float32)
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    ocode = DT_F32 if out_dtype == "f32" else DT_BF16
    out = np.empty((T, H), np.float32 if ocode == DT_F32 else np.uint16)
    exact = np.empty((T, H), np.float64)
    _check(_lib().moe_ref_combine(
        T, H, K, _dtype_code(y), _ptr(y), _ptr(slot_pos), _ptr(topk_w),
        _ptr(topk_idx), _ptr(expert_scale), ocode, _ptr(out), _ptr(exact)),
        "combine")
    return out, exact


def combine_tokens(tokens: np.ndarray, y: np.ndarray, slot_pos: np.ndarray,
                   topk_w: np.ndarray, topk_idx: Optional[np.ndarray] = None,
                   expert_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Unrounded fp64 combine of the listed tokens only ([len(tokens), H])."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    y = np.ascontiguousarray(y)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    K = slot_pos.shape[1]
    H = y.shape[1]
    if expert_scale is not None:
        expert_scale = np.ascontiguousarray(expert_scale, dtype=np.float32)
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    exact = np.empty((len(tokens), H), np.float64)
    _check(_lib().moe_ref_combine_tokens(
        len(tokens), _ptr(tokens), H, K, _dtype_code(y), _ptr(y),
        _ptr(slot_pos), _ptr(topk_w), _ptr(topk_idx), _ptr(expert_scale),
        _ptr(exact)), "combine_tokens")
    return exact


def node_rows(node_slot: np.ndarray) -> int:
    """Rows of the leg-1 buffer: the number of (token, node) crossings."""
    return int(np.count_nonzero(np.asarray(node_slot) >= 0))


def pack_nodes(x: np.ndarray, node_slot: np.ndarray) -> np.ndarray:
    """Leg 1: ``node_send[node_slot[t,n]] = x[t]`` for every crossing.

    Returns node_send [D, H] with D = number of crossings.
    """
    x = np.ascontiguousarray(x)
    node_slot = np.ascontiguousarray(node_slot, dtype=np.int32)
    T, N = node_slot.shape
    D = node_rows(node_slot)
    out = np.zeros((D,) + x.shape[1:], dtype=x.dtype)
    row_bytes = x[0].nbytes if T > 0 else 0
    _check(_lib().moe_ref_pack_nodes(T, N, row_bytes, _ptr(x),
                                     _ptr(node_slot), D, _ptr(out)),
           "pack_nodes")
    return out


def forward(node_send: np.ndarray, node_slot: np.ndarray,
            topk_idx: np.ndarray, slot_pos: np.ndarray, E: int,
            R: int) -> np.ndarray:
    """Leg 2: ``send[slot_pos[t,k]] = node_send[node_slot[t, node(e)]]``."""
    node_send = np.ascontiguousarray(node_send)
    node_slot = np.ascontiguousarray(node_slot, dtype=np.int32)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    T, N = node_slot.shape
    K = topk_idx.shape[1]
    send = np.zeros((T * K,) + node_send.shape[1:], dtype=node_send.dtype)
    row_bytes = node_send[0].nbytes if len(node_send) else 0
    _check(_lib().moe_ref_forward(T, E, K, R, N, row_bytes, _ptr(node_send),
                                  len(node_send), _ptr(node_slot),
                                  _ptr(topk_idx), _ptr(slot_pos), _ptr(send)),
           "forward")
    return send


def combine_partial(y: np.ndarray, slot_pos: np.ndarray, topk_w: np.ndarray,
                    topk_idx: np.ndarray, expert_scale: Optional[np.ndarray],
                    node_slot: np.ndarray, E: int, R: int,
                    part_dtype: str = "bf16", accumulate: str = "f64"):
    """Per-node partial sums of each token's weighted expert rows.

    Returns ``(part, exact)``: part [D, H] rounded to ``part_dtype`` and the
    unrounded sums.  ``accumulate="f64"`` sums in fp64 (``exact`` is that
    sum); ``"f32"`` forms the fp32 value a kernel stores before rounding (the
    fused multiply-add chain over the node's slots in ascending k, see
    ``moe_ref_combine_partial_f32``), and ``exact`` is that fp32 value.
    """
    if accumulate == "f32":
        return _combine_partial_f32(y, slot_pos, topk_w, topk_idx,
                                    expert_scale, node_slot, E, R, part_dtype)
    y = np.ascontiguousarray(y)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    node_slot = np.ascontiguousarray(node_slot, dtype=np.int32)
    if expert_scale is not None:
        expert_scale = np.ascontiguousarray(expert_scale, dtype=np.float32)
    T, K = slot_pos.shape
    N = node_slot.shape[1]
    H = y.shape[1]
    D = node_rows(node_slot)
    pcode = DT_F32 if part_dtype == "f32" else DT_BF16
    part = np.zeros((D, H), np.float32 if pcode == DT_F32 else np.uint16)
    exact = np.zeros((D, H), np.float64)
    _check(_lib().moe_ref_combine_partial(
        T, H, E, K, R, N, _dtype_code(y), _ptr(y), _ptr(slot_pos),
        _ptr(topk_w), _ptr(topk_idx), _ptr(expert_scale), _ptr(node_slot), D,
        pcode, _ptr(part), _ptr(exact)), "combine_partial")
    return part, exact


def _combine_partial_f32(y, slot_pos, topk_w, topk_idx, expert_scale,
                         node_slot, E, R, part_dtype):
    y = np.ascontiguousarray(y)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    node_slot = np.ascontiguousarray(node_slot, dtype=np.int32)
    if expert_scale is not None:
        expert_scale = np.ascontiguousarray(expert_scale, dtype=np.float32)
    T, K = slot_pos.shape
    N = node_slot.shape[1]
    H = y.shape[1]
    D = node_rows(node_slot)
    pcode = DT_F32 if part_dtype == "f32" else DT_BF16
    part = np.zeros((D, H), np.float32 if pcode == DT_F32 else np.uint16)
    f32 = np.zeros((D, H), np.float32)
    _check(_lib().moe_ref_combine_partial_f32(
        T, H, E, K, R, N, _dtype_code(y), _ptr(y), _ptr(slot_pos),
        _ptr(topk_w), _ptr(topk_idx), _ptr(expert_scale), _ptr(node_slot), D,
        pcode, _ptr(part), _ptr(f32)), "combine_partial_f32")
    return part, f32.astype(np.float64)


def combine_nodes(part: np.ndarray, node_slot: np.ndarray,
                  out_dtype: str = "bf16"):
    """Sum of each token's node partials: ``(out, exact)`` as in combine."""
    part = np.ascontiguousarray(part)
    node_slot = np.ascontiguousarray(node_slot, dtype=np.int32)
    T, N = node_slot.shape
    H = part.shape[1]
    ocode = DT_F32 if out_dtype == "f32" else DT_BF16
    out = np.empty((T, H), np.float32 if ocode == DT_F32 else np.uint16)
    exact = np.empty((T, H), np.float64)
    _check(_lib().moe_ref_combine_nodes(
        T, H, N, _dtype_code(part), _ptr(part), len(part), _ptr(node_slot),
        ocode, _ptr(out), _ptr(exact)), "combine_nodes")
    return out, exact


def dispatch_combine_nodes(x: np.ndarray, logits: np.ndarray, K: int, R: int,
                           N: int, expert_scale: Optional[np.ndarray] = None,
                           out_dtype: str = "bf16", part_dtype: str = "bf16",
                           renorm: bool = True,
                           accumulate: str = "f64") -> dict:
    """The two-leg path: gate -> layout -> leg 1 -> leg 2 -> per-node
    partials (Y = send; summed as ``accumulate`` says, see
    ``combine_partial``) -> sum of the stored partials at the source."""
    idx, w = gate(logits, K, renorm)
    E = logits.shape[1]
    lay = layout(idx, E, R, N)
    node_send = pack_nodes(x, lay["node_slot"])
    send = forward(node_send, lay["node_slot"], idx, lay["slot_pos"], E, R)
    part, part_exact = combine_partial(send, lay["slot_pos"], w, idx,
                                       expert_scale, lay["node_slot"], E, R,
                                       part_dtype, accumulate)
    out, out_exact = combine_nodes(part, lay["node_slot"], out_dtype)
    res = dict(lay)
    res.update(topk_idx=idx, topk_w=w, node_send=node_send, send=send,
               part=part, part_exact=part_exact, out=out,
               out_exact=out_exact)
    return res


# ---- FP8 dispatch with per-block scales ------------------------------------

def e4m3_value(codes) -> np.ndarray:
    """Exact values of E4M3 codes (uint8) as fp64."""
    f = _lib().moe_ref_e4m3_value
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([f(int(v)) for v in c.ravel()]).reshape(c.shape)


def e4m3_code(values) -> np.ndarray:
    """E4M3 codes of fp64 values (magnitude clamped to 448, ties to even)."""
    f = _lib().moe_ref_e4m3_code
    v = np.asarray(values, dtype=np.float64)
    return np.array([f(float(a)) for a in v.ravel()],
                    dtype=np.uint8).reshape(v.shape)


def fp8_row_bytes(H: int, B: int) -> int:
    return int(_lib().moe_ref_fp8_row_bytes(H, B))


def pack_fp8(x: np.ndarray, slot_pos: np.ndarray, B: int = 128) -> np.ndarray:
    """Quantise each token's row once and write it to its K send rows.

    Returns send as uint8 [T*K, round_up(H + 4*H/B, 128)]: H E4M3 codes, then
    H/B fp32 scales, then zero padding, per row.
    """
    x = np.ascontiguousarray(x)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    T, K = slot_pos.shape
    H = x.shape[1]
    send = np.zeros((T * K, fp8_row_bytes(H, B)), np.uint8)
    _check(_lib().moe_ref_pack_fp8(T, K, H, B, _dtype_code(x), _ptr(x),
                                   _ptr(slot_pos), _ptr(send)), "pack_fp8")
    return send


def fp8_rows_split(send: np.ndarray, H: int, B: int = 128):
    """(codes uint8 [rows, H], scales fp32 [rows, H/B]) of an FP8 buffer."""
    send = np.ascontiguousarray(send)
    return send[:, :H], send[:, H:H + 4 * (H // B)].copy().view(np.float32)


def combine_fp8(y: np.ndarray, slot_pos: np.ndarray, topk_w: np.ndarray,
                H: int, B: int = 128, topk_idx: Optional[np.ndarray] = None,
                expert_scale: Optional[np.ndarray] = None,
                out_dtype: str = "bf16"):
    """Weighted sum of dequantised FP8 rows: ``(out, exact)``."""
    y = np.ascontiguousarray(y, dtype=np.uint8)
    slot_pos = np.ascontiguousarray(slot_pos, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, K = slot_pos.shape
    if expert_scale is not None:
        expert_scale = np.ascontiguousarray(expert_scale, dtype=np.float32)
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    ocode = DT_F32 if out_dtype == "f32" else DT_BF16
    out = np.empty((T, H), np.float32 if ocode == DT_F32 else np.uint16)
    exact = np.empty((T, H), np.float64)
    _check(_lib().moe_ref_combine_fp8(
        T, H, K, B, _ptr(y), _ptr(slot_pos), _ptr(topk_w), _ptr(topk_idx),
        _ptr(expert_scale), ocode, _ptr(out), _ptr(exact)), "combine_fp8")
    return out, exact


def dispatch_combine_fp8(x: np.ndarray, logits: np.ndarray, K: int, R: int,
                         N: int, expert_scale: Optional[np.ndarray] = None,
                         out_dtype: str = "bf16", B: int = 128,
                         renorm: bool = True) -> dict:
    """gate -> layout -> quantising pack -> combine of the FP8 rows."""
    idx, w = gate(logits, K, renorm)
    E = logits.shape[1]
    lay = layout(idx, E, R, N)
    send = pack_fp8(x, lay["slot_pos"], B)
    out, exact = combine_fp8(send, lay["slot_pos"], w, x.shape[1], B, idx,
                             expert_scale, out_dtype)
    res = dict(lay)
    res.update(topk_idx=idx, topk_w=w, send=send, out=out, out_exact=exact)
    return res


# ---- capacity-padded and bucketed layout ----------------------------------

def capacity(T: int, K: int, E: int, gamma: float) -> int:
    """C = ceil(gamma * T * K / E), the reading of the missing formula."""
    return int(np.ceil(gamma * T * K / E))


def layout_capacity(topk_idx: np.ndarray, E: int, levels) -> dict:
    """Capacity-padded / bucketed layout (see moe_ref.c); levels ascending."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    levels = np.ascontiguousarray(levels, dtype=np.int32)
    T, K = topk_idx.shape
    cmax = int(levels[-1])
    o = {
        "expert_count": np.empty(E, np.int32),
        "expert_cap": np.empty(E, np.int32),
        "expert_off": np.empty(E + 1, np.int32),
        "slot_pos": np.empty((T, K), np.int32),
        "row_src": np.empty(E * cmax, np.int32),
    }
    dropped = np.zeros(1, np.int32)
    _check(_lib().moe_ref_layout_capacity(
        T, E, K, _ptr(topk_idx), _ptr(levels), len(levels),
        _ptr(o["expert_count"]), _ptr(o["expert_cap"]),
        _ptr(o["expert_off"]), _ptr(o["slot_pos"]), _ptr(o["row_src"]),
        _ptr(dropped)), "layout_capacity")
    o["dropped"] = int(dropped[0])
    return o


def pack_capacity(x: np.ndarray, row_src: np.ndarray, K: int) -> np.ndarray:
    """Used rows are their token's x row, padding rows are zero."""
    x = np.ascontiguousarray(x)
    row_src = np.ascontiguousarray(row_src, dtype=np.int32)
    T = x.shape[0]
    send = np.empty((len(row_src),) + x.shape[1:], dtype=x.dtype)
    row_bytes = x[0].nbytes if T > 0 else 0
    _check(_lib().moe_ref_pack_capacity(T, K, row_bytes, _ptr(x),
                                        _ptr(row_src), len(row_src),
                                        _ptr(send)), "pack_capacity")
    return send


def dispatch_combine_capacity(x: np.ndarray, logits: np.ndarray, K: int,
                              levels, expert_scale: Optional[np.ndarray] = None,
                              out_dtype: str = "bf16",
                              renorm: bool = True) -> dict:
    """gate -> capacity layout -> padded pack -> combine (dropped slots add
    nothing)."""
    idx, w = gate(logits, K, renorm)
    E = logits.shape[1]
    lay = layout_capacity(idx, E, levels)
    send = pack_capacity(x, lay["row_src"], K)
    out, exact = combine(send, lay["slot_pos"], w, idx, expert_scale,
                         out_dtype)
    res = dict(lay)
    res.update(topk_idx=idx, topk_w=w, send=send, out=out, out_exact=exact)
    return res


# ---- communication-aware task assignment -----------------------------------

def assign(topk_idx: np.ndarray, src_rank: np.ndarray, holds: np.ndarray,
           N: int, u_node: np.ndarray, u_rank: np.ndarray):
    """Cobalt Section 3.3 task assignment (see moe_ref.c).

    Returns ``(assign_rank int32 [T,K], remote_mask uint64 [T])``.
    """
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    src_rank = np.ascontiguousarray(src_rank, dtype=np.int32)
    holds = np.ascontiguousarray(holds, dtype=np.uint8)
    u_node = np.ascontiguousarray(u_node, dtype=np.uint32)
    u_rank = np.ascontiguousarray(u_rank, dtype=np.uint32)
    T, K = topk_idx.shape
    G, E = holds.shape
    ar = np.empty((T, K), np.int32)
    rm = np.empty(T, np.uint64)
    _check(_lib().moe_ref_assign(T, E, K, G, N, _ptr(topk_idx),
                                 _ptr(src_rank), _ptr(holds), _ptr(u_node),
                                 _ptr(u_rank), _ptr(ar), _ptr(rm)), "assign")
    return ar, rm


def f64_to_bf16(values) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); uint16 bits."""
    v = np.asarray(values, dtype=np.float64).ravel()
    f = _lib().moe_ref_f64_to_bf16
    return np.array([f(float(a)) for a in v], dtype=np.uint16)


def dispatch_combine(x: np.ndarray, logits: np.ndarray, K: int, R: int,
                     N: int, expert_scale: Optional[np.ndarray] = None,
                     out_dtype: str = "bf16", renorm: bool = True) -> dict:
    """The whole path: gate -> layout -> pack -> combine with Y = send."""
    idx, w = gate(logits, K, renorm)
    E = logits.shape[1]
    lay = layout(idx, E, R, N)
    send = pack(x, lay["slot_pos"])
    out, exact = combine(send, lay["slot_pos"], w, idx, expert_scale,
                         out_dtype)
    res = dict(lay)
    res.update(topk_idx=idx, topk_w=w, send=send, out=out, out_exact=exact)
    return res
