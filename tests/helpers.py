"""Test plumbing: host<->device copies, running the HIP path through the C ABI,
and the parity checks against the oracle.  torch is used only to hold device
memory and to compare buffers; every result under test comes from the HIP
library, every expected value from ``oracle``.
"""
from __future__ import annotations

import numpy as np
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle

# Combine tolerances (stated for the combine in the target of this work):
# fp32 outputs within 1e-5 relative to sum_k |w_k s_k y_k|, bf16 outputs
# within 2e-2 absolute of the unrounded fp64 value.
RTOL_F32 = 1e-5
ATOL_BF16 = 2e-2
# Gate weights: fp64 arithmetic rounded once to fp32 on both sides.
RTOL_W = 1e-6


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    moe.lib()  # fail loudly if the HIP library is missing


def dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    """numpy -> device tensor.  uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint64:
        t = torch.from_numpy(a.view(np.int64))
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cfg_of(w: mi.Workload, layout_tile: int = 0):
    return moe.make_cfg(w.T, w.H, w.E, w.K, w.R, w.N, w.x_dtype, w.out_dtype,
                        w.renorm, layout_tile)


def row_dtype(w: mi.Workload):
    return torch.float32 if w.x_dtype == mi.F32 else torch.bfloat16


def out_dtype(w: mi.Workload):
    return torch.float32 if w.out_dtype == mi.F32 else torch.bfloat16


def layout_to_host(lay: moe.Layout, T: int, K: int, N: int) -> dict:
    o = {}
    for name in moe.LAYOUT_FIELDS:
        t = getattr(lay, name)
        if t is None:
            continue
        a = host(t)
        if name == "node_mask":
            a = a.view(np.uint64)
        elif name == "node_slot":
            a = a.reshape(T, N)
        elif name == "slot_pos":
            a = a.reshape(T, K)
        o[name] = a
    return o


def run_fused(w: mi.Workload, d: dict, layout_tile: int = 0,
              keep_device: bool = False) -> dict:
    """moe_dispatch_combine through the C ABI; returns host arrays."""
    cfg = cfg_of(w, layout_tile)
    T, K = w.T, w.K
    x = dev(d["x"])
    logits = dev(d["logits"])
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    send = torch.empty((T * K, w.H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine(cfg, x, logits, scale, idx, wt, lay, send, out, ws)
    err = moe.moe_read_device_error(ws)
    res = layout_to_host(lay, T, K, w.N)
    res.update(topk_idx=host(idx).reshape(T, K), topk_w=host(wt).reshape(T, K),
               out=host(out), dev_error=err)
    if keep_device:
        res.update(send_dev=send, x_dev=x)
    else:
        res["send"] = host(send)
    return res


def check_gate(res: dict, ref_idx: np.ndarray, ref_w: np.ndarray) -> None:
    np.testing.assert_array_equal(res["topk_idx"], ref_idx)
    np.testing.assert_allclose(res["topk_w"], ref_w, rtol=RTOL_W, atol=0)


LAYOUT_KEYS = ("expert_count", "expert_off", "rank_count", "rank_off",
               "rank_token_count", "node_mask", "node_count", "node_off",
               "node_slot", "slot_pos", "row_src")


def check_layout(res: dict, ref: dict) -> None:
    for k in LAYOUT_KEYS:
        if k in res and k in ref:
            np.testing.assert_array_equal(res[k], ref[k], err_msg=k)


def check_out(out: np.ndarray, exact: np.ndarray, scale_abs: np.ndarray,
              odt: str) -> None:
    """Combine tolerance: fp32 relative to sum|terms|, bf16 absolute."""
    if odt == mi.F32:
        err = np.abs(out.astype(np.float64) - exact)
        bound = RTOL_F32 * scale_abs + 1e-30
        bad = err > bound
        assert not bad.any(), (
            f"{bad.sum()} fp32 outputs off; worst {np.max(err - bound)}")
    else:
        got = mi.bf16_bits_to_f32(out).astype(np.float64)
        err = np.abs(got - exact)
        assert err.max() <= ATOL_BF16, f"bf16 max abs error {err.max()}"


def term_scale(y_f64: np.ndarray, slot_pos: np.ndarray, coef: np.ndarray,
               rows: np.ndarray = None) -> np.ndarray:
    """sum_k |c_k| * |y[slot_k]| per output element (fp32 error scale)."""
    T, K = slot_pos.shape
    sel = np.arange(T) if rows is None else rows
    acc = np.zeros((len(sel), y_f64.shape[1]))
    for k in range(K):
        acc += np.abs(coef[sel, k])[:, None] * np.abs(y_f64[slot_pos[sel, k]])
    return acc


def rows_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return mi.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def abs_rows(a: np.ndarray) -> np.ndarray:
    """|a| for fp32 rows or bf16 bit patterns (sign bit cleared)."""
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def check_all_tokens(out: np.ndarray, T: int, exact_of, abs_of, odt: str,
                     chunk: int = 2048) -> None:
    """Every output token against the oracle, a chunk of tokens at a time.

    exact_of(toks) gives the oracle's unrounded fp64 rows of those tokens;
    abs_of(toks) the same sum over |terms| (the fp32 error scale; only
    called for fp32 outputs)."""
    for lo in range(0, T, chunk):
        toks = np.arange(lo, min(T, lo + chunk), dtype=np.int32)
        sc = abs_of(toks) if odt == mi.F32 else None
        check_out(out[lo:lo + len(toks)], exact_of(toks), sc, odt)


def check_combine_all(out: np.ndarray, y: np.ndarray, slot_pos: np.ndarray,
                      topk_w: np.ndarray, topk_idx, scale, odt: str,
                      chunk: int = 2048) -> None:
    """Every token of a combine over rows y against oracle.combine_tokens
    (slots < 0 add nothing; weights and scales are non-negative)."""
    ay = abs_rows(y) if odt == mi.F32 else None
    check_all_tokens(
        out, slot_pos.shape[0],
        lambda toks: oracle.combine_tokens(toks, y, slot_pos, topk_w,
                                           topk_idx, scale),
        lambda toks: oracle.combine_tokens(toks, ay, slot_pos,
                                           np.abs(topk_w), topk_idx,
                                           None if scale is None
                                           else np.abs(scale)),
        odt, chunk)
