"""GPU parity of the capacity-padded and bucketed layout, its padded pack and
the combine over the padded buffer (dropped slots add nothing).

Layout outputs and packed rows (including the zero padding) are bit-exact
against the CPU oracle; the combine is held to the combine tolerances
against the oracle's unrounded fp64 sum.
"""
import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle
from helpers import (cfg_of, check_gate, check_out, dev, host, out_dtype,
                     require_gpu, row_dtype, rows_f64, term_scale)

pytestmark = pytest.mark.gpu

SMALL = [
    mi.TINY,
    mi.DEEPSEEK_V3_DECODE,
    mi.MIXTRAL.replace(T=700, H=256),
    mi.QWEN3.replace(T=777, H=512),
    mi.DEEPSEEK_V3.replace(T=1000, H=520),
    mi.KIMI.replace(T=600, H=256),
]
FULL = [mi.QWEN3, mi.DEEPSEEK_V3, mi.KIMI]
CAP_KEYS = ("expert_count", "expert_cap", "expert_off", "slot_pos", "row_src")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _ids(w):
    return f"{w.name}-T{w.T}-H{w.H}"


def _cap_to_host(lay, T, K):
    o = {n: host(getattr(lay, n)) for n in CAP_KEYS}
    o["slot_pos"] = o["slot_pos"].reshape(T, K)
    o["dropped"] = int(host(lay.dropped)[0])
    return o


def _check_cap(res, ref):
    for k in CAP_KEYS:
        np.testing.assert_array_equal(res[k], ref[k], err_msg=k)
    assert res["dropped"] == ref["dropped"]


def _levels_for(w, kind):
    C = oracle.capacity(w.T, w.K, w.E, 1.25)
    if kind == "tight":
        return [oracle.capacity(w.T, w.K, w.E, 0.75)]
    if kind == "capacity":
        return [C]
    mean = w.T * w.K / w.E
    return sorted({max(1, int(mean * f)) for f in (0.5, 1.0, 1.5, 2.0)})


@pytest.mark.parametrize("kind", ["tight", "capacity", "buckets"])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_capacity_layout(w, kind):
    d = mi.make_inputs(w, with_x=False)
    idx, wt = oracle.gate(d["logits"], w.K)
    levels = _levels_for(w, kind)
    ref = oracle.layout_capacity(idx, w.E, levels)
    cfg = cfg_of(w)
    lay = moe.alloc_capacity_layout(cfg, levels)
    ws = moe.alloc_capacity_workspace(cfg)
    moe.moe_dispatch_layout_capacity(cfg, dev(idx), levels, lay, ws)
    _check_cap(_cap_to_host(lay, w.T, w.K), ref)


def run_capacity(w, d, levels, keep_device=False):
    cfg = cfg_of(w)
    T, K = w.T, w.K
    x = dev(d["x"])
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_capacity_layout(cfg, levels)
    send = torch.full((w.E * levels[-1], w.H), 7.0, dtype=row_dtype(w),
                      device="cuda")
    out = torch.empty((T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_capacity_workspace(cfg)
    moe.moe_dispatch_combine_capacity(cfg, x, dev(d["logits"]), scale, idx,
                                      wt, levels, lay, send, out, ws)
    res = _cap_to_host(lay, T, K)
    res.update(topk_idx=host(idx).reshape(T, K),
               topk_w=host(wt).reshape(T, K), out=host(out))
    res.update(send_dev=send, x_dev=x) if keep_device else \
        res.update(send=host(send))
    return res


def _coef(d, idx, wt):
    c = wt.astype(np.float64)
    if d["expert_scale"] is not None:
        c = c * d["expert_scale"][idx].astype(np.float64)
    return c


def _drop_scale(send, slot_pos, coef):
    c = np.where(slot_pos >= 0, coef, 0.0)
    return term_scale(rows_f64(send), np.maximum(slot_pos, 0), c)


@pytest.mark.parametrize("kind", ["tight", "capacity", "buckets"])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_capacity_fused_small(w, kind):
    _check_fused(w, _levels_for(w, kind))


def _check_fused(w, levels):
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine_capacity(d["x"], d["logits"], w.K, levels,
                                           d["expert_scale"], w.out_dtype)
    res = run_capacity(w, d, levels)
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    _check_cap(res, ref)
    np.testing.assert_array_equal(res["send"], ref["send"])
    check_out(res["out"], ref["out_exact"],
              _drop_scale(ref["send"], ref["slot_pos"],
                          _coef(d, ref["topk_idx"], ref["topk_w"])),
              w.out_dtype)


@pytest.mark.parametrize("w", FULL, ids=_ids)
def test_capacity_fused_full_size(w):
    d = mi.make_inputs(w)
    levels = [oracle.capacity(w.T, w.K, w.E, 1.25)]
    res = run_capacity(w, d, levels, keep_device=True)
    idx, wt = oracle.gate(d["logits"], w.K)
    check_gate(res, idx, wt)
    ref = oracle.layout_capacity(idx, w.E, levels)
    _check_cap(res, ref)
    rs = ref["row_src"]
    send, x = res["send_dev"], res["x_dev"]
    used = torch.from_numpy(np.nonzero(rs >= 0)[0]).cuda()
    tok = torch.from_numpy((rs[rs >= 0] // w.K).astype(np.int64)).cuda()
    for lo in range(0, len(used), 1 << 16):
        hi = min(lo + (1 << 16), len(used))
        assert torch.equal(send[used[lo:hi]], x[tok[lo:hi]]), (lo, hi)
    pad = torch.from_numpy(np.nonzero(rs < 0)[0]).cuda()
    if len(pad):
        assert not torch.any(send[pad] != 0)
    # every token, a chunk at a time: a kept slot's padded row is its
    # token's x row (checked above), so the oracle combines those rows
    for lo in range(0, w.T, 2048):
        toks = np.arange(lo, min(w.T, lo + 2048))
        sp = ref["slot_pos"][toks]
        y_small = np.repeat(d["x"][toks], w.K, axis=0)
        spl = np.where(sp >= 0, np.arange(len(toks) * w.K).reshape(sp.shape),
                       -1).astype(np.int32)
        _, exact = oracle.combine(y_small, spl, wt[toks], idx[toks],
                                  d["expert_scale"], "f32")
        bound = (_drop_scale(y_small, spl, _coef(d, idx[toks], wt[toks]))
                 if w.out_dtype == mi.F32 else None)
        check_out(res["out"][toks], exact, bound, w.out_dtype)


@pytest.mark.parametrize("T,H,E,K,R,N,levels", [
    (1, 64, 8, 2, 4, 2, [1]),
    (300, 64, 16, 4, 4, 2, [1]),            # every expert keeps one token
    (257, 72, 24, 3, 6, 3, [2, 5, 40, 41]),
    (128, 64, 8, 8, 8, 1, [128]),           # K = E, nothing dropped
])
def test_capacity_edge_shapes(T, H, E, K, R, N, levels):
    _check_fused(mi.Workload("edge", T, H, E, K, R, N), levels)


def test_capacity_empty_input():
    w = mi.DEEPSEEK_V3.replace(T=0, H=64)
    cfg = cfg_of(w)
    levels = [3]
    lay = moe.alloc_capacity_layout(cfg, levels)
    ws = moe.alloc_capacity_workspace(cfg)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    xb = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    send = torch.full((w.E * 3, 64), 1.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_combine_capacity(cfg, xb, f, None, e, f, levels, lay,
                                      send, xb, ws)
    assert torch.all(lay.expert_count == 0)
    assert torch.all(lay.expert_cap == 3)
    assert int(lay.dropped[0]) == 0
    assert torch.all(lay.row_src == -1) and not torch.any(send != 0)
