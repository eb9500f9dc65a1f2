"""GPU parity of the node-level two-leg dispatch and hierarchical combine.

Leg-1 rows, leg-2 rows, counts and slots are bit-exact against the CPU
oracle.  The stored partials (fp32 or bf16) are bit-exact against the
oracle's fp32 partial: the fp32 fused multiply-add chain over the node's
slots in ascending k, rounded once to the partial type, so the rounding of a
16-bit partial is decided in the same precision on both sides.  The output
is held to the combine tolerances against the oracle's unrounded fp64 sum of
those stored partials: within 2e-2 absolute (bf16 outputs) or 1e-5 *
sum_n |p_n| (fp32 outputs).  Against the one-leg exact sum, an output from
bf16 partials also stays within the derived rounding bound
2^-8 * (sum_n |p_n| + |exact|) + 2e-5 * sum|terms| (each bf16 partial loses
at most half an ulp, 2^-8 of its value, and sum_n |p_n| <= sum|terms|).
"""
import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle
from helpers import (ATOL_BF16, cfg_of, check_gate, check_layout, dev, host,
                     layout_to_host, out_dtype, require_gpu, row_dtype,
                     rows_f64)

pytestmark = pytest.mark.gpu

SMALL = [
    mi.TINY,
    mi.DEEPSEEK_V3_DECODE,
    mi.MIXTRAL.replace(T=700, H=256),
    mi.QWEN3.replace(T=777, H=512),
    mi.DEEPSEEK_V3.replace(T=1000, H=520),
    mi.KIMI.replace(T=600, H=256),
]
FULL = [mi.MIXTRAL, mi.QWEN3, mi.DEEPSEEK_V3, mi.KIMI]
TORCH_PART = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _ids(w):
    return f"{w.name}-T{w.T}-H{w.H}"


def _route(w, d):
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    return idx, wt, lay


def _coef(w, d, idx, wt):
    c = wt.astype(np.float64)
    if d["expert_scale"] is not None:
        c = c * d["expert_scale"][idx].astype(np.float64)
    return c


def _abs_rows(a):
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def _part_scale(w, d, send, idx, wt, lay):
    """sum over a partial's slots of |w s y|, exactly (fp64 oracle on |y|)."""
    _, sc = oracle.combine_partial(_abs_rows(send), lay["slot_pos"], wt, idx,
                                   d["expert_scale"], lay["node_slot"], w.E,
                                   w.R, "f32")
    return sc


def _check_part(got, exact, scale, pdt):
    g = rows_f64(got)
    err = np.abs(g - exact)
    if pdt == "f32":
        bound = 1e-5 * scale + 1e-30
    else:
        bound = 2.0 ** -8 * np.abs(exact) + 2e-5 * scale + 1e-30
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} partial values off; worst excess " \
                          f"{np.max(err - bound)}"


def _check_out(got, exact, scale, pdt, odt):
    g = rows_f64(got)
    err = np.abs(g - exact)
    if pdt == "f32":
        if odt == mi.F32:
            bound = 1e-5 * scale + 1e-30
        else:
            assert err.max() <= ATOL_BF16, f"bf16 max abs error {err.max()}"
            return
    else:
        bound = 2.0 ** -8 * (scale + np.abs(exact)) + 2e-5 * scale + 1e-30
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs off; worst excess " \
                          f"{np.max(err - bound)}"


def _flat_scale(send, slot_pos, coef, toks=None):
    y = rows_f64(send)
    T, K = slot_pos.shape
    sel = np.arange(T) if toks is None else toks
    acc = np.zeros((len(sel), y.shape[1]))
    for k in range(K):
        acc += np.abs(coef[sel, k])[:, None] * np.abs(y[slot_pos[sel, k]])
    return acc


# ------------------------------------------------------ single calls ----

@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_pack_nodes(w):
    d = mi.make_inputs(w)
    idx, wt, lay = _route(w, d)
    cfg = cfg_of(w)
    cap = moe.moe_node_rows_max(cfg)
    ns = torch.zeros((cap, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_pack_nodes(cfg, dev(d["x"]), dev(lay["node_slot"]), ns)
    ref = oracle.pack_nodes(d["x"], lay["node_slot"])
    got = host(ns)
    np.testing.assert_array_equal(got[:len(ref)], ref)
    assert not got[len(ref):].any()  # rows past the crossings untouched


def test_pack_nodes_large_ragged():
    # 200000 node rows of 6000 bytes: the pack's piece-per-wave kernel, with
    # a ragged last piece per row, an odd node count and skipped (-1) entries
    w = mi.Workload("large_ragged", T=40000, H=3000, E=60, K=5, R=15, N=5,
                    x_dtype=mi.BF16, out_dtype=mi.BF16)
    cfg = cfg_of(w)
    cap = moe.moe_node_rows_max(cfg)
    assert cap * w.H * 2 >= 1 << 30
    x = mi.random_x(w.T, w.H, w.x_dtype, seed=4)
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=4)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    assert (lay["node_slot"] < 0).any()
    ns = torch.zeros((cap, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_pack_nodes(cfg, dev(x), dev(lay["node_slot"]), ns)
    ref = oracle.pack_nodes(x, lay["node_slot"])
    got = host(ns)
    np.testing.assert_array_equal(got[:len(ref)], ref)
    assert not got[len(ref):].any()


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_forward(w):
    d = mi.make_inputs(w)
    idx, wt, lay = _route(w, d)
    cfg = cfg_of(w)
    cap = moe.moe_node_rows_max(cfg)
    ref_ns = oracle.pack_nodes(d["x"], lay["node_slot"])
    ns = torch.zeros((cap, w.H), dtype=row_dtype(w), device="cuda")
    ns[:len(ref_ns)] = dev(ref_ns)
    send = torch.zeros((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_forward(cfg, ns, dev(lay["node_slot"]), dev(idx),
                             dev(lay["slot_pos"]), send)
    np.testing.assert_array_equal(host(send),
                                  oracle.pack(d["x"], lay["slot_pos"]))


def test_forward_large_ragged():
    # 1.2 GB of send rows with a row of 375 16-byte vectors (not a multiple
    # of the wave's 64-vector stride), an odd K and 5 nodes
    w = mi.Workload("large_ragged", T=40000, H=3000, E=60, K=5, R=15, N=5,
                    x_dtype=mi.BF16, out_dtype=mi.BF16)
    assert w.T * w.K * w.H * 2 >= 1 << 30
    cfg = cfg_of(w)
    x = mi.random_x(w.T, w.H, w.x_dtype, seed=8)
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=8)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    ref_ns = oracle.pack_nodes(x, lay["node_slot"])
    ns = torch.zeros((moe.moe_node_rows_max(cfg), w.H), dtype=row_dtype(w),
                     device="cuda")
    ns[:len(ref_ns)] = dev(ref_ns)
    del ref_ns
    send = torch.zeros((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_forward(cfg, ns, dev(lay["node_slot"]), dev(idx),
                             dev(lay["slot_pos"]), send)
    np.testing.assert_array_equal(host(send), oracle.pack(x, lay["slot_pos"]))


@pytest.mark.parametrize("pdt", ["bf16", "f32"])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_partial(w, pdt):
    d = mi.make_inputs(w)
    idx, wt, lay = _route(w, d)
    cfg = cfg_of(w)
    cap = moe.moe_node_rows_max(cfg)
    send = oracle.pack(d["x"], lay["slot_pos"])
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    part = torch.zeros((cap, w.H), dtype=TORCH_PART[pdt], device="cuda")
    moe.moe_combine_partial(cfg, dev(send), dev(lay["slot_pos"]), dev(wt),
                            dev(idx), scale, dev(lay["node_slot"]), part)
    ref, _ = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                    d["expert_scale"], lay["node_slot"], w.E,
                                    w.R, pdt, accumulate="f32")
    _, pex = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                    d["expert_scale"], lay["node_slot"], w.E,
                                    w.R, pdt)
    got = host(part)
    np.testing.assert_array_equal(got[:len(ref)], ref)
    # and within the rounding bound of the fp64 partial
    _check_part(got[:len(pex)], pex,
                _part_scale(w, d, send, idx, wt, lay), pdt)
    assert not got[len(pex):].any()


@pytest.mark.parametrize("pdt", ["bf16", "f32"])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_sum_nodes(w, pdt):
    d = mi.make_inputs(w)
    idx, wt, lay = _route(w, d)
    cfg = cfg_of(w)
    cap = moe.moe_node_rows_max(cfg)
    send = oracle.pack(d["x"], lay["slot_pos"])
    rpart, _ = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                      d["expert_scale"], lay["node_slot"],
                                      w.E, w.R, pdt)
    part = torch.zeros((cap, w.H), dtype=TORCH_PART[pdt], device="cuda")
    part[:len(rpart)] = dev(rpart, bf16=(pdt == "bf16"))
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    moe.moe_combine_nodes(cfg, part, dev(lay["node_slot"]), out)
    _, ex = oracle.combine_nodes(rpart, lay["node_slot"], "f32")
    _, sc = oracle.combine_nodes(_abs_rows(rpart), lay["node_slot"], "f32")
    g = rows_f64(host(out))
    err = np.abs(g - ex)
    if w.out_dtype == mi.F32:
        bound = w.N * 2.0 ** -23 * sc + 1e-30
    else:
        bound = 2.0 ** -8 * np.abs(ex) + w.N * 2.0 ** -23 * sc + 1e-30
    assert not (err > bound).any(), np.max(err - bound)


# ------------------------------------------------------ fused path ----

def run_two_leg(w, d, pdt, keep_device=False):
    cfg = cfg_of(w)
    T, K = w.T, w.K
    cap = moe.moe_node_rows_max(cfg)
    x = dev(d["x"])
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    ns = torch.empty((cap, w.H), dtype=row_dtype(w), device="cuda")
    send = torch.empty((T * K, w.H), dtype=row_dtype(w), device="cuda")
    part = torch.empty((cap, w.H), dtype=TORCH_PART[pdt], device="cuda")
    out = torch.empty((T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine_nodes(cfg, x, dev(d["logits"]), scale, idx, wt,
                                   lay, ns, send, part, out, ws)
    err = moe.moe_read_device_error(ws)
    res = layout_to_host(lay, T, K, w.N)
    res.update(topk_idx=host(idx).reshape(T, K),
               topk_w=host(wt).reshape(T, K), out=host(out), dev_error=err)
    if keep_device:
        res.update(x_dev=x, ns_dev=ns, send_dev=send, part_dev=part)
    else:
        D = int(res["node_off"][-1])
        res.update(node_send=host(ns[:D]), send=host(send),
                   part=host(part[:D]))
    return res


@pytest.mark.parametrize("pdt", ["bf16", "f32"])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_two_leg_fused_small(w, pdt):
    _check_two_leg(w, pdt)


def _check_node_sum(got, part, node_slot, odt):
    """The output against the oracle's fp64 sum of the stored partials:
    the combine tolerances (2e-2 absolute for bf16, 1e-5 * sum_n |p_n|)."""
    _, ex = oracle.combine_nodes(part, node_slot, "f32")
    err = np.abs(rows_f64(got) - ex)
    if odt == mi.BF16:
        assert err.max() <= ATOL_BF16, f"bf16 max abs error {err.max()}"
    else:
        _, sc = oracle.combine_nodes(_abs_rows(part), node_slot, "f32")
        bad = err > 1e-5 * sc + 1e-30
        assert not bad.any(), f"{bad.sum()} fp32 outputs off"


def _check_two_leg(w, pdt):
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine_nodes(d["x"], d["logits"], w.K, w.R, w.N,
                                        d["expert_scale"], w.out_dtype, pdt,
                                        accumulate="f32")
    res = run_two_leg(w, d, pdt)
    assert res["dev_error"] == 0
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(res["node_send"], ref["node_send"])
    np.testing.assert_array_equal(res["send"], ref["send"])
    idx, wt = ref["topk_idx"], ref["topk_w"]
    np.testing.assert_array_equal(res["part"], ref["part"])
    _check_node_sum(res["out"], ref["part"], ref["node_slot"], w.out_dtype)
    # the output against the flat (one-leg) exact sum
    _, flat = oracle.combine(ref["send"], ref["slot_pos"], wt, idx,
                             d["expert_scale"], "f32")
    _check_out(res["out"], flat,
               _flat_scale(ref["send"], ref["slot_pos"], _coef(w, d, idx, wt)),
               pdt, w.out_dtype)


@pytest.mark.parametrize("w,pdt", [(w, "bf16") for w in FULL] +
                         [(mi.QWEN3, "f32"), (mi.DEEPSEEK_V3, "f32")],
                         ids=lambda v: _ids(v) if isinstance(v, mi.Workload)
                         else v)
def test_two_leg_fused_full_size(w, pdt):
    d = mi.make_inputs(w)
    res = run_two_leg(w, d, pdt, keep_device=True)
    assert res["dev_error"] == 0
    idx, wt = oracle.gate(d["logits"], w.K)
    check_gate(res, idx, wt)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    check_layout(res, lay)
    x = res["x_dev"]
    # every leg-1 row is the x row of its (token, node) crossing
    ns_tok = np.repeat(np.arange(w.T), w.N)[lay["node_slot"].ravel() >= 0]
    ns_row = lay["node_slot"].ravel()[lay["node_slot"].ravel() >= 0]
    order = np.argsort(ns_row)
    np.testing.assert_array_equal(ns_row[order], np.arange(len(ns_row)))
    ns_tok = torch.from_numpy(ns_tok[order].astype(np.int64)).cuda()
    for lo in range(0, len(ns_row), 1 << 16):
        hi = min(lo + (1 << 16), len(ns_row))
        assert torch.equal(res["ns_dev"][lo:hi], x[ns_tok[lo:hi]]), (lo, hi)
    # every send row is the x row the oracle's permutation names
    src_tok = torch.from_numpy((lay["row_src"] // w.K).astype(np.int64)).cuda()
    for lo in range(0, w.T * w.K, 1 << 16):
        hi = min(lo + (1 << 16), w.T * w.K)
        assert torch.equal(res["send_dev"][lo:hi], x[src_tok[lo:hi]]), (lo, hi)
    # every token, a chunk at a time.  A slot's send row is its token's x
    # row (checked above), so the oracle takes K copies of x[t] as token t's
    # expert rows; the chunk's crossings are renumbered in their (token,
    # node) order, which is the order of their global partial rows.
    part_dev = res["part_dev"]
    for lo in range(0, w.T, 2048):
        toks = np.arange(lo, min(w.T, lo + 2048))
        nt = len(toks)
        y_small = np.repeat(d["x"][toks], w.K, axis=0)
        sp = np.arange(nt * w.K, dtype=np.int32).reshape(nt, w.K)
        ns = lay["node_slot"][toks]
        valid = ns >= 0
        ns_local = np.full_like(ns, -1)
        ns_local[valid] = np.arange(int(valid.sum()), dtype=np.int32)
        ref_part, _ = oracle.combine_partial(
            y_small, sp, wt[toks], idx[toks], d["expert_scale"], ns_local,
            w.E, w.R, pdt, accumulate="f32")
        rows = torch.from_numpy(ns[valid].astype(np.int64)).cuda()
        np.testing.assert_array_equal(host(part_dev[rows]), ref_part,
                                      err_msg=f"partials of tokens {lo}+")
        got = res["out"][toks]
        _check_node_sum(got, ref_part, ns_local, w.out_dtype)
        _, flat = oracle.combine(y_small, sp, wt[toks], idx[toks],
                                 d["expert_scale"], "f32")
        _check_out(got, flat,
                   _flat_scale(y_small, sp, _coef(w, d, idx[toks], wt[toks])),
                   pdt, w.out_dtype)


# ------------------------------------------------------- edge cases ----

@pytest.mark.parametrize("T,H,E,K,R,N,xdt,odt", [
    (1, 64, 8, 2, 4, 2, mi.BF16, mi.BF16),
    (97, 72, 24, 3, 6, 3, mi.F32, mi.BF16),       # odd K (padded slots)
    (100, 64, 256, 32, 64, 64, mi.BF16, mi.F32),  # K = 32, N = 64
    (130, 8, 16, 16, 16, 16, mi.BF16, mi.BF16),   # K = E, one expert a node
    (65, 1032, 64, 5, 8, 8, mi.F32, mi.F32),      # wide ragged row
])
@pytest.mark.parametrize("pdt", ["bf16", "f32"])
def test_two_leg_edge_shapes(T, H, E, K, R, N, xdt, odt, pdt):
    _check_two_leg(mi.Workload("edge", T, H, E, K, R, N, x_dtype=xdt,
                               out_dtype=odt), pdt)


def test_two_leg_single_node_matches_flat_combine():
    # N = 1: one partial per token, the flat combine's value
    w = mi.MIXTRAL.replace(T=300, H=128)
    d = mi.make_inputs(w)
    res = run_two_leg(w, d, "f32")
    np.testing.assert_array_equal(res["node_slot"][:, 0], np.arange(w.T))
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    send = torch.empty((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device="cuda")
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine(cfg, dev(d["x"]), dev(d["logits"]),
                             dev(d["expert_scale"]), idx, wt, lay, send, out,
                             ws)
    # same fp32 sums in the same k order, then one rounding: equal bits
    np.testing.assert_array_equal(res["out"], host(out))


def test_two_leg_empty_input():
    w = mi.DEEPSEEK_V3.replace(T=0, H=64)
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    ws = moe.alloc_workspace(cfg)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    xb = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_combine_nodes(cfg, xb, f, None, e, f, lay, xb, xb, xb,
                                   xb, ws)
    assert moe.moe_read_device_error(ws) == 0
    assert torch.all(lay.node_off == 0)
