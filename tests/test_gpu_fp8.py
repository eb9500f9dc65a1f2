"""GPU parity of the FP8 (E4M3, per-block scale) dispatch and combine.

Codes, scales and padding of the packed rows are bit-exact against the CPU
oracle (the codes are integer decisions taken in fp32 on both sides).  The
combine of FP8 rows is held to the combine tolerances (fp32 outputs within
1e-5 of sum|terms|, bf16 outputs within 2e-2 absolute of the oracle's
unrounded fp64 sum of the dequantised rows).
"""
import functools

import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle
from helpers import (ATOL_BF16, RTOL_F32, cfg_of, check_gate, check_layout,
                     dev, host, layout_to_host, out_dtype, require_gpu,
                     rows_f64)

pytestmark = pytest.mark.gpu

SMALL = [
    mi.TINY,
    mi.DEEPSEEK_V3_DECODE,
    mi.MIXTRAL.replace(T=700, H=512),
    mi.QWEN3.replace(T=777, H=512),
    mi.DEEPSEEK_V3.replace(T=1000, H=640),
    mi.KIMI.replace(T=600, H=256),
]
FULL = [mi.MIXTRAL, mi.QWEN3, mi.DEEPSEEK_V3, mi.KIMI]
TABLE = oracle.e4m3_value(np.arange(256, dtype=np.uint8))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _ids(w):
    return f"{w.name}-T{w.T}-H{w.H}"


def _block(w):
    return 128 if w.H % 128 == 0 else 32


def _check_out(got, exact, scale_abs, odt):
    if odt == mi.F32:
        err = np.abs(got.astype(np.float64) - exact)
        bad = err > RTOL_F32 * scale_abs + 1e-30
        assert not bad.any(), f"{bad.sum()} fp32 outputs off"
    else:
        err = np.abs(rows_f64(got) - exact)
        assert err.max() <= ATOL_BF16, f"bf16 max abs error {err.max()}"


def _deq_rows(send, H, B):
    codes, scales = oracle.fp8_rows_split(send, H, B)
    return TABLE[codes] * np.repeat(scales.astype(np.float64), B, axis=1)


def _term_scale(deq, slot_pos, coef):
    acc = np.zeros((slot_pos.shape[0], deq.shape[1]))
    for k in range(slot_pos.shape[1]):
        acc += np.abs(coef[:, k])[:, None] * np.abs(deq[slot_pos[:, k]])
    return acc


def _coef(d, idx, wt):
    c = wt.astype(np.float64)
    if d["expert_scale"] is not None:
        c = c * d["expert_scale"][idx].astype(np.float64)
    return c


# ------------------------------------------------ the hardware codec ----

def test_e4m3_conversion_sweep():
    """Blocks whose largest magnitude is 448 have 448/amax = 1 exactly, so
    their codes are the device's E4M3 conversion of the values themselves."""
    rng = np.random.Generator(np.random.PCG64(3))
    pos = TABLE[:0x7F]
    vals = np.concatenate([
        2.0 ** rng.uniform(-14, np.log2(448), 20000) * rng.choice([-1, 1], 20000),
        (pos[1:] + pos[:-1]) / 2, -(pos[1:] + pos[:-1]) / 2,   # exact ties
        pos, -pos, [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 1e-38, -1e-38,
                    447.9, -447.99, 440.0, 2.0 ** -126, 2.0 ** -149]])
    vals = vals.astype(np.float32)
    B = 32
    per = B - 1
    nblk = -(-len(vals) // per)
    x = np.zeros((nblk, B), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(nblk * per, np.float32)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(nblk, per)
    H = 512
    T = -(-nblk * B // H)
    xr = np.zeros((T * H // B, B), np.float32)
    xr[:nblk] = x
    xr[nblk:, 0] = 448.0
    xr = xr.reshape(T, H)
    cfg = moe.make_cfg(T, H, 1, 1, 1, 1, "f32", "f32")
    slot = torch.arange(T, dtype=torch.int32, device="cuda")
    rb = moe.moe_fp8_row_bytes(H, B)
    send = torch.zeros((T, rb), dtype=torch.uint8, device="cuda")
    moe.moe_dispatch_pack_fp8(cfg, dev(xr), slot, send, B)
    ref = oracle.pack_fp8(xr, np.arange(T, dtype=np.int32).reshape(T, 1), B)
    got = host(send)
    np.testing.assert_array_equal(got, ref)
    # and the device's widening of every code: one-hot combine, fp32 out
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    w1 = torch.ones(T, dtype=torch.float32, device="cuda")
    moe.moe_combine_fp8(cfg, send, slot, w1, None, None, out, B)
    np.testing.assert_array_equal(host(out).astype(np.float64),
                                  _deq_rows(ref, H, B))


# ------------------------------------------------------ single calls ----

@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_pack_fp8(w):
    d = mi.make_inputs(w)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    B = _block(w)
    cfg = cfg_of(w)
    rb = moe.moe_fp8_row_bytes(w.H, B)
    assert rb == oracle.fp8_row_bytes(w.H, B)
    send = torch.full((w.T * w.K, rb), 0xAB, dtype=torch.uint8, device="cuda")
    moe.moe_dispatch_pack_fp8(cfg, dev(d["x"]), dev(lay["slot_pos"]), send, B)
    np.testing.assert_array_equal(host(send),
                                  oracle.pack_fp8(d["x"], lay["slot_pos"], B))


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_combine_fp8(w):
    d = mi.make_inputs(w)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    B = _block(w)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], B)
    cfg = cfg_of(w)
    out = torch.empty((w.T, w.H), dtype=torch.float32 if w.out_dtype == mi.F32
                      else torch.bfloat16, device="cuda")
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    moe.moe_combine_fp8(cfg, dev(send), dev(lay["slot_pos"]), dev(wt),
                        dev(idx), scale, out, B)
    _, exact = oracle.combine_fp8(send, lay["slot_pos"], wt, w.H, B, idx,
                                  d["expert_scale"], "f32")
    _check_out(host(out), exact,
               _term_scale(_deq_rows(send, w.H, B), lay["slot_pos"],
                           _coef(d, idx, wt)), w.out_dtype)


# From 512 MiB of FP8 rows the combine switches to its burst kernel (groups
# of up to 8 tokens staged in LDS, as many as fit): 20002 tokens leave a
# ragged last group both for bf16 outputs (7 tokens a group at H = 4096,
# K = 8) and for fp32 ones (3 a group).  At H = 16384 one bf16 token fills a
# group of its own and an fp32 token no longer fits the stage, so that
# combine takes the one-token-a-workgroup kernel.
@functools.lru_cache(maxsize=2)
def _burst_case(H=4096, T=20002):
    w = mi.Workload("fp8_burst_ragged", T=T, H=H, E=64, K=8, R=16,
                    N=4, x_dtype=mi.BF16)
    B = 128
    d = mi.make_inputs(w)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], B)
    _, exact = oracle.combine_fp8(send, lay["slot_pos"], wt, w.H, B, idx,
                                  d["expert_scale"], "f32")
    return w, B, d, idx, wt, lay, send, exact


@pytest.mark.parametrize("H,T", [(4096, 20002), (16384, 4001)])
@pytest.mark.parametrize("odt", [mi.BF16, mi.F32])
def test_combine_fp8_burst_ragged(odt, H, T):
    w, B, d, idx, wt, lay, send, exact = _burst_case(H, T)
    w = w.replace(out_dtype=odt)
    assert w.T * w.K * moe.moe_fp8_row_bytes(w.H, B) >= 512 << 20
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    moe.moe_combine_fp8(cfg_of(w), dev(send), dev(lay["slot_pos"]), dev(wt),
                        dev(idx), dev(d["expert_scale"]), out, B)
    got = host(out)
    # every token; fp32 outputs against sum |terms| of the dequantised rows
    for lo in range(0, w.T, 2048):
        toks = np.arange(lo, min(w.T, lo + 2048))
        bound = None
        if odt == mi.F32:
            sp = lay["slot_pos"][toks]
            deq = _deq_rows(send[sp.ravel()], w.H, B).reshape(len(toks), w.K,
                                                             w.H)
            coef = _coef(d, idx, wt)[toks]
            bound = np.einsum("tk,tkh->th", np.abs(coef), np.abs(deq))
        _check_out(got[toks], exact[toks], bound, odt)


# ------------------------------------------------------ fused path ----

def run_fp8(w, d, B, keep_device=False):
    cfg = cfg_of(w)
    T, K = w.T, w.K
    rb = moe.moe_fp8_row_bytes(w.H, B)
    x = dev(d["x"])
    scale = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    send = torch.empty((T * K, rb), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine_fp8(cfg, x, dev(d["logits"]), scale, idx, wt,
                                 lay, send, out, ws, B)
    err = moe.moe_read_device_error(ws)
    res = layout_to_host(lay, T, K, w.N)
    res.update(topk_idx=host(idx).reshape(T, K),
               topk_w=host(wt).reshape(T, K), out=host(out), dev_error=err)
    res.update(send_dev=send) if keep_device else res.update(send=host(send))
    return res


@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_fp8_fused_small(w):
    _check_fused(w)


def _check_fused(w):
    d = mi.make_inputs(w)
    B = _block(w)
    ref = oracle.dispatch_combine_fp8(d["x"], d["logits"], w.K, w.R, w.N,
                                      d["expert_scale"], w.out_dtype, B)
    res = run_fp8(w, d, B)
    assert res["dev_error"] == 0
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(res["send"], ref["send"])
    _check_out(res["out"], ref["out_exact"],
               _term_scale(_deq_rows(ref["send"], w.H, B), ref["slot_pos"],
                           _coef(d, ref["topk_idx"], ref["topk_w"])),
               w.out_dtype)


@pytest.mark.parametrize("w", FULL, ids=_ids)
def test_fp8_fused_full_size(w):
    d = mi.make_inputs(w)
    B = 128
    res = run_fp8(w, d, B, keep_device=True)
    assert res["dev_error"] == 0
    idx, wt = oracle.gate(d["logits"], w.K)
    check_gate(res, idx, wt)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    check_layout(res, lay)
    # every packed row against the oracle's, in chunks on the device
    ref = oracle.pack_fp8(d["x"], lay["slot_pos"], B)
    send = res["send_dev"]
    for lo in range(0, len(ref), 1 << 15):
        hi = min(lo + (1 << 15), len(ref))
        assert torch.equal(send[lo:hi], dev(ref[lo:hi])), (lo, hi)
    # every token, a chunk at a time: the oracle's combine of the oracle's
    # FP8 rows that the token's slots name
    for lo in range(0, w.T, 2048):
        toks = np.arange(lo, min(w.T, lo + 2048))
        sp = lay["slot_pos"][toks]
        y_small = ref[sp.ravel()]
        spl = np.arange(len(toks) * w.K, dtype=np.int32).reshape(len(toks),
                                                                  w.K)
        _, exact = oracle.combine_fp8(y_small, spl, wt[toks], w.H, B,
                                      idx[toks], d["expert_scale"], "f32")
        bound = (_term_scale(_deq_rows(y_small, w.H, B), spl,
                             _coef(d, idx[toks], wt[toks]))
                 if w.out_dtype == mi.F32 else None)
        _check_out(res["out"][toks], exact, bound, w.out_dtype)


# ------------------------------------------------------- edge cases ----

@pytest.mark.parametrize("T,H,E,K,R,N,xdt,odt", [
    (1, 128, 8, 2, 4, 2, mi.BF16, mi.BF16),
    (97, 96, 24, 3, 6, 3, mi.F32, mi.F32),        # generic K, B = 32
    (130, 256, 16, 16, 16, 16, mi.BF16, mi.F32),  # padded stride (264 -> 384)
    (65, 1056, 64, 5, 8, 8, mi.BF16, mi.BF16),    # ragged rows, B = 32
])
def test_fp8_edge_shapes(T, H, E, K, R, N, xdt, odt):
    _check_fused(mi.Workload("edge", T, H, E, K, R, N, x_dtype=xdt,
                             out_dtype=odt))


def test_fp8_rejects_bad_block():
    w = mi.DEEPSEEK_V3.replace(T=4, H=96)
    cfg = cfg_of(w)
    assert moe.moe_fp8_row_bytes(96, 128) == 0
    assert moe.moe_fp8_row_bytes(96, 48) == 0
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros(32, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_dispatch_pack_fp8(cfg, x, s, torch.zeros(10, dtype=torch.uint8,
                                                         device="cuda"), 128)
    assert e.value.code == moe.MOE_EUNSUPPORTED
