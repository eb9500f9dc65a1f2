"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer outputs (expert ids, counts, offsets, masks, slots, packed bytes) must
be bit-exact; gate weights within 1e-6 relative; the combine within 1e-5
relative (fp32 outputs) or 2e-2 absolute (bf16 outputs) of the oracle's
unrounded fp64 sum.  Sizes: reduced-T shapes that span several layout tiles
with a ragged tail, and every workload at its full size with the launch
configuration the benchmark times (there, the combine is checked on sampled
tokens and the packed buffer by a property over all rows).
"""
import numpy as np
import pytest
import torch

import combine_moe_topk_amd as moe
import moe_inputs as mi
import oracle
from helpers import (ATOL_BF16, LAYOUT_KEYS, cfg_of, check_combine_all,
                     check_gate, check_layout, check_out, dev, host,
                     layout_to_host, out_dtype, require_gpu, row_dtype,
                     rows_f64, run_fused, term_scale)

pytestmark = pytest.mark.gpu

SMALL = [
    mi.TINY,
    mi.DEEPSEEK_V3_DECODE,
    mi.MIXTRAL.replace(T=1000, H=256),
    mi.QWEN3.replace(T=777, H=512),
    mi.DEEPSEEK_V3.replace(T=1000, H=520),
    mi.KIMI.replace(T=600, H=256),
]
FULL = [mi.MIXTRAL, mi.QWEN3, mi.DEEPSEEK_V3, mi.KIMI]
ALL = SMALL + FULL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()


def _ids(w):
    return f"{w.name}-T{w.T}-H{w.H}"


# ----------------------------------------------------------------- gate ----

def gpu_gate(w, logits, renorm=True):
    cfg = moe.make_cfg(w.T, w.H, w.E, w.K, w.R, w.N, w.x_dtype, w.out_dtype,
                       renorm)
    idx = torch.empty(w.T * w.K, dtype=torch.int32, device="cuda")
    wt = torch.empty(w.T * w.K, dtype=torch.float32, device="cuda")
    moe.moe_topk_gate(cfg, dev(logits), idx, wt)
    return host(idx).reshape(w.T, w.K), host(wt).reshape(w.T, w.K)


@pytest.mark.parametrize("w", ALL, ids=_ids)
def test_gate(w):
    lg = mi.make_inputs(w, with_x=False)["logits"]
    ref_idx, ref_w = oracle.gate(lg, w.K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


ADV = [("all_equal", lambda T, E, K: mi.logits_all_equal(T, E)),
       ("signed_zeros", lambda T, E, K: mi.logits_signed_zeros(T, E, 5)),
       ("few_levels", lambda T, E, K: mi.logits_few_levels(T, E, 3, 6)),
       ("one_hot", lambda T, E, K: mi.logits_one_hot_experts(T, E, K, 3))]


@pytest.mark.parametrize("name,make", ADV, ids=[a[0] for a in ADV])
@pytest.mark.parametrize("E,K", [(8, 1), (8, 8), (16, 3), (64, 16),
                                 (256, 8), (896, 16), (1000, 32), (3500, 8),
                                 (4096, 5)])
def test_gate_ties(name, make, E, K):
    T = 300
    w = mi.Workload("adv", T=T, H=8, E=E, K=K, R=1, N=1)
    lg = make(T, E, K)
    ref_idx, ref_w = oracle.gate(lg, K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


@pytest.mark.parametrize("name,make", ADV, ids=[a[0] for a in ADV])
@pytest.mark.parametrize("E,K", [(64, 16), (256, 8), (896, 16), (1700, 20)])
def test_gate_ties_many_tokens(name, make, E, K):
    # above 1024 tokens a token takes 16 or 32 lanes instead of a wave
    T = 2000
    w = mi.Workload("adv", T=T, H=8, E=E, K=K, R=1, N=1)
    lg = make(T, E, K)
    ref_idx, ref_w = oracle.gate(lg, K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


def _gate_path_per_wave(lg, K, G):
    """Which selection path each wave of the gate kernel takes (0: at most G
    candidates a group, one LDS entry a lane; 1: at most 2G, two; 2: more,
    the general path), from the kernel's threshold rule restated in numpy:
    theta = min over the group's 16-lane rows of the row's
    ceil(K/rows)-th largest lane maximum (lane sub holds experts sub + jG)."""
    T, E = lg.shape
    C = -(-E // G)
    pad = np.full((T, G * C), -np.inf, np.float32)
    pad[:, :E] = lg
    key = pad.reshape(T, C, G).transpose(0, 2, 1)
    lane_max = key.max(axis=2)
    rows = G // 16
    kk = -(-K // rows)
    srt = -np.sort(-lane_max.reshape(T, rows, 16), axis=2)
    theta = srt[:, :, kk - 1].min(axis=1)
    valid = (np.arange(G)[:, None] + np.arange(C)[None, :] * G) < E
    M = ((key >= theta[:, None, None]) & valid[None]).sum(axis=(1, 2))
    Mw = M.reshape(-1, 64 // G).max(axis=1)
    return np.where(Mw <= G, 0, np.where(Mw <= 2 * G, 1, 2))


# Above 1024 tokens the gate takes G = 16 lanes a token for E = 256, K = 8
# and G = 32 for E = 896, K = 16; the floored logits put every wave of the
# launch on one chosen path, with distinct values (no ties).
@pytest.mark.parametrize("E,K,G,per_lane,path",
                         [(256, 8, 16, 2, 0), (256, 8, 16, 3, 1),
                          (256, 8, 16, 5, 2), (896, 16, 32, 2, 0),
                          (896, 16, 32, 3, 1), (896, 16, 32, 5, 2)])
def test_gate_selection_paths(E, K, G, per_lane, path):
    T = 2048
    lg = mi.logits_floored(T, E, G, K, per_lane, seed=E + per_lane)
    assert (_gate_path_per_wave(lg, K, G) == path).all()
    w = mi.Workload("paths", T=T, H=8, E=E, K=K, R=1, N=1)
    ref_idx, ref_w = oracle.gate(lg, K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


# Few experts (E from 1 to 16, fewer than the group's lanes, so most lanes
# hold padding keys), at a one-token, a one-wave-per-token and a 16-lane
# batch size: ties, signed zeros, few levels, masked experts and the
# no-renormalisation variant.
FEW_EK = [(1, 1), (2, 2), (3, 2), (5, 3), (8, 1), (8, 2), (8, 8), (12, 4),
           (16, 3), (16, 8)]
FEW_LOGITS = ADV + [
    ("normal", lambda T, E, K: np.random.Generator(np.random.PCG64(E + K))
     .standard_normal((T, E), dtype=np.float32)),
    ("masked", lambda T, E, K: mi.logits_masked(T, E, seed=E + K))]


@pytest.mark.parametrize("name,make", FEW_LOGITS,
                         ids=[a[0] for a in FEW_LOGITS])
@pytest.mark.parametrize("E,K", FEW_EK, ids=lambda v: str(v))
@pytest.mark.parametrize("T", [1, 77, 3000])
def test_gate_few_experts(T, E, K, name, make):
    lg = make(T, E, K)
    w = mi.Workload("few", T=T, H=8, E=E, K=K, R=1, N=1)
    ref_idx, ref_w = oracle.gate(lg, K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


@pytest.mark.parametrize("E,K", [(8, 2), (16, 8), (5, 5)])
def test_gate_few_experts_no_renorm(E, K):
    T = 2000
    lg = np.random.Generator(np.random.PCG64(7)).standard_normal(
        (T, E), dtype=np.float32)
    w = mi.Workload("few", T=T, H=8, E=E, K=K, R=1, N=1)
    ref_idx, ref_w = oracle.gate(lg, K, renorm=False)
    idx, wt = gpu_gate(w, lg, renorm=False)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


@pytest.mark.parametrize("T", [300, 2000])  # 64 lanes a token, then 16-32
@pytest.mark.parametrize("E,K", [(8, 2), (32, 8), (64, 16), (256, 8),
                                 (896, 16), (1000, 32)])
def test_gate_masked_logits(T, E, K):
    # -inf logits (masked experts): a threshold of -inf sends a wave to the
    # general path, and -inf picks go to the lowest indexes
    lg = mi.logits_masked(T, E, seed=E + K + T)
    w = mi.Workload("masked", T=T, H=8, E=E, K=K, R=1, N=1)
    ref_idx, ref_w = oracle.gate(lg, K)
    idx, wt = gpu_gate(w, lg)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


def test_gate_no_renorm():
    w = mi.DEEPSEEK_V3.replace(T=1000)
    lg = mi.make_inputs(w, with_x=False)["logits"]
    ref_idx, ref_w = oracle.gate(lg, w.K, renorm=False)
    idx, wt = gpu_gate(w, lg, renorm=False)
    check_gate({"topk_idx": idx, "topk_w": wt}, ref_idx, ref_w)


# --------------------------------------------------------------- layout ----

def gpu_layout(w, idx, layout_tile=0, optional=True):
    cfg = cfg_of(w, layout_tile)
    lay = moe.alloc_layout(cfg, optional=optional)
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_layout(cfg, dev(idx), lay, ws)
    err = moe.moe_read_device_error(ws)
    res = layout_to_host(lay, w.T, w.K, w.N)
    res["dev_error"] = err
    return res


@pytest.mark.parametrize("tile", [0, 64, 1024])
@pytest.mark.parametrize("w", ALL, ids=_ids)
def test_layout(w, tile):
    lg = mi.make_inputs(w, with_x=False)["logits"]
    idx, _ = oracle.gate(lg, w.K)
    ref = oracle.layout(idx, w.E, w.R, w.N)
    res = gpu_layout(w, idx, tile)
    assert res["dev_error"] == 0
    check_layout(res, ref)


@pytest.mark.parametrize("case", [
    # T, E, K, R, N
    (1, 8, 2, 4, 2), (63, 8, 8, 8, 8), (64, 16, 1, 16, 4), (65, 64, 16, 64, 64),
    (257, 256, 8, 64, 8), (5000, 896, 16, 128, 16), (3000, 4, 4, 2, 1),
    (2049, 128, 32, 128, 64)])
def test_layout_random_ids(case):
    T, E, K, R, N = case
    idx = mi.random_topk_idx(T, E, K, seed=T)
    w = mi.Workload("rand", T=T, H=8, E=E, K=K, R=R, N=N)
    ref = oracle.layout(idx, E, R, N)
    for tile in (0, 128):
        res = gpu_layout(w, idx, tile)
        assert res["dev_error"] == 0
        check_layout(res, ref)


def test_layout_one_hot_expert_set():
    # every token picks the same K experts: K experts with T rows each
    w = mi.DEEPSEEK_V3.replace(T=3000)
    lg = mi.logits_one_hot_experts(w.T, w.E, w.K, first=250)
    idx, _ = oracle.gate(lg, w.K)
    ref = oracle.layout(idx, w.E, w.R, w.N)
    check_layout(gpu_layout(w, idx), ref)


def test_layout_without_optional_outputs():
    w = mi.QWEN3.replace(T=999)
    idx, _ = oracle.gate(mi.make_inputs(w, with_x=False)["logits"], w.K)
    ref = oracle.layout(idx, w.E, w.R, w.N)
    res = gpu_layout(w, idx, optional=False)
    for k in ("rank_token_count", "node_mask", "node_count", "node_off",
              "node_slot"):
        assert k not in res
    check_layout(res, ref)


def test_layout_struct_follows_replaced_tensors():
    # the binding keeps a layout's C struct between calls; a field that now
    # holds another tensor (or None) must reach the library on the next call
    w = mi.QWEN3.replace(T=999)
    idx, _ = oracle.gate(mi.make_inputs(w, with_x=False)["logits"], w.K)
    ref = oracle.layout(idx, w.E, w.R, w.N)
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    ws = moe.alloc_workspace(cfg)
    ids = dev(idx.reshape(-1))
    moe.moe_dispatch_layout(cfg, ids, lay, ws)
    old = lay.slot_pos
    old.fill_(-7)
    lay.slot_pos = torch.full_like(old, -9)
    lay.node_slot = None
    moe.moe_dispatch_layout(cfg, ids, lay, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(lay.slot_pos).reshape(w.T, w.K),
                                  ref["slot_pos"])
    assert bool((old == -7).all())
    lay.node_slot = torch.empty(w.T * w.N, dtype=torch.int32, device="cuda")
    moe.moe_dispatch_layout(cfg, ids, lay, ws)
    np.testing.assert_array_equal(host(lay.node_slot).reshape(w.T, w.N),
                                  ref["node_slot"])


# ----------------------------------------------------------------- pack ----

@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_pack(w):
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    ref_lay = oracle.layout(idx, w.E, w.R, w.N)
    ref_send = oracle.pack(d["x"], ref_lay["slot_pos"])
    cfg = cfg_of(w)
    send = torch.zeros((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_pack(cfg, dev(d["x"]), dev(ref_lay["slot_pos"]), send)
    np.testing.assert_array_equal(host(send), ref_send)


# The pack switches to its piece-per-wave kernel from 1 GiB of destination
# rows up: this shape (200000 rows of 6000 bytes) reaches it with a ragged
# last piece per row (375 16-byte vectors, pieces of 128) and an odd K.
LARGE_RAGGED = mi.Workload("large_ragged", T=40000, H=3000, E=60, K=5, R=15,
                           N=5, x_dtype=mi.BF16, out_dtype=mi.BF16)
# Wider tokens: K = 20 and K = 32 put 10 and 16 waves on each piece of x,
# spread over several workgroups.
LARGE_WIDE = [mi.Workload("large_k20", T=3800, H=7168, E=40, K=20, R=8, N=4,
                          x_dtype=mi.BF16, out_dtype=mi.BF16),
              mi.Workload("large_k32", T=2400, H=7168, E=64, K=32, R=16, N=8,
                          x_dtype=mi.BF16, out_dtype=mi.BF16)]


@pytest.mark.parametrize("w", [LARGE_RAGGED] + LARGE_WIDE, ids=_ids)
def test_pack_large_ragged(w):
    assert w.T * w.K * w.H * 2 >= 1 << 30
    x = mi.random_x(w.T, w.H, w.x_dtype, seed=3)
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=3)
    slot_pos = oracle.layout(idx, w.E, w.R, w.N)["slot_pos"]
    send = torch.zeros((w.T * w.K, w.H), dtype=row_dtype(w), device="cuda")
    moe.moe_dispatch_pack(cfg_of(w), dev(x), dev(slot_pos), send)
    np.testing.assert_array_equal(host(send), oracle.pack(x, slot_pos))


# -------------------------------------------------------------- combine ----

@pytest.mark.parametrize("ydt,odt", [(mi.BF16, mi.BF16), (mi.F32, mi.F32),
                                     (mi.BF16, mi.F32), (mi.F32, mi.BF16)])
@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_combine(w, ydt, odt):
    w = w.replace(x_dtype=ydt, out_dtype=odt)
    d = mi.make_inputs(w, with_x=False)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    y = mi.random_x(w.T * w.K, w.H, ydt, seed=17)  # arbitrary expert outputs
    scale = d["expert_scale"]
    ref_out, exact = oracle.combine(y, lay["slot_pos"], wt, idx, scale, odt)
    cfg = cfg_of(w)
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    moe.moe_combine(cfg, dev(y), dev(lay["slot_pos"]), dev(wt), dev(idx),
                    None if scale is None else dev(scale), out)
    got = host(out)
    coef = wt.astype(np.float64) * (1.0 if scale is None
                                    else scale[idx].astype(np.float64))
    check_out(got, exact, term_scale(rows_f64(y), lay["slot_pos"], coef), odt)
    if odt == mi.BF16:
        # almost every bf16 element also equals the oracle's own rounding
        # (fp32 outputs differ from the fp64 sum in the last bits by design)
        assert np.mean(got == ref_out) > 0.99


# From 1 GiB of y rows the combine switches to its burst kernel (groups of 8
# tokens reduced into LDS, then written together): this shape reaches it
# with a ragged last group (45003 tokens), a row of 375 units (not a wave
# multiple) and dropped slots (-1) that must add nothing.
@pytest.mark.parametrize("odt", [mi.BF16, mi.F32])
def test_combine_burst_ragged(odt):
    w = mi.Workload("burst_ragged", T=45003, H=3000, E=60, K=4, R=15, N=5,
                    x_dtype=mi.BF16, out_dtype=odt)
    assert w.T * w.K * w.H * 2 >= 1 << 30 and w.T % 8 == 3
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=5)
    rng = np.random.Generator(np.random.PCG64(5))
    # weights summing to 1, as the gate gives: |out| stays below 8, where
    # the bf16 rounding step is within the 2e-2 bound
    wt = rng.random((w.T, w.K), dtype=np.float32) + np.float32(0.1)
    wt = (wt / wt.sum(axis=1, keepdims=True)).astype(np.float32)
    scale = (1.0 + 0.01 * (np.arange(w.E) % 8)).astype(np.float32)
    slot_pos = oracle.layout(idx, w.E, w.R, w.N)["slot_pos"].copy()
    drop = rng.random((w.T, w.K)) < 0.05
    drop[-1, :] = True  # the last token: every slot dropped, so out is 0
    slot_pos[drop] = -1
    # 1 GiB of rows drawn from 4096 distinct seeded rows (cheap to generate)
    y = mi.random_x(4096, w.H, mi.BF16, seed=6)[
        rng.integers(0, 4096, w.T * w.K)]
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    moe.moe_combine(cfg_of(w), dev(y), dev(slot_pos), dev(wt), dev(idx),
                    dev(scale), out)
    got = host(out)
    # every token, fp32 outputs against sum |terms| as well
    check_combine_all(got, y, slot_pos, wt, idx, scale, odt)
    if odt == mi.BF16:
        ref_out, _ = oracle.combine(y, slot_pos, wt, idx, scale, odt)
        assert np.mean(got == ref_out) > 0.99
    assert not got[-1].any()


# The fp32-row burst kernels (8 fp32 elements a thread take two 16-byte
# loads; K = 8 and K = 4 keep 8 row loads in flight): 1 GiB or more of fp32
# y rows, every token compared, both output types.
@pytest.mark.parametrize("K", [8, 4])
@pytest.mark.parametrize("odt", [mi.BF16, mi.F32])
def test_combine_burst_f32_rows(odt, K):
    T = 9000 if K == 8 else 18000
    w = mi.Workload("burst_f32", T=T, H=4096, E=64, K=K, R=16, N=4,
                    x_dtype=mi.F32, out_dtype=odt)
    assert w.T * w.K * w.H * 4 >= 1 << 30
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=11)
    rng = np.random.Generator(np.random.PCG64(11))
    wt = rng.random((w.T, w.K), dtype=np.float32) + np.float32(0.1)
    wt = (wt / wt.sum(axis=1, keepdims=True)).astype(np.float32)
    scale = (1.0 + 0.01 * (np.arange(w.E) % 8)).astype(np.float32)
    slot_pos = oracle.layout(idx, w.E, w.R, w.N)["slot_pos"]
    # 1.2 GB of fp32 rows drawn from 4096 distinct seeded rows
    y = mi.random_x(4096, w.H, mi.F32, seed=12)[
        rng.integers(0, 4096, w.T * w.K)]
    out = torch.empty((w.T, w.H), dtype=out_dtype(w), device="cuda")
    moe.moe_combine(cfg_of(w), dev(y), dev(slot_pos), dev(wt), dev(idx),
                    dev(scale), out)
    check_combine_all(host(out), y, slot_pos, wt, idx, scale, odt)


# ---------------------------------------------------------------- fused ----

@pytest.mark.parametrize("w", SMALL, ids=_ids)
def test_fused_small(w):
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine(d["x"], d["logits"], w.K, w.R, w.N,
                                  d["expert_scale"], w.out_dtype)
    res = run_fused(w, d)
    assert res["dev_error"] == 0
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(res["send"], ref["send"])
    coef = ref["topk_w"].astype(np.float64)
    if d["expert_scale"] is not None:
        coef = coef * d["expert_scale"][ref["topk_idx"]]
    check_out(res["out"], ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef),
              w.out_dtype)


@pytest.mark.parametrize("w,seed", [(w, None) for w in FULL] +
                         [(mi.DEEPSEEK_V3, 1), (mi.QWEN3, 1)],
                         ids=lambda v: _ids(v) if isinstance(v, mi.Workload)
                         else f"seed{v}")
def test_fused_full_size(w, seed):
    # every workload at its full size with its seed, and seed 1 as a rerun
    # of the clustered and the Zipf-skewed logits
    d = mi.make_inputs(w, seed=seed)
    res = run_fused(w, d, keep_device=True)
    assert res["dev_error"] == 0
    idx, wt = oracle.gate(d["logits"], w.K)
    check_gate(res, idx, wt)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    check_layout(res, lay)
    # every packed row is the x row the oracle's permutation names
    src_tok = torch.from_numpy((lay["row_src"] // w.K).astype(np.int64)).cuda()
    send, x = res["send_dev"], res["x_dev"]
    for lo in range(0, w.T * w.K, 1 << 16):
        hi = min(lo + (1 << 16), w.T * w.K)
        assert torch.equal(send[lo:hi], x[src_tok[lo:hi]]), (lo, hi)
    # every token: the oracle's own pack, then its fp64 combine of the
    # packed rows, a chunk of tokens at a time
    ref_send = oracle.pack(d["x"], lay["slot_pos"])
    check_combine_all(res["out"], ref_send, lay["slot_pos"], wt, idx,
                      d["expert_scale"], w.out_dtype)


# ----------------------------------------------------------- edge cases ----

def test_empty_input():
    w = mi.DEEPSEEK_V3.replace(T=0, H=64)
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    lay.expert_count.fill_(-7)
    lay.expert_off.fill_(-7)
    ws = moe.alloc_workspace(cfg)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    xb = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    moe.moe_dispatch_combine(cfg, xb, f, None, e, f, lay, xb, xb, ws)
    assert moe.moe_read_device_error(ws) == 0
    assert torch.all(lay.expert_count == 0) and torch.all(lay.expert_off == 0)
    assert torch.all(lay.node_off == 0) and torch.all(lay.rank_off == 0)


@pytest.mark.parametrize("T,H,E,K,R,N,xdt,odt", [
    (1, 8, 8, 2, 4, 2, mi.BF16, mi.BF16),      # one token, one unit per row
    (1, 7168, 256, 8, 64, 8, mi.BF16, mi.BF16),
    (130, 72, 16, 16, 4, 2, mi.BF16, mi.F32),  # K = E, 9 units: ragged lanes
    (70, 1032, 8, 1, 8, 1, mi.F32, mi.F32),    # K = 1, 129 units
    (200, 136, 32, 5, 8, 4, mi.F32, mi.BF16),  # K not a power of two
    (129, 264, 64, 32, 64, 64, mi.BF16, mi.BF16),  # K = 32, N = 64
    (300, 64, 4096, 8, 64, 8, mi.BF16, mi.BF16),  # E = 4096: 64-token tiles
    (40, 16384, 16, 4, 4, 2, mi.BF16, mi.F32),  # H = 16384: 2048 units
    # past the decode sizes: E = 4096 (64 keys a lane, one-wave layout
    # tiles, the rank kernel's loop over a wide table) and K = 32, N = 64
    (3000, 64, 4096, 8, 64, 8, mi.BF16, mi.BF16),
    (2000, 64, 64, 32, 64, 64, mi.BF16, mi.F32),
])
def test_fused_edge_shapes(T, H, E, K, R, N, xdt, odt):
    w = mi.Workload("edge", T=T, H=H, E=E, K=K, R=R, N=N, x_dtype=xdt,
                    out_dtype=odt, expert="mod8")
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine(d["x"], d["logits"], K, R, N,
                                  d["expert_scale"], odt)
    res = run_fused(w, d)
    assert res["dev_error"] == 0
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(res["send"], ref["send"])
    coef = ref["topk_w"].astype(np.float64) * d["expert_scale"][ref["topk_idx"]]
    check_out(res["out"], ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef), odt)


# Past 1024 tokens, when the gate takes 16 lanes a token (E <= 512, K <= 8)
# and the layout tile holds 64 tokens (the default tile for these sizes),
# the fused call runs the gate and the layout's count pass as one launch:
# ragged tails (a last tile of one token, partial last waves), padding keys
# (E not a multiple of 16), masked logits, no optional outputs, and one
# 128-token tile, which takes the separate launches.  Checked against the
# oracle and bit for bit against the separate gate, layout, pack and
# combine calls.
GATE_COUNT_SHAPES = [
    # T, H, E, K, R, N, tile, masked, optional
    (1025, 64, 8, 2, 8, 1, 64, False, True),
    (1500, 128, 128, 8, 64, 8, 0, False, True),
    (2049, 64, 256, 8, 64, 8, 64, False, True),
    (3000, 64, 128, 8, 64, 8, 0, True, True),
    (4133, 32, 512, 8, 128, 16, 64, True, False),
    (1100, 72, 48, 6, 8, 4, 0, False, True),
    (2100, 64, 256, 8, 64, 8, 128, False, True),
    (2000, 64, 128, 8, 64, 64, 0, False, True),  # 64 nodes: mask bit 63
]


@pytest.mark.parametrize("case", GATE_COUNT_SHAPES,
                         ids=lambda c: f"T{c[0]}-E{c[2]}-K{c[3]}-tile{c[6]}")
def test_fused_gate_count(case):
    T, H, E, K, R, N, tile, masked, optional = case
    w = mi.Workload("gate_count", T=T, H=H, E=E, K=K, R=R, N=N,
                    expert="mod8")
    d = mi.make_inputs(w)
    if masked:
        d["logits"] = mi.logits_masked(T, E, seed=T + E)
    ref = oracle.dispatch_combine(d["x"], d["logits"], K, R, N,
                                  d["expert_scale"], w.out_dtype)
    cfg = cfg_of(w, tile)
    x, lg = dev(d["x"]), dev(d["logits"])
    sc = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg, optional=optional)
    send = torch.empty((T * K, H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((T, H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine(cfg, x, lg, sc, idx, wt, lay, send, out, ws)
    assert moe.moe_read_device_error(ws) == 0
    res = layout_to_host(lay, T, K, N)
    res.update(topk_idx=host(idx).reshape(T, K), topk_w=host(wt).reshape(T, K))
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(host(send), ref["send"])
    coef = ref["topk_w"].astype(np.float64)
    if d["expert_scale"] is not None:
        coef = coef * d["expert_scale"][ref["topk_idx"]]
    check_out(host(out), ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef),
              w.out_dtype)
    # the same bits as the gate, layout, pack and combine calls one by one
    idx2, wt2 = torch.empty_like(idx), torch.empty_like(wt)
    moe.moe_topk_gate(cfg, lg, idx2, wt2)
    assert torch.equal(idx, idx2) and torch.equal(wt, wt2)
    ws2 = moe.alloc_workspace(cfg)
    lay2 = moe.alloc_layout(cfg, optional=optional)
    send2, out2 = torch.empty_like(send), torch.empty_like(out)
    moe.moe_dispatch_layout(cfg, idx2, lay2, ws2)
    moe.moe_dispatch_pack(cfg, x, lay2.slot_pos, send2)
    moe.moe_combine(cfg, send2, lay2.slot_pos, wt2, idx2, sc, out2)
    for name in LAYOUT_KEYS:
        a, b = getattr(lay, name), getattr(lay2, name)
        if a is not None:
            assert torch.equal(a, b), name
    assert torch.equal(send, send2) and torch.equal(out, out2)


def _gate_count_random_cases(n=6, seed=20261203):
    """Seeded shapes on the fused gate-count path: more than 1024 tokens,
    E <= 512 and K <= 8 (16 lanes a token), the default 64-token tile."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    while len(cases) < n:
        E = int(rng.choice([8, 16, 40, 64, 96, 128, 200, 256, 384, 512]))
        K = int(rng.integers(1, min(8, E) + 1))
        R = int(rng.choice([r for r in (1, 2, 4, 8, 16, 32, 64) if E % r == 0]))
        N = int(rng.choice([m for m in (1, 2, 4, 8) if R % m == 0]))
        T = int(rng.integers(1025, 6000))
        cases.append((T, 64, E, K, R, N))
    return cases


@pytest.mark.parametrize("case", _gate_count_random_cases(),
                         ids=lambda c: f"T{c[0]}-E{c[2]}-K{c[3]}-R{c[4]}-N{c[5]}")
def test_fused_gate_count_random(case):
    T, H, E, K, R, N = case
    w = mi.Workload("gate_count_rand", T=T, H=H, E=E, K=K, R=R, N=N,
                    expert="mod8", seed=T)
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine(d["x"], d["logits"], K, R, N,
                                  d["expert_scale"], w.out_dtype)
    res = run_fused(w, d)
    assert res["dev_error"] == 0
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(res["send"], ref["send"])
    coef = ref["topk_w"].astype(np.float64) * d["expert_scale"][ref["topk_idx"]]
    check_out(res["out"], ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef),
              w.out_dtype)


# Few experts past the decode sizes, through the fused call at several
# layout tile sizes (64-token tiles take the gate with the count pass).
FEW_COUNT_SHAPES = [
    # T, H, E, K, R, N, tile, masked, optional
    (4096, 64, 8, 2, 8, 1, 0, False, True),      # the Mixtral shape's E, K
    (1025, 64, 5, 3, 5, 1, 64, False, True),
    (3333, 32, 16, 8, 4, 2, 256, True, True),
    (5000, 64, 12, 4, 6, 3, 1024, False, False),
    (2049, 64, 16, 1, 16, 16, 128, True, True),
    (4500, 64, 2, 2, 2, 2, 0, False, True),
]


@pytest.mark.parametrize("case", FEW_COUNT_SHAPES,
                         ids=lambda c: f"T{c[0]}-E{c[2]}-K{c[3]}-tile{c[6]}")
def test_fused_few_experts(case):
    test_fused_gate_count(case)


# Batches of up to 1024 tokens (T*K <= 4096) take the one-launch decode
# step after the gate: ragged and tiny batches, K = 1 and K = E, many nodes,
# E = 1024, fp32 rows and outputs, no expert scale, no optional outputs.
DECODE_SHAPES = [
    # T, H, E, K, R, N, xdt, odt, expert, optional
    (1, 64, 8, 1, 8, 1, mi.BF16, mi.BF16, "mod8", True),
    (37, 7168, 256, 8, 64, 8, mi.BF16, mi.BF16, "mod8", True),
    (128, 7168, 256, 8, 64, 8, mi.BF16, mi.F32, "identity", False),
    (77, 520, 64, 32, 64, 64, mi.F32, mi.BF16, "mod8", True),   # K = 32
    (255, 1000, 1024, 16, 128, 16, mi.BF16, mi.BF16, "mod8", True),
    (512, 256, 128, 8, 64, 8, mi.F32, mi.F32, "mod8", True),
    (1024, 128, 32, 4, 8, 2, mi.BF16, mi.BF16, "mod8", False),
]


@pytest.mark.parametrize("case", DECODE_SHAPES,
                         ids=lambda c: f"T{c[0]}-H{c[1]}-E{c[2]}-K{c[3]}")
def test_fused_decode_path(case):
    T, H, E, K, R, N, xdt, odt, expert, optional = case
    w = mi.Workload("decode", T=T, H=H, E=E, K=K, R=R, N=N, x_dtype=xdt,
                    out_dtype=odt, expert=expert)
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine(d["x"], d["logits"], K, R, N,
                                  d["expert_scale"], odt)
    cfg = cfg_of(w)
    x, lg = dev(d["x"]), dev(d["logits"])
    sc = None if d["expert_scale"] is None else dev(d["expert_scale"])
    idx = torch.empty(T * K, dtype=torch.int32, device="cuda")
    wt = torch.empty(T * K, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg, optional=optional)
    send = torch.empty((T * K, H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((T, H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine(cfg, x, lg, sc, idx, wt, lay, send, out, ws)
    assert moe.moe_read_device_error(ws) == 0
    res = layout_to_host(lay, T, K, N)
    res.update(topk_idx=host(idx).reshape(T, K), topk_w=host(wt).reshape(T, K))
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(host(send), ref["send"])
    coef = ref["topk_w"].astype(np.float64)
    if d["expert_scale"] is not None:
        coef = coef * d["expert_scale"][ref["topk_idx"]]
    check_out(host(out), ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef), odt)
    # the same bits as the layout, pack and combine calls one by one
    ws2 = moe.alloc_workspace(cfg)
    lay2 = moe.alloc_layout(cfg, optional=optional)
    send2 = torch.empty_like(send)
    out2 = torch.empty_like(out)
    moe.moe_dispatch_layout(cfg, idx, lay2, ws2)
    moe.moe_dispatch_pack(cfg, x, lay2.slot_pos, send2)
    moe.moe_combine(cfg, send2, lay2.slot_pos, wt, idx, sc, out2)
    for name in LAYOUT_KEYS:
        a, b = getattr(lay, name), getattr(lay2, name)
        if a is not None:
            assert torch.equal(a, b), name
    assert torch.equal(send, send2) and torch.equal(out, out2)


@pytest.mark.parametrize("T,K", [(1, 3), (37, 8)])
def test_fused_decode_ids_4byte_aligned(T, K):
    # expert ids and weights in views that start 4 bytes into their storage
    # (and T*K = 3, under one 16-byte vector): the decode kernel reads ids one
    # by one, so alignment and short lengths are the caller's to choose
    w = mi.Workload("decode", T=T, H=256, E=64, K=K, R=8, N=2)
    d = mi.make_inputs(w)
    ref = oracle.dispatch_combine(d["x"], d["logits"], K, 8, 2,
                                  d["expert_scale"], w.out_dtype)
    cfg = cfg_of(w)
    idx_store = torch.full((T * K + 1,), -7, dtype=torch.int32, device="cuda")
    wt_store = torch.zeros(T * K + 1, dtype=torch.float32, device="cuda")
    idx, wt = idx_store[1:], wt_store[1:]
    assert idx.data_ptr() % 16 == 4
    lay = moe.alloc_layout(cfg)
    send = torch.empty((T * K, w.H), dtype=row_dtype(w), device="cuda")
    out = torch.empty((T, w.H), dtype=out_dtype(w), device="cuda")
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_combine(cfg, dev(d["x"]), dev(d["logits"]),
                             dev(d["expert_scale"]), idx, wt, lay, send, out,
                             ws)
    assert moe.moe_read_device_error(ws) == 0
    assert int(idx_store[0]) == -7
    res = layout_to_host(lay, T, K, 2)
    res.update(topk_idx=host(idx).reshape(T, K), topk_w=host(wt).reshape(T, K))
    check_gate(res, ref["topk_idx"], ref["topk_w"])
    check_layout(res, ref)
    np.testing.assert_array_equal(host(send), ref["send"])
    coef = ref["topk_w"].astype(np.float64) * \
        d["expert_scale"][ref["topk_idx"]]
    check_out(host(out), ref["out_exact"],
              term_scale(rows_f64(ref["send"]), ref["slot_pos"], coef),
              w.out_dtype)


def test_identity_experts_return_input():
    # renormalised weights and identity experts: out == x (bf16), the dispatch
    # permutation inverting exactly under the combine
    w = mi.DEEPSEEK_V3.replace(T=2000, H=1024, expert="identity")
    d = mi.make_inputs(w)
    res = run_fused(w, d)
    xf = mi.bf16_bits_to_f32(d["x"]).astype(np.float64)
    got = mi.bf16_bits_to_f32(res["out"]).astype(np.float64)
    assert np.max(np.abs(got - xf)) <= ATOL_BF16
    assert np.mean(res["out"] == d["x"]) > 0.999


def test_one_hot_weights_invert_pack():
    w = mi.KIMI.replace(T=500, H=512)
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    cfg = cfg_of(w)
    send = torch.empty((w.T * w.K, w.H), dtype=torch.bfloat16, device="cuda")
    sp = dev(lay["slot_pos"])
    moe.moe_dispatch_pack(cfg, dev(d["x"]), sp, send)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    for k in (0, w.K - 1):
        oh = np.zeros((w.T, w.K), np.float32)
        oh[:, k] = 1.0
        moe.moe_combine(cfg, send, sp, dev(oh), None, None, out)
        np.testing.assert_array_equal(host(out), d["x"])


# -------------------------------------------------------- determinism ----

@pytest.mark.parametrize("w", [mi.QWEN3, mi.KIMI.replace(T=5000)], ids=_ids)
def test_deterministic_across_runs_and_tiles(w):
    d = mi.make_inputs(w)
    a = run_fused(w, d, layout_tile=0)
    b = run_fused(w, d, layout_tile=0)
    c = run_fused(w, d, layout_tile=64)
    e = run_fused(w, d, layout_tile=1024)
    for other in (b, c, e):
        for k in LAYOUT_KEYS + ("topk_idx", "topk_w", "send", "out"):
            np.testing.assert_array_equal(a[k], other[k], err_msg=k)


# ------------------------------------------------------ device errors ----

def test_device_error_word():
    w = mi.Workload("err", T=100, H=8, E=16, K=2, R=4, N=2)
    idx = mi.random_topk_idx(w.T, w.E, w.K, seed=1)
    assert gpu_layout(w, idx)["dev_error"] == 0
    bad = idx.copy()
    bad[7, 1] = 16
    bad[9, 0] = -3
    res = gpu_layout(w, bad)
    assert res["dev_error"] == moe.MOE_DEVERR_EXPERT_RANGE
    assert res["slot_pos"][7, 1] == -1 and res["slot_pos"][9, 0] == -1
    ok = res["slot_pos"][res["slot_pos"] >= 0]
    assert ok.max() < w.T * w.K
    dup = idx.copy()
    dup[3, 1] = dup[3, 0]
    assert gpu_layout(w, dup)["dev_error"] == moe.MOE_DEVERR_DUP_EXPERT
    # the word is sticky until read with clear
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    ws = moe.alloc_workspace(cfg)
    moe.moe_dispatch_layout(cfg, dev(bad), lay, ws)
    moe.moe_dispatch_layout(cfg, dev(idx), lay, ws)
    assert moe.moe_read_device_error(ws, clear=False) == 1
    assert moe.moe_read_device_error(ws, clear=True) == 1
    assert moe.moe_read_device_error(ws) == 0


def test_host_errors_enqueue_nothing():
    w = mi.DEEPSEEK_V3.replace(T=64, H=64)
    cfg = cfg_of(w)
    lay = moe.alloc_layout(cfg)
    ws = moe.alloc_workspace(cfg)
    small = ws[: moe.moe_workspace_bytes(cfg) - 256]
    idx = torch.zeros(w.T * w.K, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_dispatch_layout(cfg, idx, lay, small)
    assert ei.value.code == moe.MOE_EWORKSPACE
    x = torch.zeros((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    send = torch.zeros((w.T * w.K * w.H + 1,), dtype=torch.bfloat16,
                       device="cuda")
    sp = torch.zeros(w.T * w.K, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_dispatch_pack(cfg, x, sp, send[1:])  # 2-byte aligned
    assert ei.value.code == moe.MOE_EUNSUPPORTED


def test_undersized_buffers_refused_before_enqueue():
    # the binding checks every buffer against cfg before the C call: an
    # undersized tensor raises ValueError and no kernel touches any output
    w = mi.DEEPSEEK_V3.replace(T=64, H=64)
    cfg = cfg_of(w)
    T, K, H = w.T, w.K, w.H
    d = mi.make_inputs(w)
    x, lg = dev(d["x"]), dev(d["logits"])
    idx = torch.full((T * K,), -5, dtype=torch.int32, device="cuda")
    wt = torch.full((T * K,), -5.0, dtype=torch.float32, device="cuda")
    lay = moe.alloc_layout(cfg)
    lay.slot_pos.fill_(-5)
    send = torch.full((T * K, H), 3.0, dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = moe.alloc_workspace(cfg)
    torch.cuda.synchronize()
    short = {"send": send[:-1], "out": out[:-1], "x": x[:-1],
             "logits": lg[:-1], "topk_idx": idx[:-1], "topk_w": wt[:-1]}
    for name, t in short.items():
        args = dict(x=x, logits=lg, topk_idx=idx, topk_w=wt, send=send,
                    out=out)
        args[name] = t
        with pytest.raises(ValueError, match=name):
            moe.moe_dispatch_combine(cfg, args["x"], args["logits"], None,
                                     args["topk_idx"], args["topk_w"], lay,
                                     args["send"], args["out"], ws)
    lay.node_slot = lay.node_slot[:-1]
    with pytest.raises(ValueError, match="node_slot"):
        moe.moe_dispatch_combine(cfg, x, lg, None, idx, wt, lay, send, out, ws)
    with pytest.raises(ValueError, match="^y:"):
        moe.moe_combine(cfg, send[:-1], lay.slot_pos, wt, idx, None, out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()) and bool((send == 3.0).all())
    assert bool((idx == -5).all()) and bool((wt == -5.0).all())
    assert bool((lay.slot_pos == -5).all())
