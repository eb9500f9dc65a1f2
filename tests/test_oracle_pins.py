"""Pins for the CPU oracle: it is checked against things other than itself.

Library routines (stable argsort, bincount, cumsum, lexsort, matmul, scipy's
softmax), closed forms, invariants the pages state, brute-force enumeration on
tiny inputs and a hand-worked example.  A plausible slip anywhere in the
oracle (a wrong tie rule, an off-by-one offset, a transposed index, a missing
weight or scale) fails at least one test here.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Reduced-T versions of every workload shape (full E, K, R, N).
SHAPES = [mi.TINY, mi.MIXTRAL.replace(T=512, H=64),
          mi.QWEN3.replace(T=512, H=64), mi.DEEPSEEK_V3.replace(T=512, H=64),
          mi.KIMI.replace(T=256, H=64)]


def _canon(lg):
    return lg + np.float32(0.0)  # -0.0 + 0.0 == +0.0


def _adversarial_logits():
    yield "all_equal", mi.logits_all_equal(64, 16)
    yield "signed_zeros", mi.logits_signed_zeros(64, 16, seed=3)
    yield "few_levels", mi.logits_few_levels(64, 16, levels=3, seed=4)
    yield "one_hot", mi.logits_one_hot_experts(64, 16, 4, first=13)


# ---------------------------------------------------------------- gate ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1])
def test_gate_equals_stable_argsort(w, seed):
    lg = mi.make_inputs(w, seed=seed, with_x=False)["logits"]
    idx, _ = oracle.gate(lg, w.K)
    ref = np.argsort(-_canon(lg), axis=1, kind="stable")[:, :w.K]
    np.testing.assert_array_equal(idx, ref)


@pytest.mark.parametrize("name,lg", list(_adversarial_logits()))
@pytest.mark.parametrize("K", [1, 3, 8, 16])
def test_gate_ties_equal_stable_argsort(name, lg, K):
    idx, _ = oracle.gate(lg, K)
    ref = np.argsort(-_canon(lg), axis=1, kind="stable")[:, :K]
    np.testing.assert_array_equal(idx, ref)


def _key(l, e):
    # larger logit first, then lower index
    return (float(l), -e)


@pytest.mark.parametrize("seed", range(6))
def test_gate_brute_force_subsets(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    for _ in range(20):
        E = int(rng.integers(1, 8))
        K = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 5))
        # coarse values so that ties are common
        lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
        lg[rng.random((T, E)) < 0.2] = -0.0
        idx, _ = oracle.gate(lg, K)
        for t in range(T):
            winners = []
            for S in itertools.combinations(range(E), K):
                rest = [e for e in range(E) if e not in S]
                if all(_key(lg[t, a], a) > _key(lg[t, b], b)
                       for a in S for b in rest):
                    winners.append(S)
            assert len(winners) == 1
            order = sorted(winners[0], key=lambda e: _key(lg[t, e], e),
                           reverse=True)
            assert list(idx[t]) == order


def test_gate_special_cases():
    lg = mi.make_inputs(mi.QWEN3.replace(T=200), with_x=False)["logits"]
    idx, w = oracle.gate(lg, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)
    E = lg.shape[1]
    idx, w = oracle.gate(lg[:8], E)
    np.testing.assert_array_equal(
        idx, np.argsort(-lg[:8], axis=1, kind="stable"))
    eq = mi.logits_all_equal(5, 12)
    idx, w = oracle.gate(eq, 4)
    np.testing.assert_array_equal(idx, np.tile(np.arange(4), (5, 1)))
    assert np.all(w == np.float32(0.25))


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_gate_weights_sum_and_ratios(w):
    lg = mi.make_inputs(w, with_x=False)["logits"]
    idx, wt = oracle.gate(lg, w.K)
    s = wt.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= w.K * 2.0 ** -24)
    sel = np.take_along_axis(lg, idx, axis=1).astype(np.float64)
    # w_i / w_0 = exp(l_i - l_0) with both rounded to fp32: 2 half-ulps
    ratio = wt[:, 1:].astype(np.float64) / wt[:, :1]
    np.testing.assert_allclose(ratio, np.exp(sel[:, 1:] - sel[:, :1]),
                               rtol=2.5 * 2.0 ** -24, atol=0)
    assert np.all(np.diff(wt, axis=1) <= 0)  # slots ordered by weight


def test_gate_no_renorm_is_full_softmax():
    w = mi.DEEPSEEK_V3.replace(T=300)
    lg = mi.make_inputs(w, with_x=False)["logits"]
    idx, wt = oracle.gate(lg, w.K, renorm=False)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(wt, np.take_along_axis(p, idx, axis=1),
                               rtol=2.0 ** -23, atol=0)


# -------------------------------------------------------------- layout ----

def _check_layout(idx, E, R, N, lay):
    T, K = idx.shape
    flat = idx.ravel()
    # Cobalt Section 3.1: every (token, expert) task executes once -> K*T
    assert lay["expert_count"].sum() == T * K
    np.testing.assert_array_equal(lay["expert_count"],
                                  np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(
        lay["expert_off"], np.concatenate([[0], np.cumsum(lay["expert_count"])]))
    np.testing.assert_array_equal(
        lay["rank_count"], lay["expert_count"].reshape(R, E // R).sum(axis=1))
    np.testing.assert_array_equal(
        lay["rank_off"], np.concatenate([[0], np.cumsum(lay["rank_count"])]))
    # distinct tokens per rank, via unique (token, rank) pairs
    rank = idx // (E // R)
    pairs = np.unique(np.stack([np.repeat(np.arange(T), K), rank.ravel()], 1),
                      axis=0)
    np.testing.assert_array_equal(lay["rank_token_count"],
                                  np.bincount(pairs[:, 1], minlength=R))
    rc, rtc = lay["rank_count"], lay["rank_token_count"]
    assert np.all(rc >= rtc) and np.all(rtc >= -(-rc // (E // R)))
    # dispatch permutation: stable sort of the flattened expert ids
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(lay["row_src"], order)
    sp = lay["slot_pos"].ravel()
    np.testing.assert_array_equal(np.sort(sp), np.arange(T * K))
    np.testing.assert_array_equal(sp[order], np.arange(T * K))
    for e in range(E):
        seg = lay["row_src"][lay["expert_off"][e]:lay["expert_off"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // K) > 0)  # tokens strictly increase
    # node dedup: bits = the set of distinct nodes a token reaches
    node = idx // (E // N)
    mask = lay["node_mask"]
    for t in range(T):
        bits = {n for n in range(64) if int(mask[t]) >> n & 1}
        assert bits == set(node[t].tolist())
    pop = np.array([bin(int(m)).count("1") for m in mask])
    per_node = E // N
    assert np.all(pop <= min(K, N))
    assert np.all(pop >= -(-K // per_node))
    npairs = np.unique(np.stack([np.repeat(np.arange(T), K), node.ravel()], 1),
                       axis=0)
    np.testing.assert_array_equal(lay["node_count"],
                                  np.bincount(npairs[:, 1], minlength=N))
    assert lay["node_count"].sum() == pop.sum()
    np.testing.assert_array_equal(
        lay["node_off"], np.concatenate([[0], np.cumsum(lay["node_count"])]))
    # node_slot: rank of (node, token) in lexicographic order of crossings
    o = np.lexsort((npairs[:, 0], npairs[:, 1]))
    expect = np.full((T, N), -1, np.int32)
    expect[npairs[o, 0], npairs[o, 1]] = np.arange(len(o))
    np.testing.assert_array_equal(lay["node_slot"], expect)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1])
def test_layout_pins(w, seed):
    lg = mi.make_inputs(w, seed=seed, with_x=False)["logits"]
    idx, _ = oracle.gate(lg, w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    _check_layout(idx, w.E, w.R, w.N, lay)


@pytest.mark.parametrize("case", [
    (8, 8, 1, 1, 1), (8, 8, 8, 8, 8), (64, 16, 4, 4, 2), (33, 8, 3, 8, 1),
    (100, 32, 5, 8, 4), (7, 64, 16, 64, 64), (1, 4, 4, 2, 1), (0, 8, 2, 4, 2)])
def test_layout_pins_random_ids(case):
    T, E, K, R, N = case
    idx = mi.random_topk_idx(T, E, K, seed=T + E)
    lay = oracle.layout(idx, E, R, N)
    if T:
        _check_layout(idx, E, R, N, lay)
    else:
        assert lay["expert_count"].sum() == 0


def test_layout_brute_force_definition():
    # slot of (t,k) = segment start + number of earlier tokens that chose
    # the same expert, counted by explicit loops on a tiny case
    rng = np.random.Generator(np.random.PCG64(7))
    for _ in range(30):
        E = int(rng.choice([2, 4, 8]))
        K = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 9))
        R = int(rng.choice([r for r in (1, 2, 4, 8) if E % r == 0]))
        N = int(rng.choice([n for n in (1, 2, 4) if R % n == 0]))
        idx = mi.random_topk_idx(T, E, K, seed=int(rng.integers(1 << 30)))
        lay = oracle.layout(idx, E, R, N)
        for t in range(T):
            for k in range(K):
                e = idx[t, k]
                start = sum(int((idx == f).sum()) for f in range(e))
                before = sum(1 for u in range(t) if e in idx[u])
                assert lay["slot_pos"][t, k] == start + before


def test_layout_single_node_mask_is_one():
    idx = mi.random_topk_idx(50, 16, 4, seed=2)
    lay = oracle.layout(idx, 16, 8, 1)
    assert np.all(lay["node_mask"] == 1)
    assert lay["node_count"][0] == 50
    np.testing.assert_array_equal(lay["node_slot"][:, 0], np.arange(50))


def test_layout_rejects_bad_ids():
    idx = np.array([[0, 8]], np.int32)
    with pytest.raises(ValueError):
        oracle.layout(idx, 8, 4, 2)
    with pytest.raises(ValueError):
        oracle.layout(np.array([[-1, 2]], np.int32), 8, 4, 2)


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    lg = np.array([[float(v) for v in row] for row in g["logits"]],
                  dtype=np.float32)
    assert np.signbit(lg[2, 0])
    idx, w = oracle.gate(lg, g["K"])
    np.testing.assert_array_equal(idx, g["topk_idx"])
    np.testing.assert_allclose(w, np.array(g["topk_w"]), rtol=2.0 ** -24)
    lay = oracle.layout(idx, g["E"], g["R"], g["N"])
    for key in ("expert_count", "expert_off", "rank_count", "rank_off",
                "rank_token_count", "node_count", "node_off", "node_slot",
                "slot_pos", "row_src"):
        np.testing.assert_array_equal(lay[key], np.array(g[key]), err_msg=key)
    np.testing.assert_array_equal(lay["node_mask"],
                                  np.array(g["node_mask"], np.uint64))


# ---------------------------------------------------------------- pack ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_pack_pins(w):
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack(d["x"], lay["slot_pos"])
    x = d["x"]
    np.testing.assert_array_equal(send, x[lay["row_src"] // w.K])
    for k in range(w.K):
        np.testing.assert_array_equal(send[lay["slot_pos"][:, k]], x)
    # multiset of rows: K copies of every x row
    a = np.sort(send.view(np.uint8).reshape(len(send), -1), axis=0)
    b = np.sort(np.repeat(x, w.K, axis=0).view(np.uint8).reshape(len(send), -1),
                axis=0)
    np.testing.assert_array_equal(a, b)


def test_pack_rejects_out_of_range_slot():
    x = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.pack(x, np.array([[0, 4], [1, 2]], np.int32))


# ------------------------------------------------------------- combine ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_combine_identity_experts_return_input(w):
    d = mi.make_inputs(w)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack(d["x"], lay["slot_pos"])
    out, exact = oracle.combine(send, lay["slot_pos"], wt, out_dtype=w.out_dtype)
    xf = d["x"] if w.x_dtype == mi.F32 else mi.bf16_bits_to_f32(d["x"])
    xf = xf.astype(np.float64)
    # closed form: sum_k w_k * x = x * sum_k w_k, with |sum w - 1| <= K 2^-24
    sw = wt.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(exact, xf * sw, rtol=1e-15, atol=0)
    assert np.all(np.abs(exact - xf) <= w.K * 2.0 ** -24 * np.abs(xf) + 1e-300)
    if w.out_dtype == mi.F32:
        np.testing.assert_allclose(out, xf, rtol=w.K * 2.0 ** -23, atol=0)
    else:
        # bf16 out equals x except where x*sum(w) crosses a rounding boundary
        frac = np.mean(out == d["x"])
        assert frac > 0.999


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_combine_diagonal_experts_closed_form(w):
    d = mi.make_inputs(w)
    s = d["expert_scale"]
    if s is None:
        s = (1.0 + 0.01 * np.arange(w.E)).astype(np.float32)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack(d["x"], lay["slot_pos"])
    _, exact = oracle.combine(send, lay["slot_pos"], wt, idx, s)
    xf = d["x"] if w.x_dtype == mi.F32 else mi.bf16_bits_to_f32(d["x"])
    scal = (wt.astype(np.float64) * s[idx].astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(exact, xf.astype(np.float64) * scal[:, None],
                               rtol=1e-14, atol=0)


@pytest.mark.parametrize("w", SHAPES[:3], ids=lambda w: w.name)
def test_combine_one_hot_weights_invert_pack(w):
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack(d["x"], lay["slot_pos"])
    for k in range(w.K):
        oh = np.zeros((w.T, w.K), np.float32)
        oh[:, k] = 1.0
        out, _ = oracle.combine(send, lay["slot_pos"], oh,
                                out_dtype=w.x_dtype)
        np.testing.assert_array_equal(out, d["x"])


def test_combine_general_rows_as_matrix_product():
    # arbitrary Y (not a packed x): out = M @ Y with M[t, slot] = w * s
    rng = np.random.Generator(np.random.PCG64(11))
    T, K, E, H = 24, 3, 8, 40
    idx = mi.random_topk_idx(T, E, K, seed=5)
    lay = oracle.layout(idx, E, 4, 2)
    wt = rng.random((T, K)).astype(np.float32)
    s = rng.random(E).astype(np.float32) + 0.5
    for dt in (mi.F32, mi.BF16):
        y = mi.random_x(T * K, H, dt, seed=9)
        yf = y if dt == mi.F32 else mi.bf16_bits_to_f32(y)
        M = np.zeros((T, T * K))
        for t in range(T):
            for k in range(K):
                M[t, lay["slot_pos"][t, k]] += float(wt[t, k]) * float(s[idx[t, k]])
        out, exact = oracle.combine(y, lay["slot_pos"], wt, idx, s,
                                    out_dtype=dt)
        np.testing.assert_allclose(exact, M @ yf.astype(np.float64),
                                   rtol=1e-13, atol=1e-13)
        if dt == mi.F32:
            np.testing.assert_array_equal(out, exact.astype(np.float32))
        else:
            np.testing.assert_array_equal(out, oracle.f64_to_bf16(exact).reshape(T, H))
        rows = np.array([3, 0, 17], np.int32)
        part = oracle.combine_tokens(rows, y, lay["slot_pos"], wt, idx, s)
        np.testing.assert_array_equal(part, exact[rows])


def test_bf16_rounding_known_values():
    cases = [
        (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0 ** -8, 0x3F80),             # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),         # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie
        (2.0 ** -133, 0x0001),                 # smallest subnormal
        (2.0 ** -134, 0x0000),                 # tie with zero -> even
        (3 * 2.0 ** -134, 0x0002),             # tie between 1 and 2 quanta
        (2.0 ** -126, 0x0080),                 # smallest normal
        (3.0e38, 0x7F62),                      # 1.7632 * 2^127 -> 98/128
        (3.4e38, 0x7F80),                      # past the last half-step
        (-65504.0, 0xC780),
    ]
    got = oracle.f64_to_bf16([v for v, _ in cases])
    np.testing.assert_array_equal(got, np.array([b for _, b in cases], np.uint16))


def test_bf16_rounding_matches_fp32_bit_rounding():
    # for fp32-representable inputs a single rounding equals the bit trick
    rng = np.random.Generator(np.random.PCG64(3))
    v = (rng.standard_normal(4000) * np.exp2(rng.integers(-20, 20, 4000))
         ).astype(np.float32)
    np.testing.assert_array_equal(oracle.f64_to_bf16(v.astype(np.float64)),
                                  mi.f32_to_bf16_bits(v))


def test_dispatch_combine_tiny_returns_input():
    w = mi.TINY
    d = mi.make_inputs(w)
    res = oracle.dispatch_combine(d["x"], d["logits"], w.K, w.R, w.N,
                                  None, out_dtype="f32")
    np.testing.assert_allclose(res["out"], d["x"], rtol=w.K * 2.0 ** -23,
                               atol=0)
