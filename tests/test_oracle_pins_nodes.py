"""Pins for the two-leg (node-level) dispatch and the per-node partial combine
of the CPU oracle.

"Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
Training", Section 1: a token crosses to a node once however many of its
experts live there, and is forwarded inside the node.  "MoX: Efficient MoE
Routing on Direct-Connect Topologies", Section 2.5: on the way back a node
reduces the outputs it holds for a token before forwarding one vector.

The pins tie these functions to things other than themselves: the one-leg
pack and flat combine (pinned in test_oracle_pins.py by argsort and a matrix
product), numpy's nonzero/repeat on the node masks, closed forms for diagonal
and one-expert-per-node layouts, and the bf16 rounding pinned at known values.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle

SHAPES = [mi.TINY, mi.MIXTRAL.replace(T=256, H=64),
          mi.QWEN3.replace(T=256, H=64), mi.DEEPSEEK_V3.replace(T=256, H=64),
          mi.KIMI.replace(T=128, H=64)]


def _route(w, seed=0):
    d = mi.make_inputs(w, seed=seed)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    return d, idx, wt, lay


def _popcount(mask):
    m = np.asarray(mask, dtype=np.uint64)
    return np.array([bin(int(v)).count("1") for v in m], dtype=np.int64)


def _xf64(w, x):
    xf = x if w.x_dtype == mi.F32 else mi.bf16_bits_to_f32(x)
    return xf.astype(np.float64)


# -------------------------------------------------------------- leg 1 ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_pack_nodes_segments_are_masked_tokens(w):
    d, idx, _, lay = _route(w)
    ns = oracle.pack_nodes(d["x"], lay["node_slot"])
    mask = lay["node_mask"]
    # one row per (token, node) crossing: D = sum node_count = sum popcount
    assert len(ns) == lay["node_count"].sum() == _popcount(mask).sum()
    # node n's segment holds, in token order, exactly the tokens whose mask
    # has bit n (numpy's nonzero on the mask bits, not the slot table)
    for n in range(w.N):
        toks = np.nonzero((mask >> np.uint64(n)) & np.uint64(1))[0]
        seg = ns[lay["node_off"][n]:lay["node_off"][n + 1]]
        np.testing.assert_array_equal(seg, d["x"][toks])


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_pack_nodes_multiset(w):
    d, _, _, lay = _route(w)
    ns = oracle.pack_nodes(d["x"], lay["node_slot"])
    rep = np.repeat(d["x"], _popcount(lay["node_mask"]), axis=0)
    a = np.sort(ns.view(np.uint8).reshape(len(ns), -1), axis=0)
    b = np.sort(rep.view(np.uint8).reshape(len(rep), -1), axis=0)
    np.testing.assert_array_equal(a, b)


def test_pack_nodes_dedup_bound():
    # the crossings of a token never exceed min(K, N), and a token always
    # crosses to at least ceil(K / (E/N)) nodes (a token's K experts span
    # at least that many nodes of E/N experts each)
    for w in SHAPES:
        _, _, _, lay = _route(w)
        pc = _popcount(lay["node_mask"])
        assert pc.max() <= min(w.K, w.N)
        assert pc.min() >= -(-w.K // (w.E // w.N))


# -------------------------------------------------------------- leg 2 ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("seed", [0, 1])
def test_forward_equals_one_leg_pack(w, seed):
    d, idx, _, lay = _route(w, seed)
    ns = oracle.pack_nodes(d["x"], lay["node_slot"])
    send2 = oracle.forward(ns, lay["node_slot"], idx, lay["slot_pos"], w.E,
                           w.R)
    np.testing.assert_array_equal(send2, oracle.pack(d["x"], lay["slot_pos"]))


def test_forward_random_ids():
    # random distinct experts (no gate) on an uneven placement
    T, E, K, R, N = 64, 24, 5, 6, 3
    idx = mi.random_topk_idx(T, E, K, seed=9)
    lay = oracle.layout(idx, E, R, N)
    x = np.random.Generator(np.random.PCG64(2)).standard_normal(
        (T, 16)).astype(np.float32)
    ns = oracle.pack_nodes(x, lay["node_slot"])
    send2 = oracle.forward(ns, lay["node_slot"], idx, lay["slot_pos"], E, R)
    np.testing.assert_array_equal(send2, oracle.pack(x, lay["slot_pos"]))


# ------------------------------------------------- per-node partials ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_partials_sum_to_flat_combine(w):
    d, idx, wt, lay = _route(w)
    send = oracle.pack(d["x"], lay["slot_pos"])
    s = d["expert_scale"]
    _, pex = oracle.combine_partial(send, lay["slot_pos"], wt, idx, s,
                                    lay["node_slot"], w.E, w.R, "f32")
    _, flat = oracle.combine(send, lay["slot_pos"], wt, idx, s, "f32")
    # selection matrix M[t, p] = 1 when row p of the partials belongs to t
    M = np.zeros((w.T, len(pex)))
    t_of, n_of = np.nonzero(lay["node_slot"] >= 0)
    M[t_of, lay["node_slot"][t_of, n_of]] = 1.0
    np.testing.assert_allclose(M @ pex, flat, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_partials_diagonal_experts_closed_form(w):
    # y = s_e x: node n's partial of token t is x[t] * sum_{k on n} w s
    d, idx, wt, lay = _route(w)
    s = d["expert_scale"]
    if s is None:
        s = (1.0 + 0.01 * np.arange(w.E)).astype(np.float32)
    send = oracle.pack(d["x"], lay["slot_pos"])
    _, pex = oracle.combine_partial(send, lay["slot_pos"], wt, idx, s,
                                    lay["node_slot"], w.E, w.R, "f32")
    node_of = (idx // (w.E // w.R)) // (w.R // w.N)
    coef = np.zeros((w.T, w.N))
    np.add.at(coef, (np.repeat(np.arange(w.T), w.K), node_of.ravel()),
              (wt.astype(np.float64) * s[idx].astype(np.float64)).ravel())
    xf = _xf64(w, d["x"])
    t_of, n_of = np.nonzero(lay["node_slot"] >= 0)
    want = xf[t_of] * coef[t_of, n_of][:, None]
    np.testing.assert_allclose(pex[lay["node_slot"][t_of, n_of]], want,
                               rtol=1e-14, atol=0)


def test_partials_single_node_equal_flat_combine():
    # N = 1: the one partial of a token is the flat combine, term for term
    w = mi.MIXTRAL.replace(T=128, H=32)
    d, idx, wt, lay = _route(w)
    send = oracle.pack(d["x"], lay["slot_pos"])
    _, pex = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                    d["expert_scale"], lay["node_slot"],
                                    w.E, w.R, "f32")
    _, flat = oracle.combine(send, lay["slot_pos"], wt, idx,
                             d["expert_scale"], "f32")
    np.testing.assert_array_equal(lay["node_slot"][:, 0], np.arange(w.T))
    np.testing.assert_array_equal(pex, flat)


def test_partials_one_expert_per_node_are_single_terms():
    # E = R = N: every node holds one expert, so a partial is one term
    T, E, K, H = 48, 8, 3, 24
    rng = np.random.Generator(np.random.PCG64(4))
    idx = mi.random_topk_idx(T, E, K, seed=4)
    wt = rng.random((T, K)).astype(np.float32)
    s = (1.0 + 0.125 * np.arange(E)).astype(np.float32)
    lay = oracle.layout(idx, E, E, E)
    y = rng.standard_normal((T * K, H)).astype(np.float32)
    _, pex = oracle.combine_partial(y, lay["slot_pos"], wt, idx, s,
                                    lay["node_slot"], E, E, "f32")
    for k in range(K):
        p = lay["node_slot"][np.arange(T), idx[:, k]]
        want = (wt[:, k].astype(np.float64) * s[idx[:, k]])[:, None] * \
            y[lay["slot_pos"][:, k]].astype(np.float64)
        np.testing.assert_array_equal(pex[p], want)


@pytest.mark.parametrize("pdt", ["bf16", "f32"])
def test_partial_rounding(pdt):
    w = mi.DEEPSEEK_V3.replace(T=64, H=32)
    d, idx, wt, lay = _route(w)
    send = oracle.pack(d["x"], lay["slot_pos"])
    part, pex = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                       d["expert_scale"], lay["node_slot"],
                                       w.E, w.R, pdt)
    if pdt == "f32":
        np.testing.assert_array_equal(part, pex.astype(np.float32))
    else:
        np.testing.assert_array_equal(
            part, oracle.f64_to_bf16(pex).reshape(part.shape))


# ------------------------------------------- fp32 partials as stored ----
# The fp32 value a stored partial is rounded from: c = fp32(w * s), then
# acc <- fma(c, y, acc) from +0 over the node's slots in ascending k, each
# step rounded once to fp32.  Pinned by exact rational arithmetic with a
# brute-force nearest-fp32 rounding, by a case where the slot order decides
# the result, and by the fp32 error bound around the fp64 partial.

def _round_f32(q):
    """Nearest fp32 to the rational q, ties to the even significand, found
    by comparing the exact distances of three neighbouring candidates."""
    from fractions import Fraction
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c,
             np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - q),
                                     int(np.array(v).view(np.uint32)) & 1))


@pytest.mark.parametrize("ydt", [mi.F32, mi.BF16])
def test_partial_f32_chain_exact_fractions(ydt):
    from fractions import Fraction
    w = mi.Workload("chain", T=7, H=3, E=8, K=5, R=4, N=2, x_dtype=ydt,
                    out_dtype=mi.F32, expert="mod8")
    d, idx, wt, lay = _route(w)
    rng = np.random.Generator(np.random.PCG64(21))
    y = mi.random_x(w.T * w.K, w.H, ydt, seed=21)
    yv = mi.bf16_bits_to_f32(y) if ydt == mi.BF16 else y
    s = d["expert_scale"]
    wt = (wt * np.float32(3.0) * rng.random(wt.shape, dtype=np.float32))
    part, f32 = oracle.combine_partial(y, lay["slot_pos"], wt, idx, s,
                                       lay["node_slot"], w.E, w.R, "bf16",
                                       accumulate="f32")
    per_node = (w.E // w.R) * (w.R // w.N)
    for t in range(w.T):
        for n in range(w.N):
            p = lay["node_slot"][t, n]
            if p < 0:
                continue
            for h in range(w.H):
                acc = np.float32(0.0)
                for k in range(w.K):
                    e = idx[t, k]
                    if e // per_node != n:
                        continue
                    c = _round_f32(Fraction(float(wt[t, k])) *
                                   Fraction(float(s[e])))
                    v = Fraction(float(yv[lay["slot_pos"][t, k], h]))
                    acc = _round_f32(Fraction(float(c)) * v +
                                     Fraction(float(acc)))
                assert f32[p, h] == acc, (t, n, h)
    # the stored bf16 partial is that fp32 value rounded once
    np.testing.assert_array_equal(part,
                                  oracle.f64_to_bf16(f32).reshape(part.shape))


def test_partial_f32_chain_takes_slots_in_ascending_order():
    # one token, three slots on node 0 with rows 1, 2^27, -2^27 (weights 1):
    # ascending k gives fma chain 1 -> 2^27 (2^27 + 1 rounds down) -> 0,
    # while the fp64 partial is 1 and descending order would give 1
    y = np.zeros((3, 8), np.float32)
    y[0], y[1], y[2] = 1.0, 2.0 ** 27, -(2.0 ** 27)
    idx = np.array([[0, 1, 2]], np.int32)
    sp = np.array([[0, 1, 2]], np.int32)
    wt = np.ones((1, 3), np.float32)
    ns = np.array([[0, -1]], np.int32)
    # E = 6 experts on R = 2 ranks, N = 2 nodes: experts 0-2 on node 0
    _, f32 = oracle.combine_partial(y, sp, wt, idx, None, ns, 6, 2, "f32",
                                    accumulate="f32")
    _, f64 = oracle.combine_partial(y, sp, wt, idx, None, ns, 6, 2, "f32")
    assert np.all(f32 == 0.0) and np.all(f64 == 1.0)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_partial_f32_chain_within_fp32_error(w):
    d, idx, wt, lay = _route(w)
    send = oracle.pack(d["x"], lay["slot_pos"])
    _, f32 = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                    d["expert_scale"], lay["node_slot"], w.E,
                                    w.R, "f32", accumulate="f32")
    _, f64 = oracle.combine_partial(send, lay["slot_pos"], wt, idx,
                                    d["expert_scale"], lay["node_slot"], w.E,
                                    w.R, "f32")
    ab = (send & np.uint16(0x7FFF)) if send.dtype == np.uint16 else np.abs(send)
    _, sc = oracle.combine_partial(ab, lay["slot_pos"], wt, idx,
                                   d["expert_scale"], lay["node_slot"], w.E,
                                   w.R, "f32")
    # K fma roundings and one coefficient rounding, each within 2^-24 of
    # the running magnitude, which is at most sum |terms|
    bound = (w.K + 1) * 2.0 ** -24 * sc
    assert np.all(np.abs(f32 - f64) <= bound + 1e-300)
    assert np.any(f32 != f64)  # not the fp64 sum in disguise


# --------------------------------------------------------- sum of nodes ----

@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_combine_nodes_is_selection_product(w):
    d, idx, wt, lay = _route(w)
    rng = np.random.Generator(np.random.PCG64(6))
    D = oracle.node_rows(lay["node_slot"])
    part = rng.standard_normal((D, 16)).astype(np.float32)
    _, ex = oracle.combine_nodes(part, lay["node_slot"], "f32")
    M = np.zeros((w.T, D))
    t_of, n_of = np.nonzero(lay["node_slot"] >= 0)
    M[t_of, lay["node_slot"][t_of, n_of]] = 1.0
    np.testing.assert_allclose(ex, M @ part.astype(np.float64), rtol=1e-14,
                               atol=1e-300)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_two_leg_identity_experts_return_input(w):
    d = mi.make_inputs(w)
    r = oracle.dispatch_combine_nodes(d["x"], d["logits"], w.K, w.R, w.N,
                                      None, "f32", "f32")
    xf = _xf64(w, d["x"])
    sw = r["topk_w"].astype(np.float64).sum(axis=1, keepdims=True)
    # fp32 partials: one fp32 rounding per partial on top of x * sum(w)
    bound = (w.K * 2.0 ** -24 + w.N * 2.0 ** -24) * np.abs(xf)
    assert np.all(np.abs(r["out_exact"] - xf * sw) <= bound + 1e-300)
    np.testing.assert_array_equal(r["send"], oracle.pack(
        d["x"], r["slot_pos"]))
