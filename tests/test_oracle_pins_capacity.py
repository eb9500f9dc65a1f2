"""Pins for the capacity-padded and bucketed layout of the CPU oracle.

"Workload-Static Optical Circuit Switching for Scalable LLM Inference
Decode", "Variable MoE Traffic and Regularization": fixed capacity per
expert, buffers padded to it, overflow dropped; bucketing rounds counts up to
one of q levels.  Pinned against numpy (bincount, nonzero order, searchsorted,
a matrix product), the dropless layout (itself pinned by argsort) as the
closed form when nothing is dropped, and hand-built cases.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle

SHAPES = [mi.TINY, mi.MIXTRAL.replace(T=512, H=64),
          mi.QWEN3.replace(T=512, H=64), mi.DEEPSEEK_V3.replace(T=512, H=64),
          mi.KIMI.replace(T=256, H=64)]


def _idx(w, seed=0):
    d = mi.make_inputs(w, seed=seed)
    idx, wt = oracle.gate(d["logits"], w.K)
    return d, idx, wt


def _check_capacity(idx, E, levels, lay):
    T, K = idx.shape
    levels = np.asarray(levels)
    cmax = int(levels[-1])
    count = np.bincount(idx.ravel(), minlength=E)
    np.testing.assert_array_equal(lay["expert_count"], count)
    kept = np.minimum(count, cmax)
    np.testing.assert_array_equal(
        lay["expert_cap"], levels[np.searchsorted(levels, kept)])
    np.testing.assert_array_equal(
        lay["expert_off"], np.concatenate([[0], np.cumsum(lay["expert_cap"])]))
    assert lay["dropped"] == int((count - kept).sum())
    flat = idx.ravel()
    sp = lay["slot_pos"].ravel()
    for e in range(E):
        pos = np.nonzero(flat == e)[0]          # expert e's slots, (t,k) order
        want = np.full(len(pos), -1)
        want[:kept[e]] = lay["expert_off"][e] + np.arange(kept[e])
        np.testing.assert_array_equal(sp[pos], want)
    used = sp[sp >= 0]
    assert len(np.unique(used)) == len(used)    # no row used twice
    rs = lay["row_src"]
    assert len(rs) == E * cmax
    np.testing.assert_array_equal(rs[used], np.nonzero(sp >= 0)[0])
    mask = np.ones(len(rs), bool)
    mask[used] = False
    assert np.all(rs[mask] == -1)


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("gamma", [0.5, 1.0, 1.25, 4.0])
def test_capacity_layout_pins(w, gamma):
    _, idx, _ = _idx(w)
    C = oracle.capacity(w.T, w.K, w.E, gamma)
    lay = oracle.layout_capacity(idx, w.E, [C])
    _check_capacity(idx, w.E, [C], lay)
    assert np.all(lay["expert_cap"] == C)       # q = 1: every segment C rows


@pytest.mark.parametrize("w", SHAPES[1:], ids=lambda w: w.name)
def test_bucketed_layout_pins(w):
    _, idx, _ = _idx(w, seed=1)
    mean = w.T * w.K / w.E
    levels = sorted({max(1, int(mean * f)) for f in (0.5, 1.0, 1.5, 2.0)})
    lay = oracle.layout_capacity(idx, w.E, levels)
    _check_capacity(idx, w.E, levels, lay)


def test_capacity_without_drops_is_the_dropless_layout_padded():
    # C >= max count: nothing dropped; slot = e*C + (dropless slot - offset)
    w = mi.DEEPSEEK_V3.replace(T=300, H=64)
    _, idx, _ = _idx(w)
    dl = oracle.layout(idx, w.E, w.R, w.N)
    C = int(dl["expert_count"].max())
    lay = oracle.layout_capacity(idx, w.E, [C])
    assert lay["dropped"] == 0
    e = idx
    want = e * C + (dl["slot_pos"] - dl["expert_off"][e])
    np.testing.assert_array_equal(lay["slot_pos"], want)


def test_capacity_hand_example():
    # 4 tokens, K=2, E=3, C=2: expert 0 is chosen by tokens 0,1,2 -> token 2
    # is dropped for expert 0; expert 2 by nobody (two padding rows)
    idx = np.array([[0, 1], [1, 0], [0, 1], [1, 2]], np.int32)
    lay = oracle.layout_capacity(idx, 3, [2])
    np.testing.assert_array_equal(lay["expert_count"], [3, 4, 1])
    np.testing.assert_array_equal(lay["expert_off"], [0, 2, 4, 6])
    np.testing.assert_array_equal(lay["slot_pos"],
                                  [[0, 2], [3, 1], [-1, -1], [-1, 4]])
    np.testing.assert_array_equal(lay["row_src"], [0, 3, 1, 2, 7, -1])
    assert lay["dropped"] == 3


def test_pack_capacity_rows_and_padding():
    w = mi.QWEN3.replace(T=200, H=32)
    d, idx, _ = _idx(w)
    C = oracle.capacity(w.T, w.K, w.E, 1.0)
    lay = oracle.layout_capacity(idx, w.E, [C])
    send = oracle.pack_capacity(d["x"], lay["row_src"], w.K)
    rs = lay["row_src"]
    np.testing.assert_array_equal(send[rs >= 0], d["x"][rs[rs >= 0] // w.K])
    assert not send[rs < 0].any()


@pytest.mark.parametrize("w", SHAPES[1:], ids=lambda w: w.name)
def test_combine_with_drops_is_matrix_product(w):
    d, idx, wt = _idx(w)
    C = oracle.capacity(w.T, w.K, w.E, 0.75)
    lay = oracle.layout_capacity(idx, w.E, [C])
    assert lay["dropped"] > 0
    send = oracle.pack_capacity(d["x"], lay["row_src"], w.K)
    s = d["expert_scale"]
    _, exact = oracle.combine(send, lay["slot_pos"], wt, idx, s, "f32")
    Y = mi.bf16_bits_to_f32(send).astype(np.float64)
    M = np.zeros((w.T, len(send)))
    c = wt.astype(np.float64) * s[idx].astype(np.float64)
    for k in range(w.K):
        keep = lay["slot_pos"][:, k] >= 0
        M[np.nonzero(keep)[0], lay["slot_pos"][keep, k]] = c[keep, k]
    np.testing.assert_allclose(exact, M @ Y, rtol=1e-13, atol=1e-300)


def test_capacity_rejects_bad_levels():
    idx = np.zeros((2, 1), np.int32)
    for bad in ([0], [3, 3], [4, 2]):
        with pytest.raises(ValueError):
            oracle.layout_capacity(idx, 2, bad)
