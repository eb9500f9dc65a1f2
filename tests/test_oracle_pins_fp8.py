"""Pins for the FP8 (E4M3, per-block scale) dispatch of the CPU oracle.

"Efficient and portable mixture-of-experts communication", "Envío
(Dispatch)": tokens travel with block scale factors; the format and block
size are readings (OCP E4M3, B = 128, s = amax/448, codes of x * (448/amax)).

Pins that do not reuse the oracle's arithmetic: code values worked out by
hand from the format's fields, the structure of the 256-entry value table,
an encoder by brute-force nearest search over that table (ties to the even
code), numpy float32 arithmetic for the scales and scaled values, the
dequantisation error bound, and a matrix product for the combine.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle

TABLE = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def brute_code(v: float) -> int:
    """Nearest finite E4M3 code to v by search (magnitude clamped to 448);
    on a tie the code with the even mantissa wins; the sign of v is kept."""
    a = min(abs(v), 448.0)
    pos = np.arange(0x7F, dtype=np.int64)  # non-negative codes 0x00..0x7E
    d = np.abs(TABLE[pos] - a)
    best = pos[d == d.min()]
    c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return c | (0x80 if np.signbit(v) else 0)


# ------------------------------------------------------------ codec ----

def test_code_values_from_the_format_fields():
    # value = (1 + m/8) 2^(e-7) for e >= 1, (m/8) 2^-6 for e = 0
    cases = {
        448.0: 0x7E,            # e=15, m=6: 1.75 * 2^8 (e=15, m=7 is NaN)
        1.0: 0x38,              # e=7, m=0
        0.5: 0x30,              # e=6
        -2.0: 0xC0,             # sign, e=8
        2.0 ** -6: 0x08,        # smallest normal
        2.0 ** -9: 0x01,        # smallest subnormal
        7 * 2.0 ** -9: 0x07,    # largest subnormal
        1.0 + 1 / 16: 0x38,     # tie between 1 and 1.125: even mantissa
        1.0 + 3 / 16: 0x3A,     # tie between 1.125 and 1.25: even mantissa
        2.0 ** -10: 0x00,       # tie between 0 and 2^-9: even (zero)
        3 * 2.0 ** -10: 0x02,   # tie between 2^-9 and 2^-8: even
        464.0: 0x7E,            # saturates (no code above 448)
        1e6: 0x7E,
        -0.0: 0x80,             # sign of zero kept
        -1e-30: 0x80,
    }
    got = oracle.e4m3_code(list(cases))
    np.testing.assert_array_equal(got, np.array(list(cases.values()),
                                                np.uint8))


def test_value_table_structure():
    pos = TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # strictly increasing
    np.testing.assert_array_equal(TABLE[0x80:0xFF], -pos)
    assert np.isnan(TABLE[0x7F]) and np.isnan(TABLE[0xFF])
    assert pos[0] == 0.0 and pos[1] == 2.0 ** -9 and pos[-1] == 448.0
    # subnormals are evenly spaced by 2^-9; each binade holds 8 codes whose
    # spacing is 1/8 of the binade's lower end
    np.testing.assert_array_equal(np.diff(pos[:9]), np.full(8, 2.0 ** -9))
    for e in range(1, 16):
        lo = pos[8 * e]
        assert lo == 2.0 ** (e - 7)
        np.testing.assert_array_equal(
            np.diff(pos[8 * e:8 * e + 8 - (e == 15)]), lo / 8)


def test_encoder_equals_brute_force_nearest():
    rng = np.random.Generator(np.random.PCG64(3))
    mags = 2.0 ** rng.uniform(-12, 9.5, 4000)
    vals = list(mags * rng.choice([-1.0, 1.0], len(mags)))
    # every exact midpoint between neighbouring codes is a tie
    pos = TABLE[:0x7F]
    vals += list((pos[1:] + pos[:-1]) / 2) + list(-(pos[1:] + pos[:-1]) / 2)
    vals += list(pos) + [0.0, 449.0, 463.99, 464.0, 1e9]
    got = oracle.e4m3_code(vals)
    want = np.array([brute_code(v) for v in vals], np.uint8)
    np.testing.assert_array_equal(got, want)


def test_round_trip_of_every_finite_code():
    back = oracle.e4m3_code(TABLE[FINITE])
    np.testing.assert_array_equal(back, FINITE)


# ---------------------------------------------------- quantised rows ----

def _numpy_quant(x_f32: np.ndarray, B: int):
    """Independent statement of the reading with numpy float32 arithmetic
    and the brute-force encoder."""
    T, H = x_f32.shape
    codes = np.zeros((T, H), np.uint8)
    scales = np.zeros((T, H // B), np.float32)
    for t in range(T):
        for b in range(H // B):
            blk = x_f32[t, b * B:(b + 1) * B]
            amax = np.max(np.abs(blk))
            scales[t, b] = np.float32(amax) / np.float32(448.0)
            if amax == 0:
                codes[t, b * B:(b + 1) * B] = np.where(np.signbit(blk), 0x80, 0)
                continue
            r = np.float32(448.0) / np.float32(amax)
            p = (blk * r).astype(np.float32)
            codes[t, b * B:(b + 1) * B] = [brute_code(float(v)) for v in p]
    return codes, scales


@pytest.mark.parametrize("xdt,B", [(mi.BF16, 128), (mi.F32, 32), (mi.BF16, 64)])
def test_pack_fp8_equals_independent_quantisation(xdt, B):
    w = mi.DEEPSEEK_V3.replace(T=24, H=256, x_dtype=xdt)
    d = mi.make_inputs(w)
    x = d["x"]
    x[3, :B] = 0                                 # an all-zero block
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(x, lay["slot_pos"], B)
    rb = -(-(w.H + 4 * w.H // B) // 128) * 128   # rows on 128-byte blocks
    assert send.shape == (w.T * w.K, rb)
    assert not send[:, w.H + 4 * w.H // B:].any()  # zero padding
    codes, scales = oracle.fp8_rows_split(send, w.H, B)
    xf = x if xdt == mi.F32 else mi.bf16_bits_to_f32(x)
    want_c, want_s = _numpy_quant(xf.astype(np.float32), B)
    tok = lay["row_src"] // w.K
    np.testing.assert_array_equal(codes, want_c[tok])
    np.testing.assert_array_equal(scales, want_s[tok])


@pytest.mark.parametrize("w", [mi.DEEPSEEK_V3.replace(T=64, H=512),
                               mi.KIMI.replace(T=32, H=256),
                               mi.MIXTRAL.replace(T=64, H=384)],
                         ids=lambda w: w.name)
def test_dequantisation_error_bound(w):
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], 128)
    codes, scales = oracle.fp8_rows_split(send, w.H, 128)
    deq = TABLE[codes] * np.repeat(scales.astype(np.float64), 128, axis=1)
    x = mi.bf16_bits_to_f32(d["x"]).astype(np.float64)[lay["row_src"] // w.K]
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    # half an E4M3 step: 2^-4 of the value (normals), 2^-10 * s (subnormals),
    # plus the fp32 roundings of r and x*r
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s) * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - x) <= bound + 1e-30)
    # the largest magnitude of every block is coded as +-448
    amax_code = np.max(codes & 0x7F, axis=None)
    assert amax_code == 0x7E
    blocks = (codes & 0x7F).reshape(len(codes), -1, 128).max(axis=2)
    assert np.all((blocks == 0x7E) | (scales == 0))


def test_pack_fp8_writes_k_identical_copies():
    w = mi.QWEN3.replace(T=40, H=256)
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], 128)
    for k in range(1, w.K):
        np.testing.assert_array_equal(send[lay["slot_pos"][:, k]],
                                      send[lay["slot_pos"][:, 0]])


# ------------------------------------------------------------ combine ----

@pytest.mark.parametrize("w", [mi.DEEPSEEK_V3.replace(T=48, H=256),
                               mi.KIMI.replace(T=24, H=256),
                               mi.MIXTRAL.replace(T=48, H=128)],
                         ids=lambda w: w.name)
def test_combine_fp8_is_matrix_product_of_dequantised_rows(w):
    d = mi.make_inputs(w)
    idx, wt = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], 128)
    codes, scales = oracle.fp8_rows_split(send, w.H, 128)
    Y = TABLE[codes] * np.repeat(scales.astype(np.float64), 128, axis=1)
    s = d["expert_scale"]
    _, exact = oracle.combine_fp8(send, lay["slot_pos"], wt, w.H, 128, idx, s)
    M = np.zeros((w.T, w.T * w.K))
    c = wt.astype(np.float64) * s[idx].astype(np.float64)
    for k in range(w.K):
        M[np.arange(w.T), lay["slot_pos"][:, k]] = c[:, k]
    np.testing.assert_allclose(exact, M @ Y, rtol=1e-13, atol=1e-300)


def test_combine_fp8_one_hot_returns_dequantised_row():
    w = mi.DEEPSEEK_V3.replace(T=32, H=256)
    d = mi.make_inputs(w)
    idx, _ = oracle.gate(d["logits"], w.K)
    lay = oracle.layout(idx, w.E, w.R, w.N)
    send = oracle.pack_fp8(d["x"], lay["slot_pos"], 128)
    codes, scales = oracle.fp8_rows_split(send, w.H, 128)
    deq = TABLE[codes] * np.repeat(scales.astype(np.float64), 128, axis=1)
    for k in (0, w.K - 1):
        oh = np.zeros((w.T, w.K), np.float32)
        oh[:, k] = 1.0
        _, ex = oracle.combine_fp8(send, lay["slot_pos"], oh, w.H, 128)
        np.testing.assert_array_equal(ex, deq[lay["slot_pos"][:, k]])


def _product_vs_quotient_cases(n_want=6):
    """(amax, x) pairs where the code of fp32(x * (448/amax)) differs from the
    code of fp32(x / (amax/448)): values next to an E4M3 tie."""
    rng = np.random.Generator(np.random.PCG64(21))
    pos = TABLE[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2)[8:]     # ties between normal codes
    found = []
    for _ in range(20000):
        amax = np.float32(rng.uniform(1.0, 4.0))
        r = np.float32(448.0) / amax
        s = amax / np.float32(448.0)
        m = rng.choice(mids)
        x0 = np.float32(m / float(r))
        for x in (x0, np.nextafter(x0, np.float32(0)),
                  np.nextafter(x0, np.float32(1e9))):
            if not 0 < x < amax:
                continue
            p1, p2 = np.float32(x * r), np.float32(x / s)
            if brute_code(float(p1)) != brute_code(float(p2)):
                found.append((amax, x))
                break
        if len(found) >= n_want:
            break
    return found


def test_codes_come_from_the_product_with_448_over_amax():
    cases = _product_vs_quotient_cases()
    assert len(cases) >= 3, "no distinguishing case found"
    B, H = 32, 32 * len(cases)
    x = np.zeros((1, H), np.float32)
    for j, (amax, v) in enumerate(cases):
        x[0, j * B] = amax
        x[0, j * B + 1] = v
    send = oracle.pack_fp8(x, np.zeros((1, 1), np.int32), B)
    codes, _ = oracle.fp8_rows_split(send, H, B)
    for j, (amax, v) in enumerate(cases):
        r = np.float32(448.0) / amax
        assert codes[0, j * B + 1] == brute_code(float(np.float32(v * r)))
