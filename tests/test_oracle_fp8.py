"""Pins of the FP8 (E4M3) cache oracle (CPU only).

The E4M3 codec is checked against what the OCP 8-bit floating point
specification fixes (bias 7, 3 mantissa bits, subnormals, largest finite 448,
S.1111.111 = NaN), against an exhaustive round trip of every finite code, and
against a brute-force nearest-value search with the even tie break (the MX
specification's conversion, saturating at 448).  Each planted mistake below
(bias 8, truncation, ties away from zero, no saturation, flushed subnormals)
must fail at least one pin.
"""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import fp8 as of
from oracle import mla as om

# values the specification fixes: (value, code)
SPEC = [(1.0, 0x38), (-2.0, 0xC0), (448.0, 0x7E), (-448.0, 0xFE), (2.0 ** -6, 0x08), (0.875 * 2.0 ** -6, 0x07),
        (2.0 ** -9, 0x01), (0.0, 0x00), (1.5, 0x3C), (240.0, 0x77), (256.0, 0x78), (0.1015625, 0x1D)]
# inputs with the code their rounding must give (ties to even, saturation, underflow)
ROUNDING = [(1.0625, 0x38),            # tie between 1 and 1.125: even mantissa (1.0)
            (1.1875, 0x3A),            # tie between 1.125 and 1.25: even mantissa (1.25)
            (-1.0625, 0xB8), (17.0, 0x58), (19.0, 0x5A), (464.0, 0x7E), (1.0e6, 0x7E), (-500.0, 0xFE),
            (2.0 ** -10, 0x00),        # tie between 0 and the smallest subnormal: 0
            (1.5 * 2.0 ** -10, 0x01), (1.5 * 2.0 ** -9, 0x02), (3.5e-3, 0x02), (0.3, 0x2A)]


def _finite_table():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return codes, of.e4m3_value(codes)


def _brute_encode(x):
    """Nearest finite E4M3 value by exhaustive search, ties to the code with an
    even mantissa, magnitudes above 448 saturated; the sign of zero follows x."""
    codes, vals = _finite_table()
    out = []
    for v in np.asarray(x, dtype=np.float64):
        a = min(abs(v), 448.0)
        pos = codes[(vals >= 0) & ~((codes == 0x80))]
        pv = of.e4m3_value(pos)
        d = np.abs(pv - a)
        best = np.flatnonzero(d == d.min())
        c = int(pos[best[0]]) if len(best) == 1 else int(next(pos[i] for i in best if pos[i] % 2 == 0))
        out.append(c | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def _pins(encode, value):
    """Names of the pins the codec (encode, value) fails."""
    bad = []
    for v, c in SPEC:
        if int(encode(np.array([v]))[0]) != c or value(np.array([c], np.uint8))[0] != v:
            bad.append(f"spec {v}")
    for v, c in ROUNDING:
        if int(encode(np.array([v]))[0]) != c:
            bad.append(f"rounding {v}")
    codes, vals = _finite_table()
    if not np.array_equal(encode(vals), codes):
        bad.append("round trip")
    if not np.isnan(value(np.array([0x7F, 0xFF], np.uint8))).all():
        bad.append("nan codes")
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(3000) * 4.0, rng.uniform(-1e-2, 1e-2, 1000),
                        rng.uniform(-600, 600, 500), (vals[:-1] + vals[1:]) / 2]).astype(np.float32)
    if not np.array_equal(encode(x), _brute_encode(x)):
        bad.append("brute force")
    return bad


def test_e4m3_codec_pins():
    assert _pins(of.e4m3_encode, of.e4m3_value) == []


def _mistaken_bias8_value(codes):
    return of.e4m3_value(codes) / 2.0


def _mistaken_bias8_encode(x):
    return of.e4m3_encode(np.asarray(x, np.float64) * 2.0)


def _mistaken_truncate(x):
    x = np.asarray(x, np.float64)
    c = of.e4m3_encode(x)
    v = of.e4m3_value(c)
    # step toward zero when rounding went away from zero
    away = np.abs(v) > np.abs(np.minimum(np.abs(x), 448.0))
    return np.where(away & ((c & 0x7F) > 0), c - 1, c).astype(np.uint8)


def _mistaken_ties_away(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    q = np.ldexp(1.0, (e - 3).astype(np.int64))
    v = np.minimum(np.floor(a / q + 0.5) * q, 448.0)
    return of.e4m3_encode(np.copysign(v, x))


def _mistaken_no_saturation(x):
    x = np.asarray(x, np.float64)
    c = of.e4m3_encode(x)
    return np.where(np.abs(x) >= 464.0, np.uint8(0x7F) | (c & 0x80), c).astype(np.uint8)


def _mistaken_flush_subnormals(x):
    x = np.asarray(x, np.float64)
    c = of.e4m3_encode(x)
    return np.where((c & 0x78) == 0, c & 0x80, c).astype(np.uint8)


@pytest.mark.parametrize("encode,value", [
    (_mistaken_bias8_encode, _mistaken_bias8_value),
    (_mistaken_truncate, of.e4m3_value),
    (_mistaken_ties_away, of.e4m3_value),
    (_mistaken_no_saturation, of.e4m3_value),
    (_mistaken_flush_subnormals, of.e4m3_value),
], ids=["bias8", "truncate", "ties_away", "no_saturation", "flush_subnormals"])
def test_e4m3_pins_catch_planted_mistakes(encode, value):
    assert _pins(encode, value), "a mistaken codec passed every pin"


def test_cache_quantize_multiplies_in_float32():
    # inv = fl32(1/3) = 0.3333333432674408; fl32(3 * inv) = 1.0 exactly -> code 0x38
    assert float(of.cache_inverse_scale(3.0)) == 0.3333333432674408
    assert int(of.cache_quantize_fp8(np.array([3.0]), 3.0)[0]) == 0x38
    # 2^-3 scale: exact scaling, the codes of 8 x
    x = np.array([0.125, -0.0078125, 56.0, 100.0], np.float32)
    assert of.cache_quantize_fp8(x, 0.125).tolist() == of.e4m3_encode(8.0 * x).tolist()
    # a product that rounds in float32 before the E4M3 rounding: 1.0625 * fl32(1/0.9999999)
    s = np.float32(0.99999994)
    y = np.float32(np.float32(1.0625) * (np.float32(1.0) / s))
    assert int(of.cache_quantize_fp8(np.array([1.0625]), float(s))[0]) == int(of.e4m3_encode(np.array([y]))[0])


def test_decode_over_representable_cache_is_the_bf16_decode():
    """Rows already on the E4M3 grid (times the scale) survive quantisation
    exactly, so the fp8 decode equals the absorbed decode of those rows."""
    sh = mi.WORKLOADS["tiny_fp32_t64"].replace(num_heads=3, kv_lora_rank=32, qk_rope_dim=16, qk_nope_dim=16,
                                               v_head_dim=16)
    rng = np.random.default_rng(3)
    H, r, dr, dn, dv = sh.num_heads, sh.kv_lora_rank, sh.qk_rope_dim, sh.qk_nope_dim, sh.v_head_dim
    bs, B = 4, 2
    scale = 0.0625
    codes = rng.integers(0, 256, size=(6, bs, r + dr)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30                          # no NaN codes
    cache = of.e4m3_value(codes) * scale
    table = np.array([[0, 2, 4], [5, 1, 3]], np.int32)
    lens = np.array([9, 11], np.int32)
    w = rng.standard_normal((H * (dn + dv), r)) * 0.1
    qn, qp = rng.standard_normal((B, H, dn)), rng.standard_normal((B, H, dr))
    q = of.cache_quantize_fp8(cache, scale)
    assert np.array_equal(q, codes)
    got = of.decode_absorbed_fp8(sh, w, qn, qp, q, scale, table, lens, bs)
    ref = om.decode_absorbed(sh, w, qn, qp, cache, table, lens, bs)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------- MXFP8
MX_VALUES = [  # (block contents, expected scale byte, expected codes of the first values)
    ([1.0, 0.5, -0.25], 119, [0x78, 0x70, 0xE8]),          # amax 1: X = 2^-8, 1 -> 256, 0.5 -> 128, -0.25 -> -64
    ([448.0, 1.0], 127, [0x7E, 0x38]),                     # amax 448: X = 1
    ([500.0, -3.0], 127, [0x7E, 0xC4]),                    # amax 500: X = 1, 500 saturates to 448
    ([3.0, 1.0], 120, [0x7C, 0x70]),                       # amax 3: X = 2^-7, 3 -> 384, 1 -> 128
    ([0.0, 0.0], 0, [0x00, 0x00]),                         # zero block: smallest scale
]


def _mx_pins(quantize, dequantize):
    bad = []
    for vals, sb, codes in MX_VALUES:
        x = np.zeros(32)
        x[: len(vals)] = vals
        c, s = quantize(x)
        if int(s[0]) != sb or [int(v) for v in c[: len(codes)]] != codes:
            bad.append(f"values {vals}")
    rng = np.random.default_rng(2)
    # blocks on the grid (top element in the top binade) survive exactly
    cds = rng.integers(0, 0x7E, size=(200, 32)).astype(np.uint8)
    cds[:, 0] = rng.integers(0x78, 0x7F, size=200)
    cds ^= rng.integers(0, 2, size=cds.shape).astype(np.uint8) << 7
    e = rng.integers(-20, 20, size=200)
    x = of.e4m3_value(cds) * np.ldexp(1.0, e)[:, None]
    c, s = quantize(x)
    if not (np.array_equal(c, cds) and np.array_equal(s.ravel().astype(int), e + 127)):
        bad.append("round trip")
    # power-of-two invariance and the half-ulp error bound on random blocks
    y = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-8, 8, size=(300, 1)))
    c1, s1 = quantize(y)
    c2, s2 = quantize(y * 2.0 ** 5)
    if not (np.array_equal(c1, c2) and np.array_equal(s2.astype(int), s1.astype(int) + 5)):
        bad.append("invariance")
    X = np.repeat(np.ldexp(1.0, s1.astype(int) - 127), 32, axis=-1)
    err = np.abs(dequantize(c1, s1) - y)
    # half an ulp (relative 2^-4, or 2^-10 X among the subnormals), plus what
    # saturation takes off the elements above 448 X (at most |y| < 512 X)
    sat = np.maximum(0.0, np.abs(y) - 448.0 * X)
    if not (np.all(err <= 2.0 ** -4 * np.abs(y) + 2.0 ** -10 * X * (1 + 1e-12) + sat)
            and np.all(np.abs(y) < 512.0 * X)):
        bad.append("error bound")
    return bad


def test_mxfp8_pins():
    assert _mx_pins(of.mxfp8_quantize, of.mxfp8_dequantize) == []


def _mx_with(scale_rule, saturate=True):
    def quantize(x):
        x = np.asarray(x, np.float64)
        b = x.reshape(*x.shape[:-1], -1, 32)
        a = np.abs(b).max(-1)
        e = np.where(a > 0, scale_rule(np.where(a > 0, a, 1.0)), -127).astype(np.int64)
        e = np.clip(e, -127, 127)
        y = b / np.ldexp(1.0, e)[..., None]
        c = of.e4m3_encode(y)
        if not saturate:
            c = np.where(np.abs(y) > 464, np.uint8(0x7F), c)
        return c.reshape(x.shape), (e + 127).astype(np.uint8)
    return quantize


@pytest.mark.parametrize("quantize", [
    _mx_with(lambda a: np.floor(np.log2(a)) - 7),
    _mx_with(lambda a: np.ceil(np.log2(a)) - 8),
    _mx_with(lambda a: np.floor(np.log2(a)) - 8, saturate=False),
], ids=["emax7", "ceil", "no_saturation"])
def test_mxfp8_pins_catch_planted_mistakes(quantize):
    assert _mx_pins(quantize, of.mxfp8_dequantize)


def test_q_uproj_rope_is_the_layer_query():
    """The fused up-projection's q equals the query of the pinned layer oracle
    (q_b of the normalised query latent, RoPE on each head's rope part)."""
    sh = mi.WORKLOADS["tiny_fp32_t64"]
    case = mi.make_prefill_case(sh, doc_lengths=[20, 44])
    ref = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    lat = om.rms_norm(np.asarray(case.x, np.float64) @ np.asarray(case.w["w_q_a"], np.float64).T,
                      case.w["q_a_gamma"], sh.norm_eps)
    q = of.q_uproj_rope(sh, case.w["w_q_b"], lat, ref["positions"])
    assert np.allclose(q, ref["q"].reshape(q.shape), rtol=1e-12, atol=1e-12)
    codes, scales, q2 = of.q_uproj_rope_mxfp8(sh, case.w["w_q_b"], lat, ref["positions"])
    assert codes.shape == q.shape and scales.shape == (q.shape[0], q.shape[1] // 32)
    assert np.array_equal(q2, q)
