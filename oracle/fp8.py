"""FP8 (E4M3) latent cache for the absorbed decode: codec, cache quantisation
and the decode it feeds.  TEST INFRASTRUCTURE ONLY (see the package header).

The pages name FP8 only as a recipe ("Megatron-LM MLA guide", parameter
section: ``use_fused_mla_q_uproj``, an MXFP8-quantised query up-projection,
and ``fp8_dot_product_attention``); they print no cache format.  The format
taken here is the plainest one that halves the cached bytes:

* element type: OCP 8-bit floating point, E4M3 variant (published as the OCP
  "8-bit Floating Point Specification (OFP8)" and used by the OCP Microscaling
  (MX) formats that MXFP8 refers to): sign, 4 exponent bits with bias 7, 3
  mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; no
  infinities; S.1111.111 is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448.
* conversion: round to nearest, ties to even, saturating: a value whose
  magnitude exceeds 448 becomes +-448 (the MX specification's conversion rule
  for E4M3), NaN becomes NaN.
* cache rows: each [c_n | k_pe'] row of the bf16 latent cache stored as
  r_kv + d_rope E4M3 codes with ONE float32 scale for the whole cache
  (value = code * scale).  The row x is quantised as E4M3(fl32(x * inv)) with
  inv = fl32(1 / scale), every operation in float32 (the precision in which
  the library takes the same decision), so the codes are a deterministic
  function of the bf16 rows and both sides must agree bit for bit.

The decode over such a cache is defined as the absorbed decode of
``oracle.mla.decode_absorbed`` on the dequantised rows (code * scale, exact
in float64): quantising the cache is the only approximation the format
makes; any further rounding a kernel does inside (an fp8 copy of the absorbed
query, of the probabilities) is that kernel's error, bounded by the tests.

Parity: the codec is pinned by values the OFP8 specification fixes (largest
normal, smallest normal and subnormal, the NaN code), by exhaustive
round-trips of the 254 finite codes, by brute-force nearest-value search with
the even tie break, and by planted mistakes (bias 8, truncation, ties away
from zero, no saturation) that fail those pins.

MXFP8 (the query up-projection the Megatron-LM MLA guide names,
``use_fused_mla_q_uproj``: query up-projection, per-head RoPE and MXFP8
quantisation in one kernel): the OCP Microscaling conversion of a block of
32 consecutive values V_i: shared scale X = 2^(floor(log2(max_i |V_i|)) - emax)
with emax = 8 for E4M3 (its largest binade), stored as the E8M0 byte
(exponent + 127), elements E4M3(V_i / X) with the saturating conversion above;
a block of zeros takes the smallest scale, 2^-127.  Pinned by values the rule
fixes (amax 1 -> scale 2^-8, element 1 -> 256), the exact round trip of
representable blocks, invariance under powers of two, the half-ulp error
bound, and planted mistakes (emax 7, ceil instead of floor, no saturation).
"""
from typing import Optional, Sequence

import numpy as np

from .mla import _f64, _rope, decode_absorbed, rope_cos_sin

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_value(codes) -> np.ndarray:
    """Float64 value of E4M3 codes (uint8 array): (-1)^s * 2^(e-7) * (1 + m/8)
    for exponent field e >= 1, (-1)^s * 2^-6 * m/8 for e = 0, NaN for
    S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _code_of_magnitude(v) -> np.ndarray:
    """Code (sign bit clear) of an exactly representable magnitude v in
    [0, 448]."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.int64)
    nz = v > 0
    e = np.zeros(v.shape, dtype=np.int64)
    e[nz] = np.floor(np.log2(v[nz])).astype(np.int64)
    sub = nz & (e < -6)
    nrm = nz & ~sub
    # subnormal: v = m * 2^-9
    out[sub] = np.rint(v[sub] * 512.0).astype(np.int64)
    # normal: v = 2^e (1 + m/8), field e + 7
    m = np.rint((v[nrm] / np.ldexp(1.0, e[nrm]) - 1.0) * 8.0).astype(np.int64)
    out[nrm] = ((e[nrm] + 7) << 3) | m
    return out


def e4m3_encode(x) -> np.ndarray:
    """E4M3 codes of the values x (taken as float64; callers pass float32
    values): the magnitude is rounded to the nearest point of the E4M3 grid,
    ties to the point with an even mantissa, and saturated at 448.

    The grid: in the binade [2^e, 2^(e+1)) with e >= -6 the points are
    multiples of 2^(e-3); below 2^-6 (the subnormals) multiples of 2^-9.
    Rounding the scaled magnitude x / 2^(e-3) to an integer with ties to even
    is rounding to the nearest grid point with the even-mantissa tie break,
    since consecutive points differ by one in that integer."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.where(nan, 0.0, np.abs(x))
    a = np.minimum(a, E4M3_MAX)                       # saturation (448 is on the grid)
    e = np.full(a.shape, -6, dtype=np.int64)
    pos = a > 0
    e[pos] = np.maximum(np.floor(np.log2(a[pos])).astype(np.int64), -6)
    q = np.ldexp(1.0, e - 3)                          # grid spacing of the binade
    v = np.rint(a / q) * q                            # np.rint rounds half to even
    v = np.minimum(v, E4M3_MAX)
    code = _code_of_magnitude(v)
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def cache_inverse_scale(scale: float) -> np.float32:
    """fl32(1 / scale): the multiplier both sides apply before rounding."""
    return np.float32(1.0) / np.float32(scale)


def cache_quantize_fp8(rows, scale: float) -> np.ndarray:
    """E4M3 codes of latent-cache rows (any shape; bf16 values as float
    arrays): E4M3(fl32(x * fl32(1/scale)))."""
    x = np.asarray(rows, dtype=np.float32)
    y = (x * cache_inverse_scale(scale)).astype(np.float32)
    return e4m3_encode(y)


def cache_dequantize_fp8(codes, scale: float) -> np.ndarray:
    """Float64 rows code * scale (the cache the decode attends over)."""
    return e4m3_value(codes) * float(np.float32(scale))


def decode_absorbed_fp8(shape, w_kv_b, q_nope, q_pe, cache_codes, scale: float, block_table, seq_lens,
                        block_size: int, batch_idx: Optional[Sequence[int]] = None, return_latent: bool = False):
    """Absorbed decode over an E4M3 latent cache: ``decode_absorbed`` on the
    dequantised rows."""
    return decode_absorbed(shape, w_kv_b, q_nope, q_pe, cache_dequantize_fp8(cache_codes, scale), block_table,
                           seq_lens, block_size, batch_idx=batch_idx, return_latent=return_latent)


# ----------------------------------------------------------------------------
# MXFP8 (OCP Microscaling, E4M3 elements, blocks of 32)
# ----------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_EMAX = 8


def mx_scale_exponent(amax) -> np.ndarray:
    """floor(log2 amax) - 8, within the E8M0 range [-127, 127]; -127 for a
    zero block."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64) - E4M3_EMAX
    return np.clip(e, -127, 127)


def mxfp8_quantize(x):
    """(codes, scale_bytes) of x [..., n], n a multiple of 32: blocks of 32
    consecutive values along the last axis.  scale_bytes = exponent + 127."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0
    b = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    e = mx_scale_exponent(np.abs(b).max(-1))
    codes = e4m3_encode(b / np.ldexp(1.0, e)[..., None])
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scale_bytes) -> np.ndarray:
    c = np.asarray(codes)
    v = e4m3_value(c).reshape(*c.shape[:-1], c.shape[-1] // MX_BLOCK, MX_BLOCK)
    e = np.asarray(scale_bytes).astype(np.int64) - 127
    return (v * np.ldexp(1.0, e)[..., None]).reshape(c.shape)


def q_uproj_rope(shape, w_q_b, q_latent, positions) -> np.ndarray:
    """q = q_latent W_qb^T viewed [N, H, d_nope + d_rope], the rope part of
    every head rotated at the token's position ("CSDN walkthrough of HF
    DeepseekV3Attention", forward: q_b_proj, split, apply_rotary_pos_emb on
    q_pe); not rotated for rope kind "none".  Returns [N, H * d_qk], float64."""
    H, nope, dr = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim
    q = (_f64(q_latent) @ _f64(w_q_b).T).reshape(-1, H, nope + dr)
    if shape.rope.kind != "none":
        cos, sin = rope_cos_sin(np.asarray(positions), dr, shape.rope)
        q = np.concatenate([q[..., :nope], _rope(shape, q[..., nope:], cos[:, None, :], sin[:, None, :])], -1)
    return q.reshape(q.shape[0], -1)


def q_uproj_rope_mxfp8(shape, w_q_b, q_latent, positions):
    """The fused query up-projection of the Megatron-LM MLA guide's
    ``use_fused_mla_q_uproj``: ``q_uproj_rope`` quantised to MXFP8 along each
    row (blocks of 32 within a head, as d_qk = 192 is 6 blocks).  Returns
    (codes [N, H d_qk], scale bytes [N, H d_qk / 32], q float64)."""
    q = q_uproj_rope(shape, w_q_b, q_latent, positions)
    codes, scales = mxfp8_quantize(q)
    return codes, scales, q
