"""GPU parity of the FP8 (E4M3) latent cache: the cache conversion and the
absorbed decode over it, through the C ABI, against the float64 oracle
(``oracle.fp8``).

Tolerances
  cache conversion (bf16 rows -> E4M3 codes): bit-exact, both sides rounding
      the same float32 product (integer work decided in the kernel's
      precision).
  decode, exact-arithmetic cases: keys whose latent rows are one-hot E4M3
      values, queries on the E4M3 grid of their MX blocks and a cache scale
      that makes the base-2 score scale 1, so every score is an integer in
      log2 units and every probability a power of two: the kernel's MXFP8
      roundings of the query and of the probabilities are then exact, and
      what remains is the fp16 partials and the bf16 output.  Bound: the bf16
      bound of the bf16 decode tightened tenfold (``bf16_excess_error`` <=
      2e-3).
  decode, seeded N(0, 1) caches: the kernel rounds the absorbed query and the
      probabilities to MXFP8 (E4M3 elements, 3 mantissa bits: relative error
      up to 2^-4, RMS 2^-4 / sqrt(3) = 3.6% per element), which the oracle
      does not.  A float64 emulation of exactly those two roundings on the
      DeepSeek-V3 decode workload gives a worst-head RMS error of 6-9% of the
      head's output RMS and a max-abs error of 18-33% of it.  Bound: RMS error
      per head <= 0.15 of the head's RMS and max-abs <= 0.5 of it; the bf16
      decode of the same (dequantised) cache is printed beside it.
"""
import sys

import numpy as np
import pytest

import mla_inputs as mi
from oracle import fp8 as of
from oracle import mla as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EXACT_TOL = 2e-3
RMS_TOL = 0.15
MAXABS_TOL = 0.5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    import latent_attention_forward_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def rms_rel(ref, got):
    """max over rows of RMS(got - ref) / RMS(ref)."""
    ref, got = np.asarray(ref, np.float64), np.asarray(got, np.float64)
    return float(np.max(np.sqrt(((got - ref) ** 2).mean(-1) / (ref ** 2).mean(-1))))


# ----------------------------------------------------------------------------- cache conversion
@pytest.mark.parametrize("scale", [1.0, 0.0625, 3.0, 1.0 / 48.0])
def test_cache_quantize_bit_exact(mla, scale):
    rng = np.random.default_rng(11)
    n = 2048
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x[: n // 4] *= 100.0                                   # saturating rows
    x[n // 4: n // 2] *= 1e-3                              # subnormal and flushed codes
    x[n // 2, :8] = [0.0, -0.0, 448 * scale, -448 * scale, 464 * scale, 480 * scale, 1e30, -1e30]
    x = mi.bf16_round(x)
    _say(f"case: cache conversion, {n} rows, scale {scale}")
    src = dev(x, torch.bfloat16)
    dst = torch.full((n, 576), 0x55, dtype=torch.uint8, device=DEV)
    mla.cache_quantize_fp8(src, scale, dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    want = of.cache_quantize_fp8(x, scale)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, (len(bad), bad[:5], [(x[i, j], got[i, j], want[i, j]) for i, j in bad[:5]])


def test_cache_quantize_strided_rows_leave_the_rest(mla):
    """Rows of a wider buffer: only the first row_width columns of each row
    are converted, the rest of the destination stays untouched."""
    lib = mla.load_library()
    rng = np.random.default_rng(5)
    x = mi.bf16_round(rng.standard_normal((100, 640)).astype(np.float32))
    src = dev(x, torch.bfloat16)
    dst = torch.full((100, 600), 0x33, dtype=torch.uint8, device=DEV)
    st = lib.mla_cache_quantize_fp8(src.data_ptr(), 640, 100, 576, 0.5, dst.data_ptr(), 600,
                                    torch.cuda.current_stream().cuda_stream)
    assert st == mla.MLA_OK
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.array_equal(got[:, :576], of.cache_quantize_fp8(x[:, :576], 0.5))
    assert np.all(got[:, 576:] == 0x33)


# ----------------------------------------------------------------------------- decode
def run_decode_fp8(mla, sh, dc, codes, cs):
    cfg = mla.make_config(sh)
    B = len(dc.seq_lens)
    out = torch.full((B, sh.num_heads, sh.v_head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
    mla.decode_absorbed_fp8_fwd(cfg, dev(dc.w_kv_b, torch.bfloat16), dev(dc.q_nope, torch.bfloat16),
                                dev(dc.q_pe, torch.bfloat16), torch.from_numpy(codes).to(DEV), cs,
                                torch.from_numpy(dc.block_table).to(DEV), torch.from_numpy(dc.seq_lens).to(DEV),
                                dc.seq_lens, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def run_decode_bf16(mla, sh, dc, cache):
    cfg = mla.make_config(sh)
    B = len(dc.seq_lens)
    out = torch.full((B, sh.num_heads, sh.v_head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
    mla.decode_absorbed_fwd(cfg, dev(dc.w_kv_b, torch.bfloat16), dev(dc.q_nope, torch.bfloat16),
                            dev(dc.q_pe, torch.bfloat16), dev(cache, torch.bfloat16),
                            torch.from_numpy(dc.block_table).to(DEV), torch.from_numpy(dc.seq_lens).to(DEV),
                            dc.seq_lens, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def exact_case(sh, lens, bs, seed=0):
    """Inputs of an exact-arithmetic fp8 decode (see the module header):
    W_UK[h] maps nope dim i to latent dim (4 i + h) mod 512 with weight 1, so
    the absorbed query is q_nope placed on 128 latent dims; q_nope and q_pe
    take values in {0, +-1, +-2}; every cached row holds one non-zero code,
    +-1 or +-2, at a random one of its 576 dims; the cache scale is
    fl32(1 / fl32(scale * log2 e)), so scores are integers in log2 units up to
    a relative 1e-7."""
    rng = np.random.default_rng(seed)
    dc = mi.make_decode_case(sh, seq_lens=lens, block_size=bs, poison_tail=False)
    H, r = sh.num_heads, sh.kv_lora_rank
    w = dc.w_kv_b.reshape(H, 256, r).copy()
    w[:, :128, :] = 0.0
    for h in range(H):
        w[h, np.arange(128), (4 * np.arange(128) + h) % r] = 1.0
    dc.w_kv_b = w.reshape(H * 256, r)
    dc.q_nope = rng.integers(-2, 3, size=dc.q_nope.shape).astype(np.float32)
    dc.q_pe = rng.integers(-2, 3, size=dc.q_pe.shape).astype(np.float32)
    pool = dc.cache.shape[0] * dc.cache.shape[1]
    codes = np.zeros((pool, 576), np.uint8)
    dims = rng.integers(0, 576, size=pool)
    codes[np.arange(pool), dims] = rng.choice(np.array([0x38, 0x40, 0xB8, 0xC0], np.uint8), size=pool)
    codes = codes.reshape(dc.cache.shape)
    c2 = np.float32(np.float32(om.softmax_scale(sh)) * np.float32(1.4426950408889634))
    cs = float(np.float32(1.0) / c2)
    return dc, codes, cs


@pytest.mark.parametrize("heads,lens,bs", [(128, [1, 33, 64, 65, 700, 3000, 129, 4097], 64),
                                           (32, [5, 300, 1000], 16), (96, [129, 700, 64], 32),
                                           (64, [8192, 31, 4000], 16), (128, [30000], 64)])
def test_decode_fp8_exact_arithmetic(mla, heads, lens, bs):
    sh = mi.WORKLOADS["dsv3_decode_64"].replace(num_heads=heads)
    _say(f"case: fp8 decode, exact arithmetic, heads={heads} lens={lens} block={bs}")
    dc, codes, cs = exact_case(sh, lens, bs)
    got = run_decode_fp8(mla, sh, dc, codes, cs)
    B = len(lens)
    ref = of.decode_absorbed_fp8(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, codes, cs, dc.block_table, dc.seq_lens, bs)
    ex = om.bf16_excess_error(ref.reshape(B, -1), got.reshape(B, -1))
    _say(f"  excess over half an ulp {ex:.3e} | strict {om.row_rel_error(ref.reshape(B, -1), got.reshape(B, -1)):.3e}")
    assert ex <= EXACT_TOL


def _random_case_check(mla, sh, dc, cs, label, with_bf16=True):
    codes = of.cache_quantize_fp8(dc.cache, cs)
    got = run_decode_fp8(mla, sh, dc, codes, cs)
    B = len(dc.seq_lens)
    ref = of.decode_absorbed_fp8(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, codes, cs, dc.block_table, dc.seq_lens,
                                 dc.block_size)
    r = rms_rel(ref.reshape(B * sh.num_heads, -1), got.reshape(B * sh.num_heads, -1))
    m = om.row_rel_error(ref.reshape(B * sh.num_heads, -1), got.reshape(B * sh.num_heads, -1))
    msg = f"  {label}: worst-head RMS error {r:.3e}, max-abs / head RMS {m:.3e}"
    if with_bf16:
        deq = of.cache_dequantize_fp8(codes, cs).astype(np.float32)
        deq[np.isnan(dc.cache)] = np.nan
        gb = run_decode_bf16(mla, sh, dc, deq)
        msg += (f" | bf16 decode of the dequantised cache: RMS {rms_rel(ref.reshape(B * sh.num_heads, -1), gb.reshape(B * sh.num_heads, -1)):.3e}, "
                f"max-abs {om.row_rel_error(ref.reshape(B * sh.num_heads, -1), gb.reshape(B * sh.num_heads, -1)):.3e}")
    _say(msg)
    assert np.all(np.isfinite(got))
    assert r <= RMS_TOL and m <= MAXABS_TOL, (r, m)


@pytest.mark.parametrize("heads,lens,bs", [(128, [1, 17, 64, 65, 1000, 3000], 64), (32, [5, 300], 16),
                                           (96, [129, 700], 32), (64, [8192, 31, 4000], 16)])
def test_decode_fp8_small(mla, heads, lens, bs):
    sh = mi.WORKLOADS["dsv3_decode_64"].replace(num_heads=heads)
    _say(f"case: fp8 decode heads={heads} lens={lens} block={bs}")
    dc = mi.make_decode_case(sh, seq_lens=lens, block_size=bs)
    _random_case_check(mla, sh, dc, 1.0 / 32.0, "vs oracle")


def test_decode_fp8_full_size(mla):
    """All 64 sequences of the DeepSeek-V3 decode workload over its cache
    converted to E4M3 (scale 1/32)."""
    sh = mi.WORKLOADS["dsv3_decode_64"]
    _say("case: full-size fp8 decode, 64 sequences")
    dc = mi.make_decode_case(sh)
    _random_case_check(mla, sh, dc, 1.0 / 32.0, "out (all 64 sequences)")


def test_decode_fp8_bad_block_id_poisons_only_its_sequence(mla):
    sh = mi.WORKLOADS["dsv3_decode_64"]
    dc, codes, cs = exact_case(sh, [100, 200, 150], 64)
    dc.block_table[1, 1] = 10 ** 6
    got = run_decode_fp8(mla, sh, dc, codes, cs)
    assert np.all(np.isnan(got[1]))
    ok = [0, 2]
    ref = of.decode_absorbed_fp8(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, codes, cs, dc.block_table, dc.seq_lens, 64,
                                 batch_idx=ok)
    assert om.bf16_excess_error(ref.reshape(2, -1), got[ok].reshape(2, -1)) <= EXACT_TOL


def test_decode_fp8_dominant_key_takes_the_exact_path(mla):
    """One-hot rows again, with one key in the middle of a segment of three
    sequences whose score for every head is about 80 log2 units above the
    rest: the waves of those segments leave their fixed origin and recompute
    their heads with the fp32 online softmax (which rounds neither the query
    nor the probabilities), so the result stays exact."""
    import decode_plan as dp
    sh = mi.WORKLOADS["dsv3_decode_64"]
    lens = [2000 + 37 * b for b in range(64)]
    _say("case: fp8 decode with dominant late keys (exact fallback)")
    dc, codes, cs = exact_case(sh, lens, 64, seed=4)
    dc.q_pe[:, :, 7] = 40.0                             # every head: q_pe[7] = 40
    hit = codes[..., 512 + 7] != 0                      # no other key uses k_pe[7]
    codes[hit, 0] = codes[hit, 512 + 7]
    codes[..., 512 + 7] = 0
    _, _, segs = dp.plan(lens, tile=64)
    for b in (3, 17, 40):
        k0, k1, _ = segs[b][1]                          # a segment in the middle of the sequence
        j = k0 + (k1 - k0) // 2
        assert j - k0 >= 64                             # not in the segment's first tile
        blk, off = dc.block_table[b, j // 64], j % 64
        codes[blk, off, :] = 0
        codes[blk, off, 512 + 7] = 0x40                 # k_pe[7] = 2: score 80 (log2 units)
        codes[blk, off, 5 + b] = 0x38                   # a latent value, so the output is this row's
    got = run_decode_fp8(mla, sh, dc, codes, cs)
    B = len(lens)
    ref = of.decode_absorbed_fp8(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, codes, cs, dc.block_table, dc.seq_lens, 64)
    ex = om.bf16_excess_error(ref.reshape(B, -1), got.reshape(B, -1))
    _say(f"  all sequences: excess over half an ulp {ex:.3e}")
    assert ex <= EXACT_TOL


# ----------------------------------------------------------------------------- MXFP8 query projection
EPS = 2.0 ** -14


def _mx_compare(q, got_c, got_s):
    """Codes and scales of the GPU against the oracle's MXFP8 rule applied to
    the float64 q: equal wherever the decision is clear; where the float64
    value lies within 2^-14 (relative) + 2^-12 X (absolute) of a rounding
    midpoint, or a block's max within a relative 2^-14 of a power of two, the
    fp32 product may fall on either side and either neighbour is accepted.
    Returns (elements excused, blocks excused)."""
    n, w = q.shape
    b = q.reshape(n, w // 32, 32)
    amax = np.abs(b).max(-1)
    e_lo, e_hi = of.mx_scale_exponent(amax * (1 - EPS)), of.mx_scale_exponent(amax * (1 + EPS))
    gs = got_s.astype(np.int64) - 127
    near_s = e_lo != e_hi
    assert np.array_equal(gs[~near_s], e_lo[~near_s]), "scale mismatch away from a power of two"
    assert np.all((gs[near_s] == e_lo[near_s]) | (gs[near_s] == e_hi[near_s]))
    y = b / np.ldexp(1.0, gs)[..., None]                       # the GPU's own block scale
    # -0 and +0 are the same value (a tiny element's sign may differ)
    z = lambda c: np.where(c == 0x80, np.uint8(0), c)
    want = z(of.e4m3_encode(y))
    # relative, and absolute: the fp32 sum of K = 1536 products is off by
    # about 1e-6 of the row's values, ~1e-4 in units of X (the block max is
    # 2^8..2^9 of those units), which moves small elements across a midpoint
    d = EPS * np.abs(y) + 2.0 ** -12
    lo, hi = z(of.e4m3_encode(y - d)), z(of.e4m3_encode(y + d))
    gc = z(got_c.reshape(b.shape))
    ok = (gc == want) | ((lo != hi) & ((gc == lo) | (gc == hi)))
    bad = np.argwhere(~ok)
    assert len(bad) == 0, (len(bad), [(float(y[tuple(i)]), int(gc[tuple(i)]), int(want[tuple(i)])) for i in bad[:6]])
    return int(((gc != want) & ok).sum()), int(near_s.sum())


@pytest.mark.parametrize("name,n", [("dsv3_prefill_4096", 300), ("kimi_gated_varlen_8192", 257),
                                    ("dsv3_prefill_4096", 4096)])
def test_q_uproj_rope_mxfp8(mla, name, n):
    sh = mi.WORKLOADS[name]
    _say(f"case: MXFP8 query projection {name}, {n} tokens")
    rng = np.random.default_rng(21)
    R, H, dqk = sh.q_lora_rank, sh.num_heads, sh.qk_head_dim
    lat = mi.bf16_round(rng.standard_normal((n, R)).astype(np.float32))
    w = mi.bf16_round((rng.standard_normal((H * dqk, R)) * 0.02).astype(np.float32))
    pos = rng.integers(0, 5000, size=n).astype(np.int32)
    cfg = mla.make_config(sh)
    rope = sh.rope.kind != "none"
    cos = sin = None
    if rope:
        cos, sin = mla.rope_table(cfg, 5000, DEV)
    codes = torch.zeros((n, H * dqk), dtype=torch.uint8, device=DEV)
    scales = torch.full((n, H * dqk // 32), 0xFF, dtype=torch.uint8, device=DEV)
    mla.q_uproj_rope_mxfp8(cfg, dev(lat, torch.bfloat16), dev(w, torch.bfloat16),
                           torch.from_numpy(pos).to(DEV) if rope else None, cos, sin, codes, scales)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert not np.any(got_s == 0xFF)                          # every scale written (0xFF is not an E8M0 value here)
    rows = np.arange(n) if n <= 512 else np.sort(rng.choice(n, 128, replace=False))
    q = of.q_uproj_rope(sh, w, lat[rows], pos[rows])
    ne, nb = _mx_compare(q, got_c[rows], got_s[rows])
    _say(f"  {len(rows)} rows: codes off by one near a midpoint {ne} of {q.size}, blocks near a power of two {nb}")
    deq = of.mxfp8_dequantize(got_c[rows], got_s[rows])
    err = np.abs(deq - q).max() / np.abs(q).max()
    _say(f"  max |dequantised - q| / max |q| = {err:.3e}")
