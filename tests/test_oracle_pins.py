"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each test checks a closed form,
an invariant, a special case that reduces to a library routine, a second
formulation written independently, or the scalar brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
from oracle import brute
from oracle import mla as om

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_dims.json")


def tiny_shape(**kw):
    base = dict(name="tiny", dtype="f32", hidden=8, num_heads=2, q_lora_rank=6, kv_lora_rank=4,
                qk_nope_dim=4, qk_rope_dim=4, v_head_dim=3, rope=mi.RopeSpec(kind="plain", theta=10000.0),
                num_docs=1, total_tokens=5, seed=11)
    base.update(kw)
    return mi.MLAShape(**base)


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_constant_vector_closed_form():
    for a in (-3.0, -1e-4, 0.5, 7.0):
        x = np.full((1, 16), a)
        y = om.rms_norm(x, np.ones(16), 1e-6)
        want = a / math.sqrt(a * a + 1e-6)
        assert np.allclose(y, want, rtol=0, atol=1e-15)


def test_rmsnorm_mean_square_identity_and_gain():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 0.01
    eps = 1e-4
    y = om.rms_norm(x, np.ones(33), eps)
    ms = np.mean(x * x, -1)
    assert np.allclose(np.mean(y * y, -1), ms / (ms + eps), rtol=1e-13)
    g = rng.standard_normal(33)
    assert np.allclose(om.rms_norm(x, g, eps), y * g, rtol=1e-14)


# ----------------------------------------------------------------------------- RoPE
def _plain(theta=10000.0):
    return mi.RopeSpec(kind="plain", theta=theta)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((3, 64))
    c, s = om.rope_cos_sin([0, 0, 0], 64, _plain())
    assert np.array_equal(om.apply_rope(x, c, s), x)


def test_rope_basis_vector_closed_form():
    d, p = 16, 5
    c, s = om.rope_cos_sin([p], d, _plain())
    for i in range(d // 2):
        th = 10000.0 ** (-2 * i / d)
        e = np.zeros((1, d)); e[0, i] = 1.0
        y = om.apply_rope(e, c, s)[0]
        want = np.zeros(d); want[i] = math.cos(p * th); want[i + d // 2] = math.sin(p * th)
        assert np.allclose(y, want, atol=1e-15)
        e2 = np.zeros((1, d)); e2[0, i + d // 2] = 1.0
        y2 = om.apply_rope(e2, c, s)[0]
        want2 = np.zeros(d); want2[i] = -math.sin(p * th); want2[i + d // 2] = math.cos(p * th)
        assert np.allclose(y2, want2, atol=1e-15)


@pytest.mark.parametrize("rope", [_plain(), mi.YARN_V3])
def test_rope_norm_preserving_and_relative(rope):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((2, 64))
    for m, n, dlt in [(0, 3, 11), (100, 7, 500), (4000, 4095, 1)]:
        cm, sm = om.rope_cos_sin([m, n, m + dlt, n + dlt], 64, rope)
        rq = om.apply_rope(q[None], cm[0:1], sm[0:1])[0]
        rk = om.apply_rope(k[None], cm[1:2], sm[1:2])[0]
        rq2 = om.apply_rope(q[None], cm[2:3], sm[2:3])[0]
        rk2 = om.apply_rope(k[None], cm[3:4], sm[3:4])[0]
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
        assert abs(rq @ rk - rq2 @ rk2) < 1e-9


# ----------------------------------------------------------------------------- YaRN
def test_yarn_factor_one_is_plain_rope():
    y = mi.RopeSpec(kind="yarn", theta=10000.0, factor=1.0, original_max_pos=4096, mscale=1.0, mscale_all_dim=1.0)
    assert np.allclose(om.rope_inv_freq(64, y), om.rope_inv_freq(64, _plain()), rtol=2e-16, atol=0)
    assert om.yarn_get_mscale(1.0, 1.0) == 1.0
    assert om.yarn_get_mscale(0.5, 3.0) == 1.0
    assert om.yarn_get_mscale(40.0, 0.0) == 1.0


def test_yarn_wavelength_limits():
    """High-frequency pairs (wavelength < L/beta_fast) keep their frequency;
    low-frequency pairs (wavelength > L/beta_slow) are divided by s exactly;
    the ratio in between is monotone."""
    y = mi.YARN_V3
    plain = om.rope_inv_freq(64, _plain())
    yarn = om.rope_inv_freq(64, y)
    wl = 2 * math.pi / plain
    L = y.original_max_pos
    fast = wl < L / y.beta_fast
    slow = wl > L / y.beta_slow
    assert fast.sum() >= 8 and slow.sum() >= 8
    assert np.array_equal(yarn[fast], plain[fast])
    assert np.allclose(yarn[slow], plain[slow] / y.factor, rtol=1e-15)
    ratio = yarn / plain
    assert np.all(np.diff(ratio) <= 1e-15) and ratio.min() >= 1 / y.factor - 1e-15


def _yarn(**kw):
    return mi.RopeSpec(**{**mi.YARN_V3.__dict__, **kw})


def _check_yarn_values():
    """Values the YaRN reading fixes at the DeepSeek-V3 shape (s = 40,
    original context 4096, beta_fast 32, beta_slow 1, d_rope 64, base 10000).

    Attention factor: the "CSDN walkthrough of HF DeepseekV3Attention"
    (``__init__``) squares mscale(s, mscale_all_dim) into the softmax scaling,
    citing the YaRN paper's equations 21-22, whose factor is 0.1 m ln s + 1;
    the "Megatron-LM MLA guide" (softmax scale) states mscale^2 / sqrt(q_head_dim).
      mscale(40, 1) = 1 + 0.1 ln 40 = 1.3688879454113936
      scale = 1.3688879454113936^2 / sqrt(192) = 0.1352337788608801
    The softmax takes mscale_all_dim only; mscale (the rope-side parameter)
    only enters the cos/sin amplitude mscale(s, mscale) / mscale(s, mscale_all_dim):
      mscale = 0.707, mscale_all_dim = 1: scale unchanged, amplitude 0.9210423553163399
      mscale_all_dim = 0.707:            scale 1.2608037774058554^2 / sqrt(192) = 0.11472138679292612
    Frequency ramp (pairs turning b times over the original context sit at
    index d ln(L / (2 pi b)) / (2 ln base): 10.47 for b = 32, 22.51 for b = 1,
    so low = 10, high = 23): the ratio theta'_i / theta_i is 1 for i <= 10,
    1/40 for i >= 23, and 1 - (39/40)(i - 10)/13 between, e.g. 0.925 at i = 11,
    0.55 at i = 16, 0.1 at i = 22."""
    def close(a, b, rtol=4e-16):
        assert abs(a - b) <= rtol * abs(b), (a, b)

    close(om.yarn_get_mscale(40.0, 1.0), 1.3688879454113936)
    v3 = mi.WORKLOADS["dsv3_prefill_4096"]
    close(om.softmax_scale(v3), 0.1352337788608801)
    close(om.softmax_scale(v3.replace(rope=_yarn(mscale=0.707))), 0.1352337788608801)
    close(om.softmax_scale(v3.replace(rope=_yarn(mscale_all_dim=0.707))), 0.11472138679292612)
    c, s = om.rope_cos_sin([0], 64, _yarn(mscale=0.707))
    assert np.allclose(c, 0.9210423553163399, rtol=4e-16, atol=0) and np.all(s == 0)
    c, s = om.rope_cos_sin([0], 64, mi.YARN_V3)
    assert np.array_equal(c, np.ones_like(c))
    ratio = om.rope_inv_freq(64, mi.YARN_V3) / om.rope_inv_freq(64, _plain())
    assert np.array_equal(ratio[:11], np.ones(11))
    assert np.allclose(ratio[23:], 1 / 40, rtol=1e-15, atol=0)
    for i, want in ((11, 0.925), (16, 0.55), (22, 0.1)):
        close(ratio[i], want, rtol=1e-14)
    assert np.allclose(ratio[11:23], 1 - (39 / 40) * (np.arange(11, 23) - 10) / 13, rtol=1e-14, atol=0)


def test_yarn_attention_factor_and_ramp_values():
    _check_yarn_values()


_YARN_MISTAKES = {
    # the factor with a base-10 logarithm
    "log10": ("yarn_get_mscale", lambda s, m: 1.0 if s <= 1 else 0.1 * m * math.log10(s) + 1.0),
    # the factor applied once instead of squared
    "single_mscale": ("softmax_scale", lambda sh: sh.qk_head_dim ** -0.5 * om.yarn_get_mscale(sh.rope.factor, sh.rope.mscale_all_dim)),
    # the rope-side mscale in place of mscale_all_dim
    "mscale_for_all_dim": ("softmax_scale", lambda sh: sh.qk_head_dim ** -0.5 * om.yarn_get_mscale(sh.rope.factor, sh.rope.mscale) ** 2),
    # the ramp taken over wavelength ratios r = L / lambda instead of pair indices
    "ramp_in_r": ("rope_inv_freq", lambda d, rope: _ramp_in_r(d, rope)),
    # the ramp indices rounded the other way (ceil for beta_fast, floor for beta_slow)
    "ramp_rounding": ("rope_inv_freq", lambda d, rope: _ramp_rounded_inward(d, rope)),
}


def _ramp_in_r(d, rope):
    inv = rope.theta ** (-2.0 * np.arange(d // 2) / d)
    if rope.kind != "yarn":
        return inv
    r = rope.original_max_pos * inv / (2 * math.pi)
    g = np.clip((r - rope.beta_slow) / (rope.beta_fast - rope.beta_slow), 0, 1)   # 1: keep
    return inv * g + inv / rope.factor * (1 - g)


def _ramp_rounded_inward(d, rope):
    inv = rope.theta ** (-2.0 * np.arange(d // 2) / d)
    if rope.kind != "yarn":
        return inv
    idx = lambda b: d * math.log(rope.original_max_pos / (b * 2 * math.pi)) / (2 * math.log(rope.theta))
    lo, hi = math.ceil(idx(rope.beta_fast)), math.floor(idx(rope.beta_slow))
    g = np.clip((np.arange(d // 2) - lo) / (hi - lo), 0, 1)
    return inv * (1 - g) + inv / rope.factor * g


@pytest.mark.parametrize("mistake", list(_YARN_MISTAKES))
def test_yarn_pins_catch_planted_mistakes(monkeypatch, mistake):
    name, fn = _YARN_MISTAKES[mistake]
    monkeypatch.setattr(om, name, fn)
    with pytest.raises(AssertionError):
        _check_yarn_values()


def test_softmax_scale_readings():
    ws = mi.WORKLOADS
    assert om.softmax_scale(ws["tiny_fp32_t64"]) == 48 ** -0.5
    assert om.softmax_scale(ws["megatron_2x2048"]) == 192 ** -0.5
    assert om.softmax_scale(ws["kimi_gated_varlen_8192"]) == 192 ** -0.5
    # mscale_all_dim = 0 leaves the plain scale (page 2: only applied when set)
    s0 = mi.WORKLOADS["dsv3_prefill_4096"].replace(rope=mi.YARN_V3.__class__(**{**mi.YARN_V3.__dict__, "mscale_all_dim": 0.0}))
    assert om.softmax_scale(s0) == 192 ** -0.5
    v3 = om.softmax_scale(ws["dsv3_prefill_4096"])
    assert v3 > 192 ** -0.5


# ----------------------------------------------------------------------------- attention
def _rand_qkv(n, h, dqk, dv, seed=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, h, dqk)), rng.standard_normal((n, h, dqk)), rng.standard_normal((n, h, dv))


def test_attention_single_token_returns_own_value():
    q, k, v = _rand_qkv(4, 3, 6, 5)
    out = om.causal_varlen_attention(q, k, v, 0.3, [0, 1, 2, 3, 4])
    assert np.array_equal(out, v)


def test_attention_zero_query_is_prefix_mean():
    q, k, v = _rand_qkv(9, 2, 6, 5)
    q[:] = 0
    out = om.causal_varlen_attention(q, k, v, 0.7, [0, 9])
    want = np.cumsum(v, 0) / np.arange(1, 10)[:, None, None]
    assert np.allclose(out, want, rtol=1e-13)


def test_attention_dominant_score_selects_value():
    q, k, v = _rand_qkv(6, 1, 4, 3)
    k[:] = 0
    k[2, 0, 0] = 1.0
    q[:, 0, 0] = 1e4
    out = om.causal_varlen_attention(q, k, v, 1.0, [0, 6])
    assert np.allclose(out[2:], np.broadcast_to(v[2], (4, 1, 3)), atol=1e-12)


def test_attention_causality_bit_exact_and_varlen_split():
    q, k, v = _rand_qkv(12, 2, 6, 4)
    cu = [0, 5, 12]
    base = om.causal_varlen_attention(q, k, v, 0.4, cu)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[8:] += 1.0; k2[8:] -= 2.0; v2[8:] *= 3.0
    pert = om.causal_varlen_attention(q2, k2, v2, 0.4, cu)
    assert np.array_equal(base[:8], pert[:8])
    a = om.causal_varlen_attention(q[:5], k[:5], v[:5], 0.4, [0, 5])
    b = om.causal_varlen_attention(q[5:], k[5:], v[5:], 0.4, [0, 7])
    assert np.array_equal(np.concatenate([a, b]), base)
    # evaluating selected rows only gives the same rows as the full evaluation
    rows = om.causal_varlen_attention(q, k, v, 0.4, cu, rows=[3, 11])
    assert np.allclose(rows, base[[3, 11]], rtol=1e-13)


def test_attention_matches_torch_sdpa_float64():
    q, k, v = _rand_qkv(17, 3, 12, 7)
    out = om.causal_varlen_attention(q, k, v, 12 ** -0.5, [0, 17])
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2).contiguous() for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- layer vs brute force
@pytest.mark.parametrize("kw", [
    dict(),
    dict(q_lora_rank=0, num_heads=1, total_tokens=6),
    dict(rope=mi.RopeSpec(kind="none"), output_gate=True),
])
def test_prefill_matches_scalar_brute_force(kw):
    sh = tiny_shape(**kw)
    lens = [2, 1, 4] if sh.total_tokens != 6 else [6]
    case = mi.make_prefill_case(sh, doc_lengths=lens)
    ref = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)["out"]
    bf = np.array(brute.prefill(sh, case.w, case.x, case.cu_seqlens))
    assert np.allclose(ref, bf, rtol=1e-12, atol=1e-14)


def test_tiny_fp32_workload_rows_match_brute_force():
    sh = mi.WORKLOADS["tiny_fp32_t64"]
    case = mi.make_prefill_case(sh, doc_lengths=[12])      # first 12 tokens of the workload draws
    ref = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)["out"]
    bf = np.array(brute.prefill(sh, case.w, case.x, case.cu_seqlens))
    assert np.allclose(ref, bf, rtol=1e-11, atol=1e-13)


def test_prefill_rows_equals_full():
    sh = tiny_shape(total_tokens=10, rope=mi.YARN_V3.__class__(**{**mi.YARN_V3.__dict__, "original_max_pos": 8}))
    case = mi.make_prefill_case(sh, doc_lengths=[3, 7])
    full = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    rows = [0, 2, 3, 9]
    part = om.mla_prefill_rows(sh, case.w, case.x, case.cu_seqlens, rows)
    assert np.allclose(part["out"], full["out"][rows], rtol=1e-13)


# ----------------------------------------------------------------------------- MLA identities
def _absorbed_equals_naive(sh, lens):
    case = mi.make_prefill_case(sh, doc_lengths=lens)
    res = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    A_lat = om.prefill_latent_absorbed(sh, case.w["w_kv_b"], res["q"], res["latent"], case.cu_seqlens)
    A = res["attn"].reshape(A_lat.shape)
    if sh.output_gate:
        return
    assert np.allclose(A_lat, A, rtol=1e-11, atol=1e-13)


def test_mla_latent_form_equals_decompressed_mha():
    _absorbed_equals_naive(tiny_shape(total_tokens=9), [4, 5])
    sh = mi.WORKLOADS["megatron_2x2048"].replace(hidden=64, num_heads=2)
    _absorbed_equals_naive(sh, [5, 11])


def test_decode_absorbed_equals_naive_and_paged_equals_dense():
    sh = mi.WORKLOADS["dsv3_decode_64"].replace(num_heads=4)
    dc = mi.make_decode_case(sh, batch=3, len_lo=5, len_hi=150, block_size=16)
    a = om.decode_absorbed(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, dc.cache, dc.block_table, dc.seq_lens, 16)
    n = om.decode_naive(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, dc.cache, dc.block_table, dc.seq_lens, 16)
    assert np.all(np.isfinite(a)) and np.allclose(a, n, rtol=1e-10, atol=1e-12)
    # paged gather equals the rows stored densely in table order
    b = 1
    L = int(dc.seq_lens[b])
    dense = np.concatenate([dc.cache[blk] for blk in dc.block_table[b] if blk >= 0], 0)[:L]
    assert np.array_equal(om.gather_paged(dc.cache, dc.block_table, b, L, 16), dense)


def test_prefill_last_row_equals_decode_over_written_latents():
    """Row t of a prefill over one document equals decode of the query at t over
    the latent cache that prefill wrote for tokens 0..t (ties the prefill
    latent row to the decode path)."""
    sh = mi.WORKLOADS["megatron_2x2048"].replace(hidden=32, num_heads=2)
    T = 7
    case = mi.make_prefill_case(sh, doc_lengths=[T])
    res = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    bs = 4
    nblk = (T + bs - 1) // bs
    cache = np.full((nblk + 1, bs, res["latent"].shape[1]), np.nan)
    table = np.array([[2, 0]], dtype=np.int32)
    for j in range(T):
        cache[table[0, j // bs], j % bs] = res["latent"][j]
    q = res["q"][T - 1][None]
    out = om.decode_absorbed(sh, case.w["w_kv_b"], q[..., :128], q[..., 128:], cache, table, [T], bs)
    assert np.allclose(out[0], res["attn"][T - 1].reshape(2, 128), rtol=1e-11, atol=1e-13)


def test_gate_and_nope_variant_single_token_returns_own_value():
    """A one-token document: out = W_o (v * sigmoid(g)) for the gated NoPE layer."""
    sh = tiny_shape(rope=mi.RopeSpec(kind="none"), output_gate=True, total_tokens=3)
    case = mi.make_prefill_case(sh, doc_lengths=[1, 1, 1])
    res = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    v = res["kv"][..., sh.qk_nope_dim:].reshape(3, -1)
    g = case.x.astype(np.float64) @ case.w["w_g"].astype(np.float64).T
    want = (v / (1 + np.exp(-g))) @ case.w["w_o"].astype(np.float64).T
    assert np.allclose(res["out"], want, rtol=1e-12)


# ----------------------------------------------------------------------------- page-printed dims
def test_page_dimension_relations():
    g = json.load(open(GOLD))
    d = g["megatron_config_class_defaults"]
    # cache row width per token = kv_lora_rank + qk_pos_emb_head_dim
    sh = mi.WORKLOADS["dsv3_prefill_4096"]
    assert sh.kv_lora_rank + sh.qk_rope_dim == d["kv_lora_rank"] + d["qk_pos_emb_head_dim"] == 576
    assert d["qk_head_dim"] + d["qk_pos_emb_head_dim"] == 192
    k3 = g["kimi_k3_text_config"]
    kimi = mi.WORKLOADS["kimi_gated_varlen_8192"]
    for a, b in [("hidden_size", "hidden"), ("num_attention_heads", "num_heads"), ("q_lora_rank", "q_lora_rank"),
                 ("qk_nope_head_dim", "qk_nope_dim"), ("qk_rope_head_dim", "qk_rope_dim"), ("v_head_dim", "v_head_dim")]:
        assert k3[a] == getattr(kimi, b)
    assert kimi.rope.kind == "none" and k3["mla_use_nope"]
    y = g["megatron_yarn_defaults"]
    assert (mi.YARN_V3.theta, mi.YARN_V3.factor, mi.YARN_V3.original_max_pos, mi.YARN_V3.beta_fast,
            mi.YARN_V3.beta_slow, mi.YARN_V3.mscale) == (y["rotary_base"], y["rotary_scaling_factor"],
                                                           y["original_max_position_embeddings"], y["beta_fast"],
                                                           y["beta_slow"], y["mscale"])


def test_megatron_unit_test_config_shapes_and_identity():
    """The unit-test configuration printed on the Megatron page, with YaRN at
    its defaults and original_max_position_embeddings = 32: the intermediate
    widths follow the page's projection table and the latent form of the
    attention equals the decompressed form."""
    g = json.load(open(GOLD))
    c = g["megatron_unit_test_config"]
    y = g["megatron_yarn_defaults"]
    rope = mi.RopeSpec(kind="yarn", theta=y["rotary_base"], factor=y["rotary_scaling_factor"],
                       original_max_pos=c["original_max_position_embeddings"], beta_fast=y["beta_fast"],
                       beta_slow=y["beta_slow"], mscale=y["mscale"], mscale_all_dim=y["mscale_all_dim"])
    sh = mi.MLAShape(name="megatron_test", dtype="f32", hidden=c["hidden_size"], num_heads=c["num_attention_heads"],
                     q_lora_rank=c["q_lora_rank"], kv_lora_rank=c["kv_lora_rank"], qk_nope_dim=c["qk_head_dim"],
                     qk_rope_dim=c["qk_pos_emb_head_dim"], v_head_dim=c["v_head_dim"], rope=rope, seed=7)
    case = mi.make_prefill_case(sh, doc_lengths=[6, 3])
    res = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    H = c["num_attention_heads"]
    assert res["q"].reshape(9, -1).shape[1] == H * (c["qk_head_dim"] + c["qk_pos_emb_head_dim"])
    assert res["latent"].shape[1] == c["kv_lora_rank"] + c["qk_pos_emb_head_dim"]
    assert res["kv"].reshape(9, -1).shape[1] == H * (c["qk_head_dim"] + c["v_head_dim"])
    assert res["attn"].shape[1] == c["v_head_dim"] * H and res["out"].shape[1] == c["hidden_size"]
    A_lat = om.prefill_latent_absorbed(sh, case.w["w_kv_b"], res["q"], res["latent"], case.cu_seqlens)
    assert np.allclose(A_lat.reshape(9, -1), res["attn"], rtol=1e-11, atol=1e-13)


# ----------------------------------------------------------------------------- planted mistakes
def _mask_one_ahead(q, k, v, scale, cu_seqlens, rows=None):
    """Mutant attention: every query also sees the next key of its document."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out = np.empty(q.shape[:2] + (v.shape[-1],))
    cu = np.asarray(cu_seqlens)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        for t in range(a, b):
            e = min(t + 2, b)
            s = scale * np.einsum("hd,lhd->hl", q[t], k[a:e])
            p = np.exp(s - s.max(-1, keepdims=True))
            out[t] = np.einsum("hl,lhd->hd", p / p.sum(-1, keepdims=True), v[a:e])
    return out


_PLANTED = {
    # wrong sign in rotate_half
    "rope_sign": ("rotate_half", lambda orig: (lambda x: np.concatenate(
        [x[..., x.shape[-1] // 2:], -x[..., :x.shape[-1] // 2]], -1))),
    # RMSNorm divides by the root of the sum instead of the mean
    "rmsnorm_sum": ("rms_norm", lambda orig: (lambda x, g, eps: orig(x, g, eps) / np.sqrt(x.shape[-1]))),
    # the shared rope key dropped from the scores (cos = sin = 0 zeroes q_pe)
    "rope_term_dropped": ("apply_rope", lambda orig: (lambda x, c, s: 0.0 * x)),
    # causal mask off by one
    "mask_off_by_one": ("causal_varlen_attention", lambda orig: _mask_one_ahead),
    # softmax scale inverted
    "scale_inverted": ("softmax_scale", lambda orig: (lambda sh: 1.0 / orig(sh))),
}


@pytest.mark.parametrize("mistake", sorted(_PLANTED))
def test_planted_mistakes_are_caught(monkeypatch, mistake):
    """Each plausible mistake planted in the oracle (on the CPU) makes it
    disagree with the scalar brute force, so the brute-force pin has teeth.
    The unmutated oracle agrees with it (checked first)."""
    sh = tiny_shape(num_docs=2, total_tokens=7)
    case = mi.make_prefill_case(sh, doc_lengths=[4, 3])
    bf = np.array(brute.prefill(sh, case.w, case.x, case.cu_seqlens))
    good = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)["out"]
    assert np.allclose(good, bf, rtol=1e-11, atol=1e-13)
    name, make = _PLANTED[mistake]
    monkeypatch.setattr(om, name, make(getattr(om, name)))
    bad = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)["out"]
    assert not np.allclose(bad, bf, rtol=1e-6, atol=1e-9)


def test_planted_kv_split_swap_is_caught(monkeypatch):
    """Taking W_UK from the v rows of kv_b (and W_UV from the k_nope rows)
    makes the absorbed decode disagree with the naive decode, which splits the
    decompressed kv itself."""
    sh = mi.WORKLOADS["dsv3_decode_64"].replace(num_heads=2)
    dc = mi.make_decode_case(sh, batch=2, len_lo=3, len_hi=40, block_size=16)
    args = (sh, dc.w_kv_b, dc.q_nope, dc.q_pe, dc.cache, dc.block_table, dc.seq_lens, 16)
    n = om.decode_naive(*args)
    assert np.allclose(om.decode_absorbed(*args), n, rtol=1e-10, atol=1e-12)
    orig = om._split_kv_b
    monkeypatch.setattr(om, "_split_kv_b", lambda shape, w: orig(shape, w)[::-1])
    assert not np.allclose(om.decode_absorbed(*args), n, rtol=1e-6, atol=1e-9)


# ----------------------------------------------------------------------------- comparison metrics
def test_bf16_metrics():
    rng = np.random.default_rng(9)
    y = rng.standard_normal((5, 300))
    yb = mi.bf16_round(y.astype(np.float32)).astype(np.float64)
    assert om.bf16_excess_error(y, yb) == 0.0          # a correctly rounded result is within half an ulp
    assert 0 < om.row_rel_error(y, yb) < 2e-2
    bad = y.copy(); bad[2, 7] += 0.1 * np.sqrt(np.mean(y[2] ** 2)) + abs(y[2, 7]) * 2 ** -7
    assert om.bf16_excess_error(y, bad) > 2e-2
    # the next bfloat16 value past the correctly rounded one is counted: at
    # 1.5 (ulp 2^-7) it lies 2^-7 away, 2^-8 of it beyond the allowance
    one = np.full((1, 4), 1.5)
    nxt = one.copy(); nxt[0, 1] = 1.5 + 2.0 ** -7
    assert om.bf16_excess_error(one, nxt) == (2.0 ** -7 - 2.0 ** -8 * 1.5) / 1.5
    nan = yb.copy(); nan[0, 0] = np.nan
    assert om.bf16_excess_error(y, nan) == float("inf") and om.row_rel_error(y, nan) == float("inf")


# ----------------------------------------------------------------------------- chunk over a cached prefix
def test_prefix_attention_zero_prefix_is_causal_and_tail_of_full_run():
    rng = np.random.default_rng(21)
    P, T, H = 7, 5, 3
    q = rng.standard_normal((P + T, H, 6))
    k = rng.standard_normal((P + T, H, 6))
    v = rng.standard_normal((P + T, H, 4))
    full = om.causal_varlen_attention(q, k, v, 0.4, [0, P + T])
    # no prefix: the plain causal run
    assert np.allclose(om.prefix_causal_attention(q[:T], k[:T], v[:T], 0.4, 0),
                       om.causal_varlen_attention(q[:T], k[:T], v[:T], 0.4, [0, T]), rtol=1e-13, atol=1e-15)
    # the last T queries of a causal run over P + T tokens, with the first P as the prefix
    got = om.prefix_causal_attention(q[P:], k, v, 0.4, P)
    assert np.allclose(got, full[P:], rtol=1e-13, atol=1e-15)
    # a query sees every cached key: perturbing any future new key leaves it unchanged
    k2 = k.copy(); k2[P + 3:] += 5.0
    got2 = om.prefix_causal_attention(q[P:], k2, v, 0.4, P)
    assert np.array_equal(got2[:3], got[:3]) and not np.allclose(got2[3:], got[3:])


def _paged_f64(rows, block_size, rng):
    """Store rows [L, W] (float64) in a shuffled pool of blocks; returns cache, table row."""
    nb = (len(rows) + block_size - 1) // block_size
    perm = rng.permutation(nb + 2)[:nb]                # two spare blocks stay NaN
    cache = np.full((nb + 2, block_size, rows.shape[1]), np.nan)
    for i in range(nb):
        part = rows[i * block_size:(i + 1) * block_size]
        cache[perm[i], :len(part)] = part
    return cache, perm


@pytest.mark.parametrize("rope", ["plain", "yarn", "none"])
def test_chunk_layer_equals_tail_of_full_prefill(rope):
    """Two sequences prefilled whole (oracle prefill) versus their first P
    tokens taken from a paged cache and the rest prefilled as a chunk: the
    chunk's outputs and latent rows equal the whole run's last rows."""
    spec = {"plain": mi.RopeSpec(kind="plain", theta=500.0),
            "yarn": mi.RopeSpec(kind="yarn", theta=500.0, factor=4.0, original_max_pos=8, beta_fast=4.0,
                                beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0),
            "none": mi.RopeSpec(kind="none")}[rope]
    sh = tiny_shape(rope=spec, output_gate=(rope == "none"))
    P, T = [6, 3], [4, 5]
    full_case = mi.make_prefill_case(sh, doc_lengths=[P[0] + T[0], P[1] + T[1]], seed=5)
    ref = om.mla_prefill(sh, full_case.w, full_case.x, full_case.cu_seqlens)
    rng = np.random.default_rng(3)
    bs = 4
    cu_full = full_case.cu_seqlens
    caches, tables = [], []
    for d in range(2):
        c, t = _paged_f64(ref["latent"][cu_full[d]: cu_full[d] + P[d]], bs, rng)
        caches.append(c); tables.append(t)
    # one pool: sequence 1's blocks after sequence 0's
    off = caches[0].shape[0]
    cache = np.concatenate(caches, axis=0)
    mb = max(len(t) for t in tables)
    table = np.full((2, mb), -1, dtype=np.int64)
    table[0, :len(tables[0])] = tables[0]
    table[1, :len(tables[1])] = tables[1] + off
    new_rows = np.concatenate([np.arange(cu_full[d] + P[d], cu_full[d + 1]) for d in range(2)])
    x_new = full_case.x[new_rows]
    cu_new = np.array([0, T[0], T[0] + T[1]])
    got = om.mla_prefill_with_prefix(sh, full_case.w, x_new, cu_new, P, cache, table, bs)
    assert np.allclose(got["out"], ref["out"][new_rows], rtol=1e-11, atol=1e-13)
    assert np.allclose(got["latent"], ref["latent"][new_rows], rtol=1e-12, atol=1e-14)
    assert np.array_equal(got["positions"], [6, 7, 8, 9, 3, 4, 5, 6, 7])
    # the rows variant returns the same rows
    part = om.mla_prefill_with_prefix(sh, full_case.w, x_new, cu_new, P, cache, table, bs, rows=[8, 0, 4])
    assert np.allclose(part["out"], got["out"][[8, 0, 4]], rtol=1e-13, atol=1e-15)


def test_chunk_single_query_equals_decode():
    """T = 1 per sequence: the new token attends to all P + 1 keys, which is
    the non-absorbed decode over the cache with the token's own row added."""
    sh = tiny_shape(rope=mi.RopeSpec(kind="plain", theta=100.0))
    c = mi.make_chunk_case(sh, [1, 1, 1], [5, 1, 9], block_size=4, poison_tail=False, seed=7)
    got = om.mla_prefill_with_prefix(sh, c.w, c.x, c.cu_seqlens, c.prefix_lens, c.cache, c.block_table, 4)
    H, nope, dr, dv = sh.num_heads, sh.qk_nope_dim, sh.qk_rope_dim, sh.v_head_dim
    # append each token's own latent row to its sequence (one fresh block each)
    pool = np.concatenate([c.cache.astype(np.float64), np.zeros((3, 4, c.cache.shape[2]))], axis=0)
    table = np.concatenate([c.block_table.astype(np.int64), np.full((3, 1), -1)], axis=1)
    lens = c.prefix_lens.astype(np.int64) + 1
    for b in range(3):
        P = int(c.prefix_lens[b])
        if P % 4 == 0:
            table[b, P // 4] = c.cache.shape[0] + b
        pool[table[b, P // 4], P % 4] = got["latent"][b]
    A = om.decode_naive(sh, c.w["w_kv_b"], got["q"][:, :, :nope], got["q"][:, :, nope:], pool, table, lens, 4)
    assert np.allclose(got["attn"].reshape(3, H, dv), A, rtol=1e-12, atol=1e-14)
    assert not np.any(np.isnan(got["out"]))


# ----------------------------------------------------------------------------- interleaved RoPE, grouped output projection
def _il_to_half(d):
    """Index map: half-split position j takes interleaved feature perm[j]."""
    return np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])


def test_interleaved_rope_is_rotate_half_on_regrouped_features():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((5, 3, 16))
    c, s = om.rope_cos_sin(np.arange(5), 16, _plain(77.0))
    perm = _il_to_half(16)
    got = om.apply_rope_interleaved(x, c[:, None, :], s[:, None, :])
    want_half = om.apply_rope(x[..., perm], c[:, None, :], s[:, None, :])
    back = np.empty_like(want_half)
    back[..., perm] = want_half
    assert np.allclose(got, back, rtol=1e-14, atol=1e-15)
    # norm preserved, position 0 the identity
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(om.apply_rope_interleaved(x[:1], c[:1, None, :], s[:1, None, :]), x[:1])


@pytest.mark.parametrize("rope", ["plain", "yarn"])
def test_interleaved_layer_equals_rotate_half_layer_with_regrouped_weights(rope):
    """With weights laid out for interleaved pairs, the layer with interleaved
    pairs equals the rotate_half layer whose query and key rope rows are
    regrouped."""
    spec = {"plain": mi.RopeSpec(kind="plain", theta=500.0),
            "yarn": mi.RopeSpec(kind="yarn", theta=500.0, factor=4.0, original_max_pos=8, beta_fast=4.0,
                                beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0)}[rope]
    sh_il = tiny_shape(rope=spec, rope_interleave=True, num_heads=3, qk_rope_dim=6)
    sh_h = sh_il.replace(rope_interleave=False)
    case = mi.make_prefill_case(sh_il, doc_lengths=[6, 4], seed=9)
    dn, dr, r = sh_il.qk_nope_dim, sh_il.qk_rope_dim, sh_il.kv_lora_rank
    perm = _il_to_half(dr)
    w2 = dict(case.w)
    Wqb = case.w["w_q_b"].reshape(sh_il.num_heads, dn + dr, -1).copy()
    Wqb[:, dn:, :] = Wqb[:, dn + perm, :]
    w2["w_q_b"] = Wqb.reshape(case.w["w_q_b"].shape)
    Wkva = case.w["w_kv_a"].copy()
    Wkva[r:, :] = case.w["w_kv_a"][r + perm, :]
    w2["w_kv_a"] = Wkva
    a = om.mla_prefill(sh_il, case.w, case.x, case.cu_seqlens)
    b = om.mla_prefill(sh_h, w2, case.x, case.cu_seqlens)
    assert np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    assert np.allclose(a["latent"][:, r + perm], b["latent"][:, r:], rtol=1e-12, atol=1e-14)
    # and the pairing matters: without regrouping the outputs differ
    c_ = om.mla_prefill(sh_h, case.w, case.x, case.cu_seqlens)
    assert not np.allclose(a["out"], c_["out"], rtol=1e-6)


def test_grouped_low_rank_output_projection_equals_its_product():
    sh = tiny_shape(num_heads=4, v_head_dim=3, o_groups=2, o_lora_rank=5, output_gate=True)
    case = mi.make_prefill_case(sh, doc_lengths=[7], seed=4)
    got = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    G, r = 2, 5
    fg = sh.num_heads * sh.v_head_dim // G
    Wa = case.w["w_o_a"].astype(np.float64).reshape(G, r, fg)
    Wb = case.w["w_o_b"].astype(np.float64)
    W_o = np.concatenate([Wb[:, g * r:(g + 1) * r] @ Wa[g] for g in range(G)], axis=1)
    w2 = dict(case.w); w2["w_o"] = W_o
    want = om.mla_prefill(sh.replace(o_groups=0, o_lora_rank=0), w2, case.x, case.cu_seqlens)
    assert np.allclose(got["out"], want["out"], rtol=1e-12, atol=1e-14)
