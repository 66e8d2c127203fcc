"""Host-side tests of the C ABI (no GPU needed): the library loads and exports
every function declared in include/mla.h, argument checks reject bad input
before any device work, and the host-only helpers (softmax scale, RoPE / YaRN
table) agree with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_inputs as mi
from oracle import mla as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("latent_attention_forward_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        pytest.skip("libmla.so not built")
    return mla.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mla.exported_symbols())
    assert lib.mla_abi_version() == 6


def test_config_validation(lib):
    ok = mla.make_config(mi.WORKLOADS["dsv3_prefill_4096"])
    assert lib.mla_validate_config(ctypes.byref(ok)) == mla.MLA_OK
    bad = [
        dict(qk_rope_dim=63), dict(num_heads=0), dict(dtype=7), dict(rope_kind=9),
        dict(yarn_beta_fast=0.5), dict(rope_theta=0.0), dict(output_gate=3), dict(kv_lora_rank=-1),
        dict(rope_interleave=2), dict(o_groups=-1), dict(o_groups=8, o_lora_rank=0), dict(o_groups=3, o_lora_rank=64),
        dict(attn_operand=2), dict(attn_operand=-1), dict(dtype=mla.MLA_F32, attn_operand=mla.MLA_ATTN_BF16),
    ]
    for kw in bad:
        c = mla.make_config(mi.WORKLOADS["dsv3_prefill_4096"], **kw)
        assert lib.mla_validate_config(ctypes.byref(c)) == mla.MLA_ERR_INVALID_ARG, kw
        assert lib.mla_last_error().decode()
    assert lib.mla_validate_config(None) == mla.MLA_ERR_INVALID_ARG
    for kw in (dict(rope_interleave=1), dict(o_groups=8, o_lora_rank=1024), dict(attn_operand=mla.MLA_ATTN_BF16)):
        c = mla.make_config(mi.WORKLOADS["dsv3_prefill_4096"], **kw)
        assert lib.mla_validate_config(ctypes.byref(c)) == mla.MLA_OK, kw
    # the ctypes mirror of the config has the C layout: its size includes the appended variant fields
    assert ctypes.sizeof(mla.MlaConfig) == 120 and ctypes.sizeof(mla.MlaWeights) == 11 * 8


def test_softmax_scale_matches_oracle(lib):
    for name in ("tiny_fp32_t64", "megatron_2x2048", "dsv3_prefill_4096", "kimi_gated_varlen_8192"):
        sh = mi.WORKLOADS[name]
        got = mla.softmax_scale(mla.make_config(sh))
        assert got == np.float32(om.softmax_scale(sh)), name
    c = mla.make_config(mi.WORKLOADS["megatron_2x2048"], softmax_scale=0.5)
    assert mla.softmax_scale(c) == 0.5
    # the DeepSeek-V3 YaRN value (1 + 0.1 ln 40)^2 / sqrt(192), rounded to float32
    assert mla.softmax_scale(mla.make_config(mi.WORKLOADS["dsv3_prefill_4096"])) == np.float32(0.1352337788608801)


@pytest.mark.parametrize("name", ["tiny_fp32_t64", "megatron_2x2048", "dsv3_prefill_4096"])
def test_rope_table_equals_oracle_rounded(lib, name):
    sh = mi.WORKLOADS[name]
    cfg = mla.make_config(sh)
    P = 4096
    cos, sin = mla.rope_table_host(cfg, P)
    oc, os_ = om.rope_cos_sin(np.arange(P), sh.qk_rope_dim, sh.rope)
    assert np.array_equal(cos, oc.astype(np.float32))
    assert np.array_equal(sin, os_.astype(np.float32))


def test_rope_table_rejects_nope(lib):
    cfg = mla.make_config(mi.WORKLOADS["kimi_gated_varlen_8192"])
    buf = np.empty(64, np.float32)
    assert lib.mla_rope_table(ctypes.byref(cfg), 2, buf.ctypes.data, buf.ctypes.data) == mla.MLA_ERR_INVALID_ARG


def test_workspace_sizes(lib):
    cfg = mla.make_config(mi.WORKLOADS["dsv3_prefill_4096"])
    s1 = mla.prefill_workspace_size(cfg, 4096, 1)
    H = 128
    # bf16 buffers, the fp32 q down-projection and the joint one as two split-K partials
    need = 4096 * ((1536 + H * 192 + 576 + 64 + H * 256 + H * 128) * 2 + (1536 + 2 * 576) * 4)
    assert s1 >= need and s1 < need + 16 * 4096
    assert mla.prefill_workspace_size(cfg, 8192, 1) > s1
    d = mla.decode_workspace_size(mla.make_config(mi.WORKLOADS["dsv3_decode_64"]), [1024] * 64)
    assert d >= 2 * 64 * 128 * 512 * 2


def test_device_calls_reject_bad_arguments_before_launch(lib):
    """Every check below fails on the host; no HIP call is made."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"]
    cfg = mla.make_config(sh)
    w = mla.MlaWeights()
    cu = np.array([0, 16], np.int32)
    f = lib.mla_prefill_fwd
    # missing weights
    st = f(ctypes.byref(cfg), ctypes.byref(w), 16, 16, cu.ctypes.data, 1, None, None, None, 0, 16, None, 16, 1 << 30, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    # non-monotone offsets
    bad_cu = np.array([0, 8, 4], np.int32)
    st = f(ctypes.byref(cfg), ctypes.byref(w), 16, 16, bad_cu.ctypes.data, 2, None, None, None, 0, 16, None, 16, 0, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    # bf16 with an unsupported head shape
    c2 = mla.make_config(sh, qk_nope_dim=64)
    st = f(ctypes.byref(c2), ctypes.byref(w), 16, 16, cu.ctypes.data, 1, None, None, None, 0, 16, None, 16, 0, None)
    assert st == mla.MLA_ERR_UNSUPPORTED
    # workspace too small (weights present, fake aligned addresses, nothing is launched)
    for name, _ in mla.MlaWeights._fields_:
        setattr(w, name, 4096)
    w.w_q = None
    w.w_g = None
    st = f(ctypes.byref(cfg), ctypes.byref(w), 4096, 4096, cu.ctypes.data, 1, None, 4096, 4096, 64, 4096, None, 4096, 16, None)
    assert st == mla.MLA_ERR_WORKSPACE
    # misaligned x
    st = f(ctypes.byref(cfg), ctypes.byref(w), 4098, 4096, cu.ctypes.data, 1, None, 4096, 4096, 64, 4096, None, 4096, 1 << 40, None)
    assert st == mla.MLA_ERR_MISALIGNED
    # decode: fp32 unsupported, bad lengths, bad block size
    dcfg = mla.make_config(mi.WORKLOADS["dsv3_decode_64"])
    lens = np.array([100, 0], np.int32)
    g = lib.mla_decode_absorbed_fwd
    st = g(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096, 1 << 30, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    lens = np.array([100, 300], np.int32)
    st = g(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096, 1 << 30, None)
    assert st == mla.MLA_ERR_INVALID_ARG       # 300 > max_blocks * block_size
    st = g(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 10, 60, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096, 1 << 30, None)
    assert st == mla.MLA_ERR_INVALID_ARG       # block size not a power of two
    d2 = mla.make_config(mi.WORKLOADS["dsv3_decode_64"], num_heads=48)
    lens = np.array([100, 200], np.int32)
    st = g(ctypes.byref(d2), 4096, 4096, 4096, 4096, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096, 1 << 30, None)
    assert st == mla.MLA_ERR_UNSUPPORTED
    f32 = mla.make_config(mi.WORKLOADS["tiny_fp32_t64"])
    st = g(ctypes.byref(f32), 4096, 4096, 4096, 4096, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096, 1 << 30, None)
    assert st == mla.MLA_ERR_UNSUPPORTED
    # decode without a workspace: a batch whose plan needs more than the 64 MiB
    # static scratch is refused before anything runs
    big = np.full(300, 8192, np.int32)
    assert mla.decode_workspace_size(dcfg, big) > 64 << 20
    st = lib.mla_decode_absorbed_fwd_noalloc(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 10, 64, 4096, 128, 4096,
                                             big.ctypes.data, 300, 4096, None)
    assert st == mla.MLA_ERR_WORKSPACE and b"static scratch" in lib.mla_last_error()
    st = lib.mla_decode_absorbed_fwd_noalloc(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 10, 60, 4096, 4, 4096,
                                             lens.ctypes.data, 2, 4096, None)
    assert st == mla.MLA_ERR_INVALID_ARG       # the same argument checks as with a workspace
    # fp8 decode: the same checks, then the cache scale; cache quantisation
    lens = np.array([100, 200], np.int32)
    h = lib.mla_decode_absorbed_fp8_fwd
    st = h(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 1.0, 10, 60, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096,
           1 << 30, None)
    assert st == mla.MLA_ERR_INVALID_ARG       # block size not a power of two
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        st = h(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, bad, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096,
               4096, 1 << 30, None)
        assert st == mla.MLA_ERR_INVALID_ARG and b"cache_scale" in lib.mla_last_error()
    st = h(ctypes.byref(dcfg), 4096, 4096, 4096, 4096, 1.0, 10, 64, 4096, 4, 4096, lens.ctypes.data, 2, 4096, 4096,
           16, None)
    assert st == mla.MLA_ERR_WORKSPACE
    q = lib.mla_cache_quantize_fp8
    assert q(4096, 576, 10, 576, 0.0, 8192, 576, None) == mla.MLA_ERR_INVALID_ARG
    assert q(4096, 576, 10, 570, 1.0, 8192, 576, None) == mla.MLA_ERR_MISALIGNED
    assert q(4096, 576, 10, 576, 1.0, 8196, 576, None) == mla.MLA_ERR_MISALIGNED
    assert q(4096, 576, 10, 576, 1.0, None, 576, None) == mla.MLA_ERR_INVALID_ARG
    assert q(4096, 576, 0, 576, 1.0, 8192, 576, None) == mla.MLA_OK   # nothing to convert
    # attention backward: dtype, missing pointers, alignment, workspace
    b = lib.mla_attention_prefill_bwd
    cu2 = np.array([0, 100, 300], np.int32)
    args = lambda **kw: [kw.get(k, 4096) for k in ("q", "kv", "kpe")] + [kw.get("kpe_stride", 576), 4096,
                                                                          cu2.ctypes.data, 2, kw.get("out", 4096),
                                                                          kw.get("lse", None)] + \
        [kw.get(k, 4096) for k in ("dout", "dq", "dkv", "dkpe", "ws")] + [kw.get("wsb", 1 << 30), None]
    assert b(ctypes.byref(f32), *args()) == mla.MLA_ERR_UNSUPPORTED
    assert b(ctypes.byref(cfg), *args(dout=None)) == mla.MLA_ERR_INVALID_ARG
    assert b(ctypes.byref(cfg), *args(kpe_stride=32)) == mla.MLA_ERR_INVALID_ARG
    assert b(ctypes.byref(cfg), *args(dq=4100)) == mla.MLA_ERR_MISALIGNED
    assert b(ctypes.byref(cfg), *args(kpe_stride=580)) == mla.MLA_ERR_MISALIGNED
    assert b(ctypes.byref(cfg), *args(wsb=16)) == mla.MLA_ERR_WORKSPACE
    assert b(ctypes.byref(cfg), *args(lse=4098)) == mla.MLA_ERR_MISALIGNED
    # attention forward: the log-sum-exp output needs a bf16 config and 4-byte alignment
    fa = lib.mla_attention_prefill
    fargs = lambda c, op, lse: [ctypes.byref(c), op, 4096, 4096, 4096, 576, 4096, cu2.ctypes.data, 2, 4096, lse,
                                None, 0, None]
    assert fa(*fargs(f32, mla.MLA_F32, 4096)) == mla.MLA_ERR_UNSUPPORTED
    assert fa(*fargs(cfg, mla.MLA_BF16, 4098)) == mla.MLA_ERR_MISALIGNED
    assert mla.attention_bwd_workspace_size(cfg, 300) == 2 * 153600 + 300 * 128 * 64 * 4
    empty = np.array([0, 0], np.int32)
    assert b(ctypes.byref(cfg), None, None, None, 576, None, empty.ctypes.data, 1, None, None, None, None, None,
             None, None, 0, None) == mla.MLA_OK
    # layer backward: fp32 config, a missing weight gradient, workspace
    lb = lib.mla_prefill_bwd
    for name, _ in mla.MlaWeights._fields_:
        setattr(w, name, 4096)
    w.w_q = w.w_g = w.w_o_a = w.w_o_b = None
    dw = mla.MlaWeightGrads()
    for name, _ in mla.MlaWeightGrads._fields_:
        setattr(dw, name, 4096)
    lb_args = lambda c, g, wsb: [ctypes.byref(c), ctypes.byref(w), 4096, 4096, cu.ctypes.data, 1, None, 4096, 4096,
                                 64, 4096, 4096, ctypes.byref(g), 4096, wsb, None]
    assert lb(*lb_args(f32, dw, 1 << 40)) == mla.MLA_ERR_UNSUPPORTED
    assert lb(*lb_args(cfg, dw, 16)) == mla.MLA_ERR_WORKSPACE
    dw.w_kv_b = None
    assert lb(*lb_args(cfg, dw, 1 << 40)) == mla.MLA_ERR_INVALID_ARG and b"w_kv_b" in lib.mla_last_error()
    assert mla.prefill_bwd_workspace_size(cfg, 4096) > mla.attention_bwd_workspace_size(cfg, 4096)
    # norm/rope: rope slices overlapping the norm region, slot mapping in place
    st = lib.mla_latent_norm_rope(ctypes.byref(cfg), 4096, 576, 4, 576, 512, 4096, 500, 1, 64, 4096, 4096, 16, 4096,
                                  8192, 576, None, 0, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    st = lib.mla_latent_norm_rope(ctypes.byref(cfg), 4096, 576, 4, 576, 512, 4096, 512, 1, 64, 4096, 4096, 16, 4096,
                                  4096, 576, 4096, 8, None)
    assert st == mla.MLA_ERR_INVALID_ARG
    assert mla.MLAError(1, "x", "y").status == 1


def test_binding_refuses_host_tensors():
    """The binding passes raw device addresses: a host tensor is refused before
    any call, never handed to a kernel."""
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        mla._ptr(torch.zeros(4))
    with pytest.raises(ValueError):
        mla._ptr(torch.zeros(4, 4), rows=True)
    assert mla._ptr(None) is None


@pytest.mark.parametrize("lens", [[1], [5, 300], [1024, 8192, 4000, 17], [30600] * 68, [8192] * 300,
                                  list(range(1, 200, 7))])
def test_decode_plan_matches_workspace_size(lib, lens):
    """The library's decode workspace equals what the split plan (restated in
    tests/decode_plan.py) needs, and every segment the plan makes is a
    non-empty-or-cut key range of its sequence that covers it exactly once."""
    import decode_plan as dp
    cfg = mla.make_config(mi.WORKLOADS["dsv3_decode_64"])
    assert mla.decode_workspace_size(cfg, lens) == dp.workspace_bytes(lens, 128, 512)
    assert mla.decode_fp8_workspace_size(cfg, lens) == dp.workspace_bytes(lens, 128, 512, tile=64)
    for tile in (32, 64):
        quota, groups, segs = dp.plan(lens, tile)
        assert quota % tile == 0 and quota <= dp.max_quota(tile)
        for L, s in zip(lens, segs):
            cover = [k for k0, k1, _ in s for k in range(k0, k1)]
            assert cover == list(range(L))
            assert [slot for _, _, slot in s] == list(range(len(s)))
            # tiles start on multiples of the tile inside the sequence
            assert all(k0 % tile == 0 for k0, k1, _ in s if k1 > k0)
            # a segment spans at most the blocks of 16 tokens one workgroup stages
            assert all((k1 - 1) // 16 - k0 // 16 + 1 <= dp.MAX_CHUNK_BLOCKS for k0, k1, _ in s if k1 > k0)
        ent, n_ent = dp.entries(lens, tile)
        assert len(set(ent.values())) == len(ent) and max(ent.values()) < n_ent
