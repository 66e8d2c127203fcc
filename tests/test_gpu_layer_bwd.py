"""GPU parity of the layer backward (``mla_prefill_bwd``) against the float64
oracle (``oracle.backward.mla_prefill_backward``).

Inputs: the seeded bf16 layer case (x ~ N(0, 1), weights ~ N(0, 0.02)), norm
gains 1 + 0.1 N(0, 1) (so their gradients are exercised), output gradient
dout ~ N(0, 1) in bf16.  Every gradient the configuration has (dx and each
weight's) is compared with the oracle's, as the normwise relative error
||g - r|| / ||r|| and the worst row's relative error; the bounds are stated
beside ``REL_TOL`` below.  (Rows, not elements against the tensor RMS: the dx
rows of a document's first tokens, whose keys every later token attends to,
are up to 17 times the tensor's RMS.)
"""
import sys

import numpy as np
import pytest

import mla_inputs as mi
from oracle import backward as ob

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# The library evaluates the gradient at the bf16-rounded forward (q, kv, the
# latent, the attention output) and rounds every GEMM operand, the attention's
# P and dS and the gradients between the steps to bf16 (unit roundoff
# u = 2^-8).  The longest chain from dout to a gradient passes about 12 such
# roundings; independent roundings of relative size <= u add up to a relative
# RMS error of about u sqrt(12 / 3) = 2u.  Bounds: normwise 4u (twice that);
# each row within 8u of its norm, rows below a tenth of the RMS row norm
# measured against that tenth.
REL_TOL = 4 * 2.0 ** -8
ROW_TOL = 8 * 2.0 ** -8


def row_error(g, r):
    g2, r2 = g.reshape(g.shape[0], -1), r.reshape(r.shape[0], -1)
    if g.ndim == 1:
        g2, r2 = g[None, :], r[None, :]
    norms = np.linalg.norm(r2, axis=1)
    floor = 0.1 * np.sqrt(np.mean(norms ** 2))
    return float(np.max(np.linalg.norm(g2 - r2, axis=1) / np.maximum(norms, floor)))


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


def run_case(mla, sh, lens, seed=0):
    case = mi.make_prefill_case(sh, doc_lengths=lens, seed=seed)
    rng = np.random.default_rng(seed + 100)
    w = dict(case.w)
    for g in ("q_a_gamma", "kv_a_gamma"):
        if w.get(g) is not None:
            w[g] = mi.bf16_round((1.0 + 0.1 * rng.standard_normal(w[g].shape)).astype(np.float32))
    n = case.x.shape[0]
    dout = mi.bf16_round(rng.standard_normal((n, sh.hidden)).astype(np.float32))
    ref = ob.mla_prefill_backward(sh, {k: (None if v is None else v.astype(np.float64)) for k, v in w.items()},
                                  case.x.astype(np.float64), case.cu_seqlens, dout.astype(np.float64))
    cfg = mla.make_config(sh)
    W = {k: (None if v is None else dev(v, torch.bfloat16)) for k, v in w.items()}
    cu = case.cu_seqlens
    cos = sin = None
    if sh.rope.kind != "none":
        cos, sin = mla.rope_table(cfg, int(np.max(np.diff(cu))), DEV)
    grads = {k: torch.full(w[k].shape, float("nan"), dtype=torch.float32, device=DEV) for k in ref if k != "x"}
    dx = torch.full((n, sh.hidden), float("nan"), dtype=torch.float32, device=DEV)
    mla.prefill_bwd(cfg, W, dev(case.x, torch.bfloat16), torch.from_numpy(cu).to(DEV), cu,
                    dev(dout, torch.bfloat16), dx, grads, rope_cos=cos, rope_sin=sin)
    torch.cuda.synchronize()
    got = {"x": dx.cpu().numpy(), **{k: v.cpu().numpy() for k, v in grads.items()}}
    worst = {}
    for name, g in got.items():
        r = ref[name]
        assert g.shape == r.shape, name
        assert np.all(np.isfinite(g)), name
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        row = row_error(g, r)
        _say(f"  d{name}: relative error {rel:.3e}, worst row {row:.3e}")
        worst[name] = (rel, row)
    assert set(got) == set(ref)
    for name, (rel, row) in worst.items():
        assert rel <= REL_TOL and row <= ROW_TOL, (name, rel, row)


SMALL = dict(hidden=256, num_heads=4)
VARIANTS = {
    "v3_yarn_q_lora": mi.WORKLOADS["dsv3_prefill_4096"].replace(q_lora_rank=128, **SMALL),
    "direct_q_plain_rope": mi.WORKLOADS["megatron_2x2048"].replace(**SMALL),
    "kimi_gate_nope": mi.WORKLOADS["kimi_gated_varlen_8192"].replace(q_lora_rank=128, **SMALL),
    "interleaved_rope": mi.WORKLOADS["dsv3_prefill_4096"].replace(q_lora_rank=128, rope_interleave=True, **SMALL),
    "grouped_o_proj": mi.WORKLOADS["dsv3_prefill_4096"].replace(q_lora_rank=128, o_groups=2, o_lora_rank=64,
                                                                **SMALL),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_layer_backward_variants(mla, variant):
    _say(f"case: layer backward {variant}, lens=[37, 100, 3]")
    run_case(mla, VARIANTS[variant], [37, 100, 3])


# 128 heads: dW_kv_b ([128 * 256, 512]) and, with the direct q projection
# and hidden 768, dW_q ([128 * 192, 768]) have at least 256 output tiles of
# 256 x 256, so they run on K-major operands over the first 288 of the 300
# tokens, the last 12 added from their transposes.
MANY_HEADS = {
    "q_lora": mi.WORKLOADS["dsv3_prefill_4096"].replace(q_lora_rank=128, hidden=256, num_heads=128),
    "direct_q": mi.WORKLOADS["megatron_2x2048"].replace(hidden=768, num_heads=128),
}


@pytest.mark.parametrize("variant", list(MANY_HEADS))
def test_layer_backward_many_heads(mla, variant):
    _say(f"case: layer backward 128 heads {variant}, lens=[37, 100, 163]")
    run_case(mla, MANY_HEADS[variant], [37, 100, 163], seed=6)


def test_layer_backward_wide_hidden(mla):
    """4096 tokens, hidden 4096, 8 heads, q latent 1536: the NN products dx =
    dc W_kv_a + dq_lat W_q_a (16 x 16 output tiles) and the split-K product
    dq W_q_b (16 x 6 tiles x 4 slices) have at least 256 tiles of 256 x 256
    and read their [k, n] weight K-major on the 256x256 kernel."""
    _say("case: layer backward, hidden 4096, 8 heads, lens=[2048, 2048]")
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(q_lora_rank=1536, hidden=4096, num_heads=8)
    run_case(mla, sh, [2048, 2048], seed=7)


def test_layer_backward_one_token_documents(mla):
    """Documents of one token (their attention gradient reaches only v) beside
    a document longer than one 128-row tile."""
    _say("case: layer backward, lens=[1, 1, 150, 1]")
    run_case(mla, VARIANTS["v3_yarn_q_lora"], [1, 1, 150, 1], seed=2)


def test_layer_backward_empty_document(mla):
    """An empty document between two others (repeated offset in cu_seqlens)."""
    _say("case: layer backward, lens=[20, 0, 60]")
    run_case(mla, VARIANTS["direct_q_plain_rope"], [20, 0, 60], seed=4)


def test_layer_backward_megatron_full_size(mla):
    """The Megatron-default layer at its full size: hidden 2048, 16 heads,
    direct q projection, two documents of 2048 tokens."""
    _say("case: layer backward, Megatron shape 2 x 2048")
    run_case(mla, mi.WORKLOADS["megatron_2x2048"], [2048, 2048], seed=5)
