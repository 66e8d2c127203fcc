"""GPU parity of the layout / config variants against the float64 oracle:
RoPE on interleaved pairs and the grouped low-rank output projection, in the
prefill layer (bf16 and fp32) and the chunked prefill.  Bounds as in
test_gpu_parity."""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import mla as om
from test_gpu_parity import F32_TOL, _say, bf16_check, run_prefill  # noqa: F401
from test_gpu_chunk import run_chunk

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import latent_attention_forward_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


V3 = mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=4, q_lora_rank=256)
VARIANTS = {
    "interleaved_rope_yarn": (V3.replace(rope_interleave=True), [70, 1, 131]),
    "grouped_o_proj": (V3.replace(o_groups=2, o_lora_rank=64), [70, 1, 131]),
    "interleaved_grouped_direct_q": (mi.WORKLOADS["megatron_2x2048"].replace(hidden=256, num_heads=2, rope_interleave=True,
                                                                           o_groups=4, o_lora_rank=32), [128, 40]),
    "grouped_gate_nope": (mi.WORKLOADS["kimi_gated_varlen_8192"].replace(hidden=384, num_heads=3, q_lora_rank=128,
                                                                         o_groups=3, o_lora_rank=96), [33, 190]),
}


@pytest.mark.parametrize("name", list(VARIANTS))
def test_prefill_variant(mla, name):
    sh, lens = VARIANTS[name]
    _say(f"case: prefill variant {name} lens={lens}")
    case = mi.make_prefill_case(sh, doc_lengths=lens)
    got, lat = run_prefill(mla, sh, case, latent=True)
    ref = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    bf16_check(ref["out"], got, "out")
    bf16_check(ref["latent"], lat, "latent")


def test_prefill_variants_fp32(mla):
    sh = mi.WORKLOADS["tiny_fp32_t64"].replace(rope_interleave=True, o_groups=2, o_lora_rank=16)
    _say("case: tiny fp32, interleaved RoPE + grouped output projection")
    case = mi.make_prefill_case(sh)
    got, lat = run_prefill(mla, sh, case, latent=True)
    ref = om.mla_prefill(sh, case.w, case.x, case.cu_seqlens)
    err = om.row_rel_error(ref["out"], got)
    _say(f"  err {err:.3e}")
    assert err <= F32_TOL
    assert om.row_rel_error(ref["latent"], lat) <= F32_TOL


def test_chunk_interleaved_rope(mla):
    sh = V3.replace(rope_interleave=True, o_groups=4, o_lora_rank=128)
    _say("case: chunk over prefix, interleaved RoPE + grouped output projection")
    c = mi.make_chunk_case(sh, [40, 100], [300, 64], block_size=64)
    got, lat = run_chunk(mla, sh, c)
    ref = om.mla_prefill_with_prefix(sh, c.w, c.x, c.cu_seqlens, c.prefix_lens, c.cache, c.block_table, 64)
    bf16_check(ref["out"], got, "out")
    bf16_check(ref["latent"], lat, "latent")


def test_grouped_o_proj_full_megatron_defaults_sampled_rows(mla):
    """DeepSeek-V3 shape with the guide's defaults: 8 groups of rank 1024."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(o_groups=8, o_lora_rank=1024, rope_interleave=True)
    lens = [512]
    _say("case: full-size layer, 8 x 1024 grouped output projection, interleaved RoPE, 512 tokens")
    case = mi.make_prefill_case(sh, doc_lengths=lens)
    got, _ = run_prefill(mla, sh, case)
    rows = [0, 1, 100, 255, 400, 511]
    ref = om.mla_prefill_rows(sh, case.w, case.x, case.cu_seqlens, rows)
    bf16_check(ref["out"], got[rows], "out (sampled rows)")
