"""CPU oracle for the Multi-Latent Attention (MLA) forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers); the only module both sides use
is ``mla_inputs``, which draws the seeded inputs and holds none of the method's
arithmetic.

Everything is float64 NumPy (``mla.py``, ``fp8.py``, ``backward.py``) or pure-Python scalar
loops (``brute.py``), written from the pages' statement of the layer:

* "CSDN walkthrough of HF DeepseekV3Attention" (``__init__`` and ``forward``
  listing): projections, latent RMSNorm, split, RoPE on the 64-wide slice with a
  single shared key head, concatenation, YaRN softmax-scale correction.
* "kimi_vl.py - KimiVL (DeepSeek-V3 architecture) attention adapter", sections
  "Q projection and KV compression" and "concatenating the final Q and K".
* "MiniMind: attention forward pass", section 3 (RMSNorm in fp32, rotate_half
  RoPE), section 5 (scaled dot product, causal mask, fp32 softmax, and the mask
  of a forward with a cache: only the new T x T block is triangular), section 7
  (merge heads, output projection).
* "Megatron-LM MLA guide", sections on projection dimensions, YaRN parameters,
  softmax scale, THD packing and the inference section (latent cache, weight
  absorption for decode-only steps, decompression of the cached latents for
  prefill and mixed steps).
* "Kimi-K3 atlas: Gated MLA" (mla-init, mla-forward, rmsnorm excerpts): the
  unrotated shared key part and the full-rank output gate.
* The FP8 latent cache (``fp8.py``): the pages name FP8 / MXFP8 only as a
  recipe ("Megatron-LM MLA guide", parameter section); the element format is
  the published OCP 8-bit floating point E4M3 with the OCP Microscaling
  conversion rule (round to nearest even, saturate at 448).

Parity status of each function is listed in its docstring ("pinned by ...").
The pages cite the YaRN paper for the attention factor (``yarn_get_mscale``)
and the frequency blend (``rope_inv_freq`` for kind "yarn") without printing
either formula; the paper's forms are taken, and the values they give at the
DeepSeek-V3 shape (attention factor, softmax scale, the ramp between pair
indices 10 and 23) are pinned, together with their structural properties
(identity at factor 1, wavelength limits).  That a trained DeepSeek-V3 uses
exactly these constants is not claimed: no page prints a value to check.
"""
from .mla import (  # noqa: F401
    rms_norm, yarn_get_mscale, softmax_scale, rope_inv_freq, rope_cos_sin,
    rotate_half, apply_rope, causal_varlen_attention, mla_prefill, mla_prefill_rows,
    kv_latent, gather_paged, decode_naive, decode_absorbed, prefill_latent_absorbed,
    row_rel_error, bf16_excess_error, prefix_causal_attention, mla_prefill_with_prefix,
    apply_rope_interleaved,
)
from .backward import (  # noqa: F401
    attention_backward, attention_core_backward, rms_norm_backward, rope_backward, mla_prefill_backward,
)
from .fp8 import (  # noqa: F401
    e4m3_value, e4m3_encode, cache_inverse_scale, cache_quantize_fp8, cache_dequantize_fp8, decode_absorbed_fp8,
    mx_scale_exponent, mxfp8_quantize, mxfp8_dequantize, q_uproj_rope, q_uproj_rope_mxfp8,
)
