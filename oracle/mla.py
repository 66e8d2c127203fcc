"""Float64 NumPy oracle of the MLA forward pass (test infrastructure only).

Plain, slow, unblocked.  No intermediate rounding: inputs are the bf16-valued
float32 arrays from ``mla_inputs`` promoted to float64, every step runs in
float64, outputs are returned unrounded.  Library primitives used as steps:
``numpy.matmul``/``einsum`` (plain contractions) and ``numpy.exp``.

Notation: N tokens, H heads, d_nope / d_rope / d_v head widths, d_qk = d_nope +
d_rope, r_q / r_kv the query / key-value latent ranks.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------
def rms_norm(x, gamma, eps: float):
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).

    Follows "Kimi-K3 atlas: Gated MLA" (rmsnorm excerpt: one gain per feature,
    computed in float32 there, float64 here) and "MiniMind: attention forward
    pass" section 3 (x * rsqrt(mean(x^2) + eps), then the gain).  With unit
    gains, as in every workload here, the two orders of gain and cast agree.

    Pinned by: closed form for a constant vector, the output mean-square
    identity ms/(ms+eps), and the scalar brute force.
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(gamma) * (x / np.sqrt(ms + eps))


# ----------------------------------------------------------------------------
# YaRN and RoPE
# ----------------------------------------------------------------------------
def yarn_get_mscale(scale: float, mscale: float) -> float:
    """YaRN attention factor.

    "CSDN walkthrough of HF DeepseekV3Attention" (``__init__``) multiplies the
    softmax scaling by mscale twice, citing equations 21-22 of the YaRN paper;
    "Megatron-LM MLA guide" (MLA overview / softmax scale) states
    softmax_scale = mscale * mscale / sqrt(q_head_dim).  The pages do not print
    the function; the YaRN paper's form is 0.1 * m * ln(s) + 1 for s > 1, and
    1 otherwise.  Pinned: s <= 1 gives 1, m = 0 gives 1, and the values this
    form gives at the DeepSeek-V3 shape (1.3688879454113936 for s = 40, m = 1;
    softmax scale 0.1352337788608801), which a base-10 logarithm, a single
    factor or the rope-side mscale would miss.  The 0.1 itself is the paper's
    constant; no page prints it.
    """
    if scale <= 1.0:
        return 1.0
    return 0.1 * mscale * math.log(scale) + 1.0


def softmax_scale(shape) -> float:
    """Softmax scale: q_head_dim^-0.5, times mscale^2 when the YaRN rope config
    has a non-zero mscale_all_dim ("CSDN walkthrough of HF DeepseekV3Attention",
    ``__init__``; "Kimi-K3 atlas" mla-init uses q_head_dim^-0.5 alone)."""
    s = float(shape.qk_head_dim) ** -0.5
    r = shape.rope
    if r.kind == "yarn" and r.mscale_all_dim:
        m = yarn_get_mscale(r.factor, r.mscale_all_dim)
        s = s * m * m
    return s


def rope_inv_freq(d_rope: int, rope) -> np.ndarray:
    """Per-pair rotation frequencies theta_i, i < d_rope/2.

    Plain RoPE: theta_i = base^(-2i/d_rope).  YaRN ("Megatron-LM MLA guide",
    normalization and position-encoding parameters: rotary_base, scaling factor
    s, original_max_position_embeddings L, beta_fast, beta_slow): the
    NTK-by-parts blend of the YaRN paper.  A pair that turns b times over L has
    index i(b) = d_rope * ln(L / (2 pi b)) / (2 ln base); pairs below
    floor(i(beta_fast)) keep theta_i, pairs above ceil(i(beta_slow)) use
    theta_i / s, and a linear ramp in i blends the two in between.

    Pinned by: factor 1 reduces to plain RoPE; pairs whose wavelength is shorter
    than L / beta_fast are unchanged, pairs whose wavelength is longer than
    L / beta_slow are divided by s exactly; the blend is monotone.
    """
    half = d_rope // 2
    i = np.arange(half, dtype=F64)
    base = float(rope.theta)
    inv = base ** (-2.0 * i / d_rope)
    if rope.kind != "yarn":
        return inv
    s = float(rope.factor)
    L = float(rope.original_max_pos)

    def corr_index(b):
        return d_rope * math.log(L / (b * 2.0 * math.pi)) / (2.0 * math.log(base))

    low = max(math.floor(corr_index(rope.beta_fast)), 0)
    high = min(math.ceil(corr_index(rope.beta_slow)), d_rope - 1)
    if low == high:
        high = high + 0.001
    gamma = np.clip((i - low) / (high - low), 0.0, 1.0)   # 0: keep, 1: interpolate
    return inv * (1.0 - gamma) + (inv / s) * gamma


def rope_cos_sin(positions, d_rope: int, rope):
    """cos / sin of position * theta_i, shape [P, d_rope/2], float64.

    The table holds each frequency once; ``apply_rope`` uses it for both halves
    of the rotated slice, which is the duplicated-halves [T, d] table of
    "MiniMind: attention forward pass" section 3.  For YaRN the amplitude is
    mscale(s, mscale) / mscale(s, mscale_all_dim), which is 1 whenever the two
    parameters are equal (reading; not printed on the pages).
    """
    p = np.asarray(positions, dtype=F64)[:, None]
    ang = p * rope_inv_freq(d_rope, rope)[None, :]
    amp = 1.0
    if rope.kind == "yarn":
        amp = yarn_get_mscale(rope.factor, rope.mscale) / yarn_get_mscale(rope.factor, rope.mscale_all_dim)
    return np.cos(ang) * amp, np.sin(ang) * amp


def rotate_half(x):
    """[-x2, x1] for x = [x1, x2] split in halves along the last axis
    ("MiniMind: attention forward pass" section 3)."""
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def apply_rope(x, cos, sin):
    """x * cos + rotate_half(x) * sin with the half-width table duplicated over
    both halves.  ``cos``/``sin`` broadcast against x[..., :d/2].

    Pinned by: position 0 is the identity; norms are preserved; scores depend
    only on relative position; a basis vector maps to (cos, sin) at the
    documented indices."""
    x = _f64(x)
    c = np.concatenate([cos, cos], axis=-1)
    s = np.concatenate([sin, sin], axis=-1)
    return x * c + rotate_half(x) * s


def apply_rope_interleaved(x, cos, sin):
    """RoPE on interleaved pairs: features (2i, 2i+1) rotate together by
    position * theta_i, results in place.  The "CSDN walkthrough of HF
    DeepseekV3Attention" (``forward``) branches on ``rope_interleave`` to a
    variant, for weights whose rope features come in interleaved pairs, that
    it does not print; this is the
    reading taken (pairing only, layout kept).

    Pinned by: equal to ``apply_rope`` on the features regrouped from
    interleaved to half-split order (and back); the layer with interleaved
    pairs equals the layer with rotate_half pairs and the rope rows of the
    query and key weights regrouped the same way."""
    x = _f64(x)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * cos - x1 * sin
    y[..., 1::2] = x1 * cos + x0 * sin
    return y


def _rope(shape, x, cos, sin):
    """The layer's RoPE: interleaved pairs when the shape asks for them."""
    if getattr(shape, "rope_interleave", False):
        return apply_rope_interleaved(x, cos, sin)
    return apply_rope(x, cos, sin)


def _out_proj(shape, w, A2):
    """Output projection of the attention rows A2 [N, H d_v].  Plain: A2 W_o^T.
    Grouped low rank ("Megatron-LM MLA guide", output_projection_groups and
    output_projection_lora_rank, the grouped low-rank output projection wo_a;
    the page gives only these two settings, so the rest is a reading): the
    H d_v features split into G consecutive groups, group g projected to
    rank r_o by its own block of W_o_a ([G r_o, H d_v / G], rows g r_o ..),
    the G results concatenated and projected to hidden by W_o_b
    ([hidden, G r_o]).

    Pinned by: equal to a plain projection with W_o = W_o_b blockdiag(W_o_a)."""
    G = getattr(shape, "o_groups", 0)
    if not G:
        return A2 @ _f64(w["w_o"]).T
    r = shape.o_lora_rank
    n, f = A2.shape
    fg = f // G
    Wa = _f64(w["w_o_a"]).reshape(G, r, fg)
    t = np.concatenate([A2[:, g * fg:(g + 1) * fg] @ Wa[g].T for g in range(G)], axis=1)
    return t @ _f64(w["w_o_b"]).T


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------
def _softmax_rows(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_varlen_attention(q, k, v, scale: float, cu_seqlens, rows: Optional[Sequence[int]] = None):
    """Scaled-dot-product attention, causal within each packed document.

    q [N, H, d_qk], k [N, H, d_qk], v [N, H, d_v] -> [N, H, d_v] (or [len(rows),
    H, d_v]).  Scores scale * q.k, -inf for keys after the query or in another
    document, softmax over keys, weighted sum of v ("MiniMind: attention forward
    pass" section 5; "Megatron-LM MLA guide", THD packing).  No padding of v:
    d_v may differ from d_qk.

    Pinned by: a one-token document returns its own v; zero queries return the
    causal prefix mean; per-document runs equal the packed run; torch's
    scaled_dot_product_attention in float64; the scalar brute force.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n, h, _ = q.shape
    if rows is None:
        out = np.empty((n, h, v.shape[-1]), dtype=F64)
        for d in range(len(cu) - 1):
            a, b = int(cu[d]), int(cu[d + 1])
            if b == a:
                continue
            qd = np.transpose(q[a:b], (1, 0, 2))             # [H, L, dqk]
            kd = np.transpose(k[a:b], (1, 2, 0))             # [H, dqk, L]
            vd = np.transpose(v[a:b], (1, 0, 2))             # [H, L, dv]
            s = scale * np.matmul(qd, kd)                     # [H, L, L]
            L = b - a
            mask = np.triu(np.ones((L, L), dtype=bool), k=1)
            s[:, mask] = -np.inf
            p = _softmax_rows(s)
            out[a:b] = np.transpose(np.matmul(p, vd), (1, 0, 2))
        return out
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), h, v.shape[-1]), dtype=F64)
    doc = np.searchsorted(cu, rows, side="right") - 1
    for r, (t, d) in enumerate(zip(rows, doc)):
        a = int(cu[d])
        s = scale * np.einsum("hd,lhd->hl", q[t], k[a: t + 1])
        p = _softmax_rows(s)
        out[r] = np.einsum("hl,lhd->hd", p, v[a: t + 1])
    return out


# ----------------------------------------------------------------------------
# Prefill layer
# ----------------------------------------------------------------------------
def _positions(cu_seqlens, n):
    """0 .. len-1 within each packed document (reading of position_ids)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.empty(n, dtype=np.int64)
    for d in range(len(cu) - 1):
        pos[cu[d]: cu[d + 1]] = np.arange(cu[d + 1] - cu[d])
    return pos


def _q_proj(shape, w, x):
    """Query path: q_b(RMSNorm_q(q_a(x))) with a query latent, else q(x)
    ("kimi_vl.py - KimiVL attention adapter", Q projection; "Megatron-LM MLA
    guide", --q-lora-rank None means no query compression)."""
    if shape.q_lora_rank > 0:
        lat = x @ _f64(w["w_q_a"]).T
        lat = rms_norm(lat, w["q_a_gamma"], shape.norm_eps)
        return lat @ _f64(w["w_q_b"]).T
    return x @ _f64(w["w_q"]).T


def kv_latent(shape, w, x, positions):
    """Joint down-projection, latent RMSNorm and the shared rope key.

    [c | k_pe] = x W_kv_a^T ("CSDN walkthrough of HF DeepseekV3Attention",
    forward: kv_a_proj_with_mqa and the split); c_n = RMSNorm_kv(c); k_pe is one
    head, rotated with RoPE at each token's position unless the rope kind is
    "none" (Kimi-K3 atlas: the 64 shared key features are not rotated).
    Returns [N, r_kv + d_rope] = [c_n | k_pe'], the per-token latent-cache row
    ("Megatron-LM MLA guide", inference section: the cache keeps the compressed
    kv and the positional key instead of full keys and values)."""
    x = _f64(x)
    ckv = x @ _f64(w["w_kv_a"]).T
    r = shape.kv_lora_rank
    c, k_pe = ckv[:, :r], ckv[:, r:]
    c_n = rms_norm(c, w["kv_a_gamma"], shape.norm_eps)
    if shape.rope.kind != "none":
        cos, sin = rope_cos_sin(positions, shape.qk_rope_dim, shape.rope)
        k_pe = _rope(shape, k_pe, cos, sin)
    return np.concatenate([c_n, k_pe], axis=-1)


def _split_kv_b(shape, w_kv_b):
    """kv_b rows viewed head-major as [H, d_nope + d_v, r_kv]: rows of head h
    are [k_nope part | v part] ("kimi_vl.py" KV compression: view as
    [num_heads, nope + v] then split)."""
    h, nope, dv = shape.num_heads, shape.qk_nope_dim, shape.v_head_dim
    W = _f64(w_kv_b).reshape(h, nope + dv, -1)
    return W[:, :nope, :], W[:, nope:, :]


def mla_prefill(shape, w: Dict[str, np.ndarray], x, cu_seqlens) -> Dict[str, np.ndarray]:
    """The full MLA prefill layer on packed documents, float64.

    q -> [N, H, d_qk] split [q_nope | q_pe]; latent row [c_n | k_pe']; kv =
    c_n W_kv_b^T viewed [N, H, d_nope + d_v] split [k_nope | v]; q_pe rotated at
    the token positions (not for rope kind "none"); keys [k_nope_h | k_pe'] with
    the single k_pe broadcast to every head; causal attention per document with
    d_qk != d_v; optional gate A * sigmoid(x W_g^T) ("Kimi-K3 atlas" mla-init:
    full-rank output gate); out = A.reshape(N, H d_v) W_o^T ("MiniMind"
    section 7; "CSDN walkthrough", the end of forward).

    Returns the output and the intermediates the library also materialises.
    """
    x = _f64(x)
    n = x.shape[0]
    H, nope, dr, dv = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim, shape.v_head_dim
    pos = _positions(cu_seqlens, n)
    q = _q_proj(shape, w, x).reshape(n, H, nope + dr)
    lat = kv_latent(shape, w, x, pos)
    c_n, k_pe = lat[:, : shape.kv_lora_rank], lat[:, shape.kv_lora_rank:]
    kv = (c_n @ _f64(w["w_kv_b"]).T).reshape(n, H, nope + dv)
    k_nope, v = kv[..., :nope], kv[..., nope:]
    q_nope, q_pe = q[..., :nope], q[..., nope:]
    if shape.rope.kind != "none":
        cos, sin = rope_cos_sin(pos, dr, shape.rope)
        q_pe = _rope(shape, q_pe, cos[:, None, :], sin[:, None, :])
    qf = np.concatenate([q_nope, q_pe], axis=-1)
    kf = np.concatenate([k_nope, np.broadcast_to(k_pe[:, None, :], (n, H, dr))], axis=-1)
    A = causal_varlen_attention(qf, kf, v, softmax_scale(shape), cu_seqlens)
    A2 = A.reshape(n, H * dv)
    if shape.output_gate:
        g = x @ _f64(w["w_g"]).T
        A2 = A2 * (1.0 / (1.0 + np.exp(-g)))
    out = _out_proj(shape, w, A2)
    return {"out": out, "q": qf, "latent": lat, "kv": kv, "attn": A2, "positions": pos}


def mla_prefill_rows(shape, w, x, cu_seqlens, rows: Sequence[int]) -> Dict[str, np.ndarray]:
    """The same layer evaluated only at the query rows ``rows`` (for full-size
    parity checks): every quantity a row depends on is computed from the same
    definitions as ``mla_prefill``; keys and values are formed for all tokens."""
    x = _f64(x)
    n = x.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    H, nope, dr, dv = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim, shape.v_head_dim
    pos = _positions(cu_seqlens, n)
    q = _q_proj(shape, w, x[rows]).reshape(len(rows), H, nope + dr)
    lat = kv_latent(shape, w, x, pos)
    c_n, k_pe = lat[:, : shape.kv_lora_rank], lat[:, shape.kv_lora_rank:]
    kv = (c_n @ _f64(w["w_kv_b"]).T).reshape(n, H, nope + dv)
    k_nope, v = kv[..., :nope], kv[..., nope:]
    q_nope, q_pe = q[..., :nope], q[..., nope:]
    if shape.rope.kind != "none":
        cos, sin = rope_cos_sin(pos[rows], dr, shape.rope)
        q_pe = _rope(shape, q_pe, cos[:, None, :], sin[:, None, :])
    qf = np.empty((n, H, nope + dr), dtype=F64)
    qf[rows] = np.concatenate([q_nope, q_pe], axis=-1)
    kf = np.concatenate([k_nope, np.broadcast_to(k_pe[:, None, :], (n, H, dr))], axis=-1)
    A = causal_varlen_attention(qf, kf, v, softmax_scale(shape), cu_seqlens, rows=rows)
    A2 = A.reshape(len(rows), H * dv)
    if shape.output_gate:
        g = x[rows] @ _f64(w["w_g"]).T
        A2 = A2 * (1.0 / (1.0 + np.exp(-g)))
    out = _out_proj(shape, w, A2)
    return {"out": out, "attn": A2, "latent": lat, "q": qf[rows], "kv": kv}


def prefill_latent_absorbed(shape, w_kv_b, q, latent, cu_seqlens):
    """Attention computed entirely in the latent space (the absorbed form of
    "Megatron-LM MLA guide", inference section: up_k folded into the query,
    up_v applied after attention), for packed causal documents.

    q [N, H, d_qk] (q_pe already rotated), latent [N, r_kv + d_rope].
    Returns A [N, H, d_v].  An independent formulation used to pin
    ``mla_prefill``: it never forms per-head keys or values."""
    q, latent = _f64(q), _f64(latent)
    W_uk, W_uv = _split_kv_b(shape, w_kv_b)          # [H, nope, r], [H, dv, r]
    nope, r = shape.qk_nope_dim, shape.kv_lora_rank
    qt = np.einsum("thd,hdc->thc", q[..., :nope], W_uk)   # [N, H, r]
    c, kpe = latent[:, :r], latent[:, r:]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n, H = q.shape[0], q.shape[1]
    out = np.empty((n, H, shape.v_head_dim), dtype=F64)
    sc = softmax_scale(shape)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        for t in range(a, b):
            s = sc * (qt[t] @ c[a: t + 1].T + q[t, :, nope:] @ kpe[a: t + 1].T)   # [H, L]
            p = _softmax_rows(s)
            o_lat = p @ c[a: t + 1]                                            # [H, r]
            out[t] = np.einsum("hvc,hc->hv", W_uv, o_lat)
    return out


# ----------------------------------------------------------------------------
# Decode over the paged latent cache
# ----------------------------------------------------------------------------
def gather_paged(cache, block_table, b: int, length: int, block_size: int):
    """Rows 0..length-1 of sequence b: slot(j) = block_table[b, j // bs] * bs +
    j % bs in the pool viewed as [n_blocks * bs, width]."""
    cache = np.asarray(cache)
    flat = cache.reshape(-1, cache.shape[-1])
    j = np.arange(length)
    slots = np.asarray(block_table)[b, j // block_size].astype(np.int64) * block_size + j % block_size
    return _f64(flat[slots])


def decode_naive(shape, w_kv_b, q_nope, q_pe, cache, block_table, seq_lens, block_size: int, batch_idx=None):
    """Non-absorbed decode: decompress every cached latent row into per-head
    k_nope and v with W_kv_b, form keys [k_nope | k_pe'] and attend with the one
    new query, which sees every cached key including its own ("MiniMind"
    section 5: with a cache, a single query is masked nowhere).  Returns
    [B, H, d_v]."""
    H, nope, dv, r = shape.num_heads, shape.qk_nope_dim, shape.v_head_dim, shape.kv_lora_rank
    W = _f64(w_kv_b)
    sc = softmax_scale(shape)
    bs = range(len(seq_lens)) if batch_idx is None else batch_idx
    out = np.empty((len(list(bs)), H, dv), dtype=F64)
    for o, b in enumerate(bs):
        C = gather_paged(cache, block_table, b, int(seq_lens[b]), block_size)
        kv = (C[:, :r] @ W.T).reshape(-1, H, nope + dv)
        k = np.concatenate([kv[..., :nope], np.broadcast_to(C[:, None, r:], (C.shape[0], H, C.shape[1] - r))], -1)
        qv = np.concatenate([_f64(q_nope[b]), _f64(q_pe[b])], -1)   # [H, dqk]
        s = sc * np.einsum("hd,lhd->hl", qv, k)
        p = _softmax_rows(s)
        out[o] = np.einsum("hl,lhd->hd", p, kv[..., nope:])
    return out


def decode_absorbed(shape, w_kv_b, q_nope, q_pe, cache, block_table, seq_lens, block_size: int, batch_idx=None,
                    return_latent: bool = False):
    """Absorbed decode ("Megatron-LM MLA guide", inference section: the kv
    up-projection is split by head into up_k and up_v; up_k is folded into the
    no-position query, attention runs over the cached latents, up_v restores
    d_v afterwards).  q~ = W_UK[h]^T q_nope; s = scale (q~.c + q_pe.k_pe');
    o_lat = sum_j p_j c_j; out = W_UV[h] o_lat.  Returns [B, H, d_v] (and the
    normalised o_lat [B, H, r_kv] when asked)."""
    r = shape.kv_lora_rank
    W_uk, W_uv = _split_kv_b(shape, w_kv_b)
    sc = softmax_scale(shape)
    bs = list(range(len(seq_lens))) if batch_idx is None else list(batch_idx)
    out = np.empty((len(bs), shape.num_heads, shape.v_head_dim), dtype=F64)
    lat = np.empty((len(bs), shape.num_heads, r), dtype=F64)
    for o, b in enumerate(bs):
        C = gather_paged(cache, block_table, b, int(seq_lens[b]), block_size)
        qt = np.einsum("hd,hdc->hc", _f64(q_nope[b]), W_uk)          # [H, r]
        s = sc * (qt @ C[:, :r].T + _f64(q_pe[b]) @ C[:, r:].T)        # [H, L]
        p = _softmax_rows(s)
        lat[o] = p @ C[:, :r]
        out[o] = np.einsum("hvc,hc->hv", W_uv, lat[o])
    return (out, lat) if return_latent else out


# ----------------------------------------------------------------------------
# Prefill of a new chunk over a cached prefix
# ----------------------------------------------------------------------------
def prefix_causal_attention(q, k, v, scale: float, prefix: int, rows: Optional[Sequence[int]] = None):
    """Attention of T new queries over P cached + T new keys of one sequence.

    q [T, H, d_qk], k [P + T, H, d_qk], v [P + T, H, d_v] -> [T, H, d_v].
    With ``rows``, q holds only the queries rows[0], rows[1], ... (indices in
    0 .. T-1) and the result has len(rows) rows.  Query i stands at
    position P + i; it sees every cached key and the new keys up to itself:
    keys j <= P + i.  This is the causal mask of "MiniMind: attention forward
    pass" section 5 for a forward with a cache: the upper triangle is masked
    only inside the last T x T block of the score matrix, every column of the
    history stays visible, and a single query (T = 1) is masked nowhere.

    Pinned by: P = 0 equals ``causal_varlen_attention``; a full causal run
    over P + T tokens restricted to its last T rows equals this with the first
    P keys as the prefix; T = 1 equals the non-absorbed decode.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    t = k.shape[0] - prefix
    sel = np.arange(t) if rows is None else np.asarray(rows, dtype=np.int64)
    assert q.shape[0] == len(sel) and v.shape[0] == k.shape[0] and np.all((sel >= 0) & (sel < t))
    out = np.empty((len(sel), q.shape[1], v.shape[-1]), dtype=F64)
    for r, i in enumerate(sel):
        last = prefix + int(i)                                   # last visible key
        s = scale * np.einsum("hd,lhd->hl", q[r], k[: last + 1])
        p = _softmax_rows(s)
        out[r] = np.einsum("hl,lhd->hd", p, v[: last + 1])
    return out


def mla_prefill_with_prefix(shape, w: Dict[str, np.ndarray], x, cu_seqlens, prefix_lens, cache, block_table,
                            block_size: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """The MLA layer for new tokens of sequences whose first tokens are
    already in the paged latent cache (chunked prefill, mixed prefill/decode).

    x [N, hidden] holds the new tokens packed by ``cu_seqlens``; sequence s
    has ``prefix_lens[s]`` = P_s cached tokens, read from the pool ``cache``
    [n_blocks, block_size, r_kv + d_rope] through ``block_table`` (rows
    [c_n | k_pe'] as the decode path stores them).  New token i of s stands at
    position P_s + i (its q_pe and k_pe are rotated there).  The cached
    latents are decompressed with the same kv up-projection as the new
    tokens' ("Megatron-LM MLA guide", inference section: prefill and mixed
    steps decompress k/v from the cached latents, only decode-only steps use
    the absorbed form), keys [k_nope_h | k_pe'] over P_s + T_s tokens, and
    query i attends to keys 0 .. P_s + i (``prefix_causal_attention``).  Gate
    and output projection as in ``mla_prefill``.

    ``rows`` restricts the returned query rows (global indices into x).
    Returns the output, the new tokens' latent rows and the attention result.
    """
    x = _f64(x)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pre = np.asarray(prefix_lens, dtype=np.int64)
    n = x.shape[0]
    H, nope, dr, dv, r = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim, shape.v_head_dim, shape.kv_lora_rank
    pos = np.empty(n, dtype=np.int64)
    for d in range(len(cu) - 1):
        pos[cu[d]: cu[d + 1]] = pre[d] + np.arange(cu[d + 1] - cu[d])
    sel = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    lat = kv_latent(shape, w, x, pos)                                  # new tokens' cache rows
    q = _q_proj(shape, w, x[sel]).reshape(len(sel), H, nope + dr)
    q_nope, q_pe = q[..., :nope], q[..., nope:]
    if shape.rope.kind != "none":
        cos, sin = rope_cos_sin(pos[sel], dr, shape.rope)
        q_pe = _rope(shape, q_pe, cos[:, None, :], sin[:, None, :])
    qf = np.concatenate([q_nope, q_pe], axis=-1)
    W = _f64(w["w_kv_b"])
    sc = softmax_scale(shape)
    A = np.empty((len(sel), H, dv), dtype=F64)
    doc = np.searchsorted(cu, sel, side="right") - 1
    for d in range(len(cu) - 1):
        mine = np.nonzero(doc == d)[0]
        if len(mine) == 0:
            continue
        a, b = int(cu[d]), int(cu[d + 1])
        ctx = np.concatenate([gather_paged(cache, block_table, d, int(pre[d]), block_size), lat[a:b]], axis=0)
        kv = (ctx[:, :r] @ W.T).reshape(-1, H, nope + dv)
        k = np.concatenate([kv[..., :nope], np.broadcast_to(ctx[:, None, r:], (ctx.shape[0], H, dr))], axis=-1)
        A[mine] = prefix_causal_attention(qf[mine], k, kv[..., nope:], sc, int(pre[d]), rows=sel[mine] - a)
    A2 = A.reshape(len(sel), H * dv)
    if shape.output_gate:
        g = x[sel] @ _f64(w["w_g"]).T
        A2 = A2 * (1.0 / (1.0 + np.exp(-g)))
    out = _out_proj(shape, w, A2)
    return {"out": out, "attn": A2, "latent": lat, "q": qf, "positions": pos}


# ----------------------------------------------------------------------------
# Comparison metric
# ----------------------------------------------------------------------------
def bf16_excess_error(ref, got, rtol: float = 2.0 ** -8) -> float:
    """max over rows of max_k (|got - ref| - rtol |ref|)_+ / RMS_k(ref): the
    error left after allowing, at each element, the rounding of a correctly
    rounded bfloat16 result (half an ulp, at most 2^-8 of |ref|).  A result
    within atol * RMS(row) + rtol * |ref| everywhere scores <= atol; the exact
    answer rounded to bfloat16 scores 0.  NaN anywhere in ``got`` gives inf."""
    ref = _f64(ref).reshape(-1, np.shape(ref)[-1])
    got = _f64(got).reshape(ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    rms = np.where(rms > 0, rms, 1.0)
    ex = np.maximum(np.abs(got - ref) - rtol * np.abs(ref), 0.0)
    return float(np.max(np.max(ex, axis=-1) / rms))


def row_rel_error(ref, got) -> float:
    """max over rows of max_k |got - ref| / RMS_k(ref), rows = last axis.
    NaN anywhere in ``got`` gives inf."""
    ref = _f64(ref).reshape(-1, np.shape(ref)[-1])
    got = _f64(got).reshape(ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    rms = np.where(rms > 0, rms, 1.0)
    return float(np.max(np.max(np.abs(got - ref), axis=-1) / rms))
