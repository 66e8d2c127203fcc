"""Backward of the MLA prefill layer, float64.  TEST INFRASTRUCTURE ONLY (see
the package header).

"Megatron-LM MLA guide" (training section) trains the MLA layer end to end:
gradients flow to every projection (``backward_dw`` for the KV, Q and output
projections), through the latent norms and RoPE, and through the attention
to the query, the per-head k_nope / v from the latent, and the one shared
k_pe.  The pages print no backward formulas; the backward here is the chain
rule applied to the forward of ``oracle.mla`` step by step, in reverse:

* attention (per head, causal within each document), with S = scale q k^T,
  P = softmax_rows(S), O = P v:
  dv = P^T dO, dP = dO v^T, D = rowsum(dO * O), dS = P * (dP - D),
  dq = scale dS k, dk = scale dS^T q; the shared k_pe's gradient is the sum
  of its per-head key gradients;
* RoPE is a rotation per pair, so its backward is the rotation by -theta;
* RMSNorm y = g x / r, r = sqrt(mean(x^2) + eps):
  dg = sum_rows dy x / r, dx = (g dy) / r - x mean(g dy x) / r^3;
* a projection y = x W^T: dx = dy W, dW = dy^T x; the gate
  A2 = A sigmoid(g): dA = dA2 sigmoid(g), dg = dA2 A sigmoid(g) (1 - sigmoid(g)).

Parity: pinned by central finite differences of L = sum(dout * out) for
sampled entries of every input and weight (float64, several layer variants),
and by planted mistakes (the D term dropped, the scale left out of dq, RoPE
undone with +theta, the shared k_pe gradient taken from one head, the
RMSNorm mean term dropped) that the finite differences catch.
"""
from typing import Dict, Optional

import numpy as np

from .mla import (_f64, _out_proj, _positions, _rope, _softmax_rows, rms_norm, rope_cos_sin, softmax_scale)


def attention_backward(q, k, v, scale: float, cu_seqlens, dout, out=None):
    """(dq, dk, dv, lse) of ``causal_varlen_attention(q, k, v, scale, cu)``
    for the output gradient dout [N, H, d_v]; k is per head here.  lse is the
    natural-log log-sum-exp of each (row, head)'s scaled scores.

    ``out`` is the forward output as handed to the backward (for instance
    stored in bf16 by the forward); D = rowsum(dout * out) is formed from it.
    None recomputes it exactly, giving the true gradient."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    out = None if out is None else _f64(out)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n, h, _ = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    lse = np.zeros((n, h))
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        if b == a:
            continue
        L = b - a
        qd = np.transpose(q[a:b], (1, 0, 2))             # [H, L, dqk]
        kd = np.transpose(k[a:b], (1, 0, 2))
        vd = np.transpose(v[a:b], (1, 0, 2))             # [H, L, dv]
        gd = np.transpose(dout[a:b], (1, 0, 2))
        s = scale * np.matmul(qd, np.transpose(kd, (0, 2, 1)))
        mask = np.triu(np.ones((L, L), dtype=bool), k=1)
        s[:, mask] = -np.inf
        m = np.max(s, axis=-1, keepdims=True)
        lse[a:b] = np.transpose((m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0])
        p = _softmax_rows(s)
        o = np.matmul(p, vd)
        dvd = np.matmul(np.transpose(p, (0, 2, 1)), gd)
        dp = np.matmul(gd, np.transpose(vd, (0, 2, 1)))
        if out is not None:
            o = np.transpose(out[a:b], (1, 0, 2))
        D = np.sum(gd * o, axis=-1, keepdims=True)
        ds = p * (dp - D)
        dq[a:b] = np.transpose(scale * np.matmul(ds, kd), (1, 0, 2))
        dk[a:b] = np.transpose(scale * np.matmul(np.transpose(ds, (0, 2, 1)), qd), (1, 0, 2))
        dv[a:b] = np.transpose(dvd, (1, 0, 2))
    return dq, dk, dv, lse


def rms_norm_backward(x, gamma, eps: float, dy):
    """(dx, dgamma) of ``rms_norm(x, gamma, eps)``."""
    x, g, dy = _f64(x), _f64(gamma), _f64(dy)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gdy = g * dy
    dx = gdy / r - x * np.mean(gdy * x, axis=-1, keepdims=True) / r ** 3
    dg = np.sum(dy * x / r, axis=tuple(range(x.ndim - 1)))
    return dx, dg


def rope_backward(shape, dy, cos, sin):
    """Gradient through the layer's RoPE: the rotation by -theta."""
    return _rope(shape, dy, cos, -sin)


def mla_prefill_backward(shape, w: Dict[str, np.ndarray], x, cu_seqlens, dout) -> Dict[str, np.ndarray]:
    """Gradients of sum(dout * mla_prefill(shape, w, x, cu)["out"]) with
    respect to x and every weight the layer uses (keys as in ``w``).  The
    forward is recomputed step by step, from the same definitions as
    ``oracle.mla.mla_prefill``."""
    x, dout = _f64(x), _f64(dout)
    n = x.shape[0]
    H, nope, dr, dv, r = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim, shape.v_head_dim, shape.kv_lora_rank
    dqk = nope + dr
    rope = shape.rope.kind != "none"
    pos = _positions(cu_seqlens, n)
    if rope:
        cos, sin = rope_cos_sin(pos, dr, shape.rope)
    W = {k_: _f64(v_) for k_, v_ in w.items() if v_ is not None}
    grads: Dict[str, np.ndarray] = {}

    # ---- forward, keeping what the backward needs
    if shape.q_lora_rank > 0:
        q_lat = x @ W["w_q_a"].T
        q_lat_n = rms_norm(q_lat, W["q_a_gamma"], shape.norm_eps)
        q = (q_lat_n @ W["w_q_b"].T).reshape(n, H, dqk)
    else:
        q = (x @ W["w_q"].T).reshape(n, H, dqk)
    ckv = x @ W["w_kv_a"].T
    c, k_pe_raw = ckv[:, :r], ckv[:, r:]
    c_n = rms_norm(c, W["kv_a_gamma"], shape.norm_eps)
    k_pe = _rope(shape, k_pe_raw, cos, sin) if rope else k_pe_raw
    kv = (c_n @ W["w_kv_b"].T).reshape(n, H, nope + dv)
    k_nope, v = kv[..., :nope], kv[..., nope:]
    q_pe = _rope(shape, q[..., nope:], cos[:, None, :], sin[:, None, :]) if rope else q[..., nope:]
    qf = np.concatenate([q[..., :nope], q_pe], axis=-1)
    kf = np.concatenate([k_nope, np.broadcast_to(k_pe[:, None, :], (n, H, dr))], axis=-1)
    sc = softmax_scale(shape)
    from .mla import causal_varlen_attention
    A = causal_varlen_attention(qf, kf, v, sc, cu_seqlens)
    A2 = A.reshape(n, H * dv)
    gate = None
    if shape.output_gate:
        gpre = x @ W["w_g"].T
        gate = 1.0 / (1.0 + np.exp(-gpre))
        A2g = A2 * gate
    else:
        A2g = A2

    # ---- output projection
    G = getattr(shape, "o_groups", 0)
    if not G:
        grads["w_o"] = dout.T @ A2g
        dA2g = dout @ W["w_o"]
    else:
        ro = shape.o_lora_rank
        fg = A2g.shape[1] // G
        Wa = W["w_o_a"].reshape(G, ro, fg)
        t = np.concatenate([A2g[:, g * fg:(g + 1) * fg] @ Wa[g].T for g in range(G)], axis=1)
        grads["w_o_b"] = dout.T @ t
        dt = dout @ W["w_o_b"]
        dWa = np.zeros_like(Wa)
        dA2g = np.zeros_like(A2g)
        for g in range(G):
            dtg = dt[:, g * ro:(g + 1) * ro]
            dWa[g] = dtg.T @ A2g[:, g * fg:(g + 1) * fg]
            dA2g[:, g * fg:(g + 1) * fg] = dtg @ Wa[g]
        grads["w_o_a"] = dWa.reshape(W["w_o_a"].shape)
    dx = np.zeros_like(x)
    if gate is not None:
        dA2 = dA2g * gate
        dgpre = dA2g * A2 * gate * (1.0 - gate)
        grads["w_g"] = dgpre.T @ x
        dx += dgpre @ W["w_g"]
    else:
        dA2 = dA2g

    # ---- attention
    dq_f, dk_f, dv_, _ = attention_backward(qf, kf, v, sc, cu_seqlens, dA2.reshape(n, H, dv))
    dq_nope, dq_pe = dq_f[..., :nope], dq_f[..., nope:]
    dk_nope, dk_pe = dk_f[..., :nope], np.sum(dk_f[..., nope:], axis=1)     # the shared key: sum over heads
    if rope:
        dq_pe = rope_backward(shape, dq_pe, cos[:, None, :], sin[:, None, :])
        dk_pe = rope_backward(shape, dk_pe, cos, sin)
    dq = np.concatenate([dq_nope, dq_pe], axis=-1).reshape(n, H * dqk)

    # ---- kv up-projection and latent norm
    dkv = np.concatenate([dk_nope, dv_], axis=-1).reshape(n, H * (nope + dv))
    grads["w_kv_b"] = dkv.T @ c_n
    dc_n = dkv @ W["w_kv_b"]
    dc, grads["kv_a_gamma"] = rms_norm_backward(c, W["kv_a_gamma"], shape.norm_eps, dc_n)
    dckv = np.concatenate([dc, dk_pe], axis=-1)
    grads["w_kv_a"] = dckv.T @ x
    dx += dckv @ W["w_kv_a"]

    # ---- query path
    if shape.q_lora_rank > 0:
        grads["w_q_b"] = dq.T @ q_lat_n
        dq_lat_n = dq @ W["w_q_b"]
        dq_lat, grads["q_a_gamma"] = rms_norm_backward(q_lat, W["q_a_gamma"], shape.norm_eps, dq_lat_n)
        grads["w_q_a"] = dq_lat.T @ x
        dx += dq_lat @ W["w_q_a"]
    else:
        grads["w_q"] = dq.T @ x
        dx += dq @ W["w_q"]
    grads["x"] = dx
    return grads


def attention_core_backward(q, kv, kpe, scale: float, cu_seqlens, dout, nope: int, out=None):
    """Backward of the attention core as the library computes it: q
    [N, H, nope + rope], kv [N, H, nope + d_v] = per head [k_nope | v], kpe
    [N, rope] the one shared key part, ``out`` the forward output the caller
    hands over (None: exact).  Returns (dq [N, H, nope + rope], dkv
    [N, H, nope + d_v], dkpe [N, rope] summed over heads, lse [N, H])."""
    q, kv, kpe = _f64(q), _f64(kv), _f64(kpe)
    n, H, _ = q.shape
    k = np.concatenate([kv[..., :nope], np.broadcast_to(kpe[:, None, :], (n, H, kpe.shape[-1]))], axis=-1)
    dq, dk, dv, lse = attention_backward(q, k, kv[..., nope:], scale, cu_seqlens, dout, out)
    return dq, np.concatenate([dk[..., :nope], dv], axis=-1), np.sum(dk[..., nope:], axis=1), lse
