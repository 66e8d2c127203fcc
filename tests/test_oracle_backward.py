"""Pins of the backward oracle (CPU only): central finite differences of
L = sum(dout * out) in float64 against the analytic gradients, for sampled
entries of every input and weight, on tiny layers of every variant; and
planted mistakes in the backward that the differences catch."""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import backward as ob
from oracle import mla as om

TINY = mi.WORKLOADS["tiny_fp32_t64"]
VARIANTS = {
    "plain_rope_q_lora": TINY,
    "direct_q": TINY.replace(q_lora_rank=0),
    "yarn": TINY.replace(rope=TINY.rope.__class__(kind="yarn", theta=10000.0, factor=40.0, original_max_pos=16,
                                                  beta_fast=32.0, beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0)),
    "nope_gate": TINY.replace(rope=TINY.rope.__class__(kind="none", theta=10000.0, factor=1.0, original_max_pos=0,
                                                       beta_fast=32.0, beta_slow=1.0, mscale=1.0, mscale_all_dim=0.0),
                              output_gate=True),
    "interleaved": TINY.replace(rope_interleave=True),
    "grouped_o": TINY.replace(o_groups=2, o_lora_rank=16),
}


def _case(sh, seed=0):
    case = mi.make_prefill_case(sh, doc_lengths=[7, 12], seed=seed)
    w = {k: (None if v is None else np.asarray(v, np.float64)) for k, v in case.w.items()}
    if sh.q_lora_rank == 0:
        w["w_q_a"] = w["q_a_gamma"] = w["w_q_b"] = None
    # non-unit norm gains, so their gradients are exercised
    rng = np.random.default_rng(seed + 1)
    for g in ("q_a_gamma", "kv_a_gamma"):
        if w.get(g) is not None:
            w[g] = 1.0 + 0.1 * rng.standard_normal(w[g].shape)
    x = np.asarray(case.x, np.float64)
    dout = rng.standard_normal((x.shape[0], sh.hidden))
    return w, x, case.cu_seqlens, dout


def _loss(sh, w, x, cu, dout):
    return float(np.sum(dout * om.mla_prefill(sh, w, x, cu)["out"]))


def _fd_check(sh, w, x, cu, dout, grads, n_samples=6, seed=3):
    """Worst relative gap between sampled finite differences and grads."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    tensors = {"x": x, **{k: v for k, v in w.items() if v is not None}}
    for name, t in tensors.items():
        if name not in grads:
            continue
        assert grads[name].shape == t.shape, name
        flat = t.reshape(-1)
        gflat = grads[name].reshape(-1)
        scale = np.max(np.abs(gflat)) + 1e-30
        for i in rng.choice(flat.size, size=min(n_samples, flat.size), replace=False):
            h = 1e-5 * max(1.0, abs(flat[i]))
            old = flat[i]
            flat[i] = old + h
            lp = _loss(sh, w, x, cu, dout)
            flat[i] = old - h
            lm = _loss(sh, w, x, cu, dout)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            worst = max(worst, abs(fd - gflat[i]) / scale)
    return worst


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_layer_gradients_match_finite_differences(variant):
    sh = VARIANTS[variant]
    w, x, cu, dout = _case(sh)
    grads = ob.mla_prefill_backward(sh, w, x, cu, dout)
    expected = {"x", "w_kv_a", "kv_a_gamma", "w_kv_b"} | ({"w_q_a", "q_a_gamma", "w_q_b"} if sh.q_lora_rank else {"w_q"})
    expected |= {"w_o_a", "w_o_b"} if getattr(sh, "o_groups", 0) else {"w_o"}
    if sh.output_gate:
        expected |= {"w_g"}
    assert expected <= set(grads)
    assert _fd_check(sh, w, x, cu, dout, grads) < 1e-6


def test_attention_core_gradients_match_finite_differences():
    """dq, dkv and the shared dkpe of the core the library computes."""
    rng = np.random.default_rng(5)
    n, H, nope, dr, dv = 19, 3, 8, 4, 6
    cu = np.array([0, 7, 19])
    q, kv, kpe = rng.standard_normal((n, H, nope + dr)), rng.standard_normal((n, H, nope + dv)), rng.standard_normal((n, dr))
    dout = rng.standard_normal((n, H, dv))
    scale = 0.3

    def loss():
        k = np.concatenate([kv[..., :nope], np.broadcast_to(kpe[:, None, :], (n, H, dr))], -1)
        return float(np.sum(dout * om.causal_varlen_attention(q, k, kv[..., nope:], scale, cu)))
    dq, dkv, dkpe, lse = ob.attention_core_backward(q, kv, kpe, scale, cu, dout, nope)
    for t, g in ((q, dq), (kv, dkv), (kpe, dkpe)):
        flat, gf = t.reshape(-1), g.reshape(-1)
        for i in rng.choice(flat.size, 12, replace=False):
            old = flat[i]
            flat[i] = old + 1e-6
            lp = loss()
            flat[i] = old - 1e-6
            lm = loss()
            flat[i] = old
            assert abs((lp - lm) / 2e-6 - gf[i]) < 1e-7 * (1 + np.abs(gf).max())
    # the log-sum-exp of row t of document d over its keys up to t
    k = np.concatenate([kv[..., :nope], np.broadcast_to(kpe[:, None, :], (n, H, dr))], -1)
    s = scale * np.einsum("hd,lhd->hl", q[10], k[7:11])
    assert np.allclose(lse[10], np.log(np.sum(np.exp(s), axis=-1)))


def test_attention_backward_with_given_output_moves_linearly_in_D():
    """The backward formed with a forward output other than the exact one
    (as stored in bf16 by a forward): D = rowsum(dO * out) enters
    dS = P (dP - D) linearly, so with out' = out + delta and
    dD = rowsum(dO * delta): dq' - dq = -scale dD (P k), the forward attention
    with k in place of v; dk' - dk = -scale P^T (dD q), the dv formula with q
    in place of dO's values; dv unchanged."""
    rng = np.random.default_rng(11)
    n, H, dqk, dv_ = 23, 2, 10, 6
    cu = np.array([0, 1, 9, 23])
    q, k, v = rng.standard_normal((n, H, dqk)), rng.standard_normal((n, H, dqk)), rng.standard_normal((n, H, dv_))
    dout = rng.standard_normal((n, H, dv_))
    scale = 0.4
    exact = ob.attention_backward(q, k, v, scale, cu, dout)
    o = om.causal_varlen_attention(q, k, v, scale, cu)
    same = ob.attention_backward(q, k, v, scale, cu, dout, out=o)
    for a, b in zip(exact, same):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    delta = 1e-2 * rng.standard_normal(o.shape)
    dq2, dk2, dv2, _ = ob.attention_backward(q, k, v, scale, cu, dout, out=o + delta)
    dD = np.sum(dout * delta, axis=-1)
    pk = om.causal_varlen_attention(q, k, k, scale, cu)
    assert np.allclose(dq2 - exact[0], -scale * dD[..., None] * pk, rtol=1e-10, atol=1e-12)
    _, _, ptq, _ = ob.attention_backward(q, k, q, scale, cu, dD[..., None] * q)
    assert np.allclose(dk2 - exact[1], -scale * ptq, rtol=1e-10, atol=1e-12)
    assert np.array_equal(dv2, exact[2])


# ----------------------------------------------------------------------------- planted mistakes
def _planted(monkeypatch, which):
    if which == "no_D_term":
        orig = ob.attention_backward

        def bad(q, k, v, scale, cu, dout):
            # dS = P * dP (the rowsum(dO * O) term dropped)
            q, k, v, dout = map(np.asarray, (q, k, v, dout))
            dq, dk, dv, lse = orig(q, k, v, scale, cu, dout)
            o = om.causal_varlen_attention(q, k, v, scale, cu)
            D = np.sum(dout * o, axis=-1)
            # add back the removed contribution: - sum_j P_ij D_i k_j = -D_i * (attention of k)
            ok = om.causal_varlen_attention(q, k, k, scale, cu)
            return dq + scale * D[..., None] * ok, dk, dv, lse
        monkeypatch.setattr(ob, "attention_backward", bad)
    elif which == "dq_unscaled":
        orig = ob.attention_backward

        def bad(q, k, v, scale, cu, dout):
            dq, dk, dv, lse = orig(q, k, v, scale, cu, dout)
            return dq / scale, dk, dv, lse
        monkeypatch.setattr(ob, "attention_backward", bad)
    elif which == "rope_forward_rotation":
        monkeypatch.setattr(ob, "rope_backward", lambda shape, dy, cos, sin: om._rope(shape, dy, cos, sin))
    elif which == "kpe_one_head":
        orig = ob.attention_backward

        def bad(q, k, v, scale, cu, dout):
            dq, dk, dv, lse = orig(q, k, v, scale, cu, dout)
            H = dk.shape[1]
            dk = dk.copy()
            dk[:, 1:, q.shape[-1] - 16:] = 0.0          # only head 0 reaches the shared key (rope = 16)
            return dq, dk, dv, lse
        monkeypatch.setattr(ob, "attention_backward", bad)
    elif which == "norm_no_mean_term":
        def bad(x, gamma, eps, dy):
            x, g, dy = map(lambda a: np.asarray(a, np.float64), (x, gamma, dy))
            r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
            return g * dy / r, np.sum(dy * x / r, axis=0)
        monkeypatch.setattr(ob, "rms_norm_backward", bad)


@pytest.mark.parametrize("which", ["no_D_term", "dq_unscaled", "rope_forward_rotation", "kpe_one_head",
                                   "norm_no_mean_term"])
def test_backward_pins_catch_planted_mistakes(monkeypatch, which):
    sh = VARIANTS["plain_rope_q_lora"]
    w, x, cu, dout = _case(sh)
    _planted(monkeypatch, which)
    grads = ob.mla_prefill_backward(sh, w, x, cu, dout)
    assert _fd_check(sh, w, x, cu, dout, grads, n_samples=10) > 1e-4
