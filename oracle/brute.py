"""Scalar brute force of the MLA prefill layer (test infrastructure only).

Pure-Python loops over Python floats with ``math.fsum`` for every sum, for tiny
shapes (a few tokens, one or two heads, widths of a few elements).  It shares no
code with ``oracle.mla``: it re-derives each step from the pages' statement of
the layer so that the two agree only if both follow the same definitions.
Plain RoPE and the unrotated (NoPE) variant only.
"""
from __future__ import annotations

import math
from typing import List


def _mv(W, v) -> List[float]:
    """y_i = sum_j W[i][j] v[j] (nn.Linear without bias)."""
    return [math.fsum(W[i][j] * v[j] for j in range(len(v))) for i in range(len(W))]


def _rms(v, g, eps) -> List[float]:
    ms = math.fsum(a * a for a in v) / len(v)
    inv = 1.0 / math.sqrt(ms + eps)
    return [g[i] * v[i] * inv for i in range(len(v))]


def _rope(v, pos, theta) -> List[float]:
    """Rotate pair (i, i + d/2) by pos * theta^(-2i/d)."""
    d = len(v)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = v[i] * c - v[i + h] * s
        out[i + h] = v[i + h] * c + v[i] * s
    return out


def _lst(a):
    return [list(map(float, r)) for r in a] if hasattr(a[0], "__len__") else list(map(float, a))


def prefill(shape, w, x, cu_seqlens):
    """Return out[N][hidden] as nested lists."""
    H, nope, dr, dv = shape.num_heads, shape.qk_nope_dim, shape.qk_rope_dim, shape.v_head_dim
    r = shape.kv_lora_rank
    dqk = nope + dr
    eps = shape.norm_eps
    X = _lst(x)
    n = len(X)
    Wkva, Wkvb, Wo = _lst(w["w_kv_a"]), _lst(w["w_kv_b"]), _lst(w["w_o"])
    gkv = _lst(w["kv_a_gamma"])
    use_rope = shape.rope.kind != "none"
    theta = shape.rope.theta
    sc = dqk ** -0.5
    if shape.rope.kind == "yarn":
        raise NotImplementedError("brute force covers plain RoPE and NoPE only")
    cu = [int(c) for c in cu_seqlens]
    pos = [0] * n
    for d in range(len(cu) - 1):
        for t in range(cu[d], cu[d + 1]):
            pos[t] = t - cu[d]
    # per token: queries, shared key part, per-head keys and values
    Q, KPE, KN, V = [], [], [], []
    for t in range(n):
        if shape.q_lora_rank > 0:
            ql = _rms(_mv(_lst(w["w_q_a"]), X[t]), _lst(w["q_a_gamma"]), eps)
            qt = _mv(_lst(w["w_q_b"]), ql)
        else:
            qt = _mv(_lst(w["w_q"]), X[t])
        ckv = _mv(Wkva, X[t])
        cn = _rms(ckv[:r], gkv, eps)
        kpe = ckv[r:]
        if use_rope:
            kpe = _rope(kpe, pos[t], theta)
        kvt = _mv(Wkvb, cn)
        qh, knh, vh = [], [], []
        for h in range(H):
            qq = qt[h * dqk:(h + 1) * dqk]
            qn, qp = qq[:nope], qq[nope:]
            if use_rope:
                qp = _rope(qp, pos[t], theta)
            qh.append(qn + qp)
            kk = kvt[h * (nope + dv):(h + 1) * (nope + dv)]
            knh.append(kk[:nope])
            vh.append(kk[nope:])
        Q.append(qh)
        KPE.append(kpe)
        KN.append(knh)
        V.append(vh)
    out = []
    for d in range(len(cu) - 1):
        for t in range(cu[d], cu[d + 1]):
            merged = []
            for h in range(H):
                keys = range(cu[d], t + 1)
                sco = [sc * math.fsum(a * b for a, b in zip(Q[t][h], KN[j][h] + KPE[j])) for j in keys]
                m = max(sco)
                e = [math.exp(s - m) for s in sco]
                z = math.fsum(e)
                merged += [math.fsum(e[i] * V[j][h][c] for i, j in enumerate(keys)) / z for c in range(dv)]
            if shape.output_gate:
                g = _mv(_lst(w["w_g"]), X[t])
                merged = [merged[i] / (1.0 + math.exp(-g[i])) for i in range(len(merged))]
            out.append(_mv(Wo, merged))
    return out
