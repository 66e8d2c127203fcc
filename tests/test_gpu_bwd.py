"""GPU parity of the attention-core backward (``mla_attention_prefill_bwd``)
against the float64 oracle (``oracle.backward.attention_core_backward``).

Inputs: seeded N(0, 1) bf16 q, kv, k_pe and output gradient dout; the forward
output passed to the kernel is the oracle's, rounded to bf16, and the oracle
forms D = rowsum(dout * out) from the same bf16 output (a short row with a
large output is badly conditioned in D: the bf16 output alone moves such a
row's exact dq by up to a quarter of its value).

The kernel's gradients are fp32 sums of products of bf16 operands, two of
which it rounds to bf16 itself: P (for dv = P^T dO) and dS (for dq = scale dS k
and dk = scale dS^T q).  With u = 2^-8 (bf16 unit roundoff, round to nearest)
each such product is off by at most u of its magnitude, so element by element
  |dq - ref| <= u scale sum_j |dS_ij| |k_j|,  |dk - ref| <= u scale sum_i |dS_ij| |q_i|,
  |dv - ref| <= u sum_i P_ij |dO_i|,  dk_pe: the sum over heads of dk's bound,
to first order.  The test allows twice that plus 2^-12 of the tensor's RMS for
the fp32 arithmetic (scores, exponentials, dP - D), and prints the largest
error as a fraction of the allowance and of the tensor RMS.
"""
import sys

import numpy as np
import pytest

import mla_inputs as mi
from oracle import backward as ob
from oracle import mla as om

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -8


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


def conditioning(q, k, v, dout, out, scale, cu, lse):
    """Per element: scale sum_j |dS_ij| |k_j| (dq), scale sum_i |dS_ij| |q_i|
    (dk) and sum_i P_ij |dO_i| (dv), with P from the oracle's lse and D from
    the given output; one head of one document at a time."""
    cq, ck, cv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for d in range(len(cu) - 1):
        a, b = int(cu[d]), int(cu[d + 1])
        causal = np.tril(np.ones((b - a, b - a), dtype=bool))
        for h in range(q.shape[1]):
            qh, kh, vh, gh = (x[a:b, h].astype(np.float64) for x in (q, k, v, dout))
            p = np.where(causal, np.exp(scale * qh @ kh.T - lse[a:b, h, None]), 0.0)
            ds = np.abs(p * (gh @ vh.T - np.sum(gh * out[a:b, h], axis=-1, keepdims=True)))
            cq[a:b, h] = scale * ds @ np.abs(kh)
            ck[a:b, h] = scale * ds.T @ np.abs(qh)
            cv[a:b, h] = p.T @ np.abs(gh)
    return cq, ck, cv


def run_case(mla, sh, lens, seed=0, kpe_in_latent=False, with_lse=False):
    H = sh.num_heads
    rng = np.random.default_rng(seed)
    n = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = mi.bf16_round(rng.standard_normal((n, H, 192)).astype(np.float32))
    kv = mi.bf16_round(rng.standard_normal((n, H, 256)).astype(np.float32))
    kpe = mi.bf16_round(rng.standard_normal((n, 64)).astype(np.float32))
    dout = mi.bf16_round(rng.standard_normal((n, H, 128)).astype(np.float32))
    cfg = mla.make_config(sh)
    scale = om.softmax_scale(sh)
    k = np.concatenate([kv[..., :128], np.broadcast_to(kpe[:, None, :], (n, H, 64))], -1)
    o = mi.bf16_round(om.causal_varlen_attention(q, k, kv[..., 128:], scale, cu).astype(np.float32))
    rdq, rdkv, rdkpe, lse = ob.attention_core_backward(q, kv, kpe, scale, cu, dout, 128, out=o)
    cq, ck, cv = conditioning(q, k, kv[..., 128:], dout, o.astype(np.float64), scale, cu, lse)
    allow = {"dq": cq, "dkv": np.concatenate([ck[..., :128], cv], axis=-1), "dkpe": np.sum(ck[..., 128:], axis=1)}
    dq = torch.full((n, H, 192), float("nan"), dtype=torch.float32, device=DEV)
    dkv = torch.full((n, H, 256), float("nan"), dtype=torch.float32, device=DEV)
    dkpe = torch.full((n, 64), float("nan"), dtype=torch.float32, device=DEV)
    kpe_d = dev(kpe, torch.bfloat16)
    if kpe_in_latent:
        lat = torch.randn(n, 576, device=DEV).to(torch.bfloat16)
        lat[:, 512:] = kpe_d
        kpe_d = lat[:, 512:]
    q_d, kv_d, cu_d = dev(q, torch.bfloat16), dev(kv, torch.bfloat16), torch.from_numpy(cu).to(DEV)
    lse_d = None
    if with_lse:
        # the forward's log-sum-exp (base 2, [H, N]) against the oracle's
        # natural one, then handed to the backward in place of its statistics.
        # The forward sums P after rounding it to the operand type (the same
        # P it multiplies by v), so its denominator is within a factor 1 +- u
        # of the exact one: |lse error| <= u (+ fp32 arithmetic).
        lse_d = torch.full((H, n), float("nan"), dtype=torch.float32, device=DEV)
        attn = torch.empty(n, H, 128, dtype=torch.bfloat16, device=DEV)
        mla.attention_prefill(cfg, q_d, kv_d, kpe_d, cu_d, cu, attn, lse=lse_d)
        torch.cuda.synchronize()
        got_lse = lse_d.cpu().numpy().T.astype(np.float64) * np.log(2.0)
        err = float(np.max(np.abs(got_lse - lse)))
        _say(f"  forward lse: max-abs error {err:.3e}")
        assert err <= U + 1e-5, err
    mla.attention_prefill_bwd(cfg, q_d, kv_d, kpe_d, cu_d, cu, dev(o, torch.bfloat16),
                              dev(dout, torch.bfloat16), dq, dkv, dkpe, lse=lse_d)
    torch.cuda.synchronize()
    got = {"dq": dq.cpu().numpy(), "dkv": dkv.cpu().numpy(), "dkpe": dkpe.cpu().numpy()}
    ref = {"dq": rdq, "dkv": rdkv, "dkpe": rdkpe}
    for name in ("dq", "dkv", "dkpe"):
        g, r = got[name], ref[name]
        assert np.all(np.isfinite(g)), name
        rms = float(np.sqrt(np.mean(r * r)))
        frac = float(np.max(np.abs(g - r) / (2 * U * allow[name] + 2.0 ** -12 * rms)))
        _say(f"  {name}: max-abs / tensor RMS {np.max(np.abs(g - r)) / rms:.3e}, of the allowance {frac:.3f}")
        assert frac <= 1.0, (name, frac)


@pytest.mark.parametrize("heads,lens", [(16, [1, 33, 200, 300]), (128, [257]), (32, [64, 128, 129]),
                                        (128, [1000, 24]), (8, [5, 0, 130])])
def test_attention_backward(mla, heads, lens):
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=heads)
    _say(f"case: attention backward heads={heads} lens={lens}")
    run_case(mla, sh, lens)


@pytest.mark.parametrize("heads,lens", [(16, [1, 33, 200, 300]), (128, [257]), (8, [5, 0, 130]),
                                        (16, [1500, 700])])
def test_attention_backward_with_forward_lse(mla, heads, lens):
    """The forward's log-sum-exp output (checked against the oracle's) passed
    to the backward, which then skips its statistics pass and forms D in the dq
    pass; 128 heads x [257] and 16 heads x [1500, 700] run the forward paired."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=heads)
    _say(f"case: attention backward with the forward lse, heads={heads} lens={lens}")
    run_case(mla, sh, lens, seed=5, with_lse=True)


def test_attention_backward_megatron_shape(mla):
    """The Megatron-default head count and softmax scale (plain RoPE, scale
    192^-0.5), two documents of 1024."""
    sh = mi.WORKLOADS["megatron_2x2048"]
    _say("case: attention backward, Megatron shape, 2 x 1024")
    run_case(mla, sh, [1024, 1024], seed=3)


def test_attention_backward_strided_kpe(mla):
    """k_pe read in place from the latent rows [c_n | k_pe] (row stride 576),
    as the forward leaves it."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=16)
    _say("case: attention backward, k_pe strided in the latent rows, lens=[70, 130]")
    run_case(mla, sh, [70, 130], seed=4, kpe_in_latent=True)


def test_attention_backward_full_size(mla):
    """The 4096-token document with 128 heads, as timed: all heads run, the
    oracle checks four of them (the heads are independent apart from the
    shared k_pe, and the full-size oracle would hold [128, 4096, 4096]
    float64 arrays).  dkpe: the kernel's per-head gradients of the shared key
    part (left in its workspace) are checked on those heads, and their sum over
    all heads against dkpe.  Heads outside the sample get a seeded stand-in
    for the forward output (any bf16 values are valid input)."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"]
    H, n = sh.num_heads, 4096
    heads = [0, 37, 90, 127]
    _say(f"case: attention backward full size, heads={H} lens=[{n}], oracle heads {heads}")
    rng = np.random.default_rng(9)
    cu = np.array([0, n], np.int32)
    q = mi.bf16_round(rng.standard_normal((n, H, 192)).astype(np.float32))
    kv = mi.bf16_round(rng.standard_normal((n, H, 256)).astype(np.float32))
    kpe = mi.bf16_round(rng.standard_normal((n, 64)).astype(np.float32))
    dout = mi.bf16_round(rng.standard_normal((n, H, 128)).astype(np.float32))
    o = mi.bf16_round((0.1 * rng.standard_normal((n, H, 128))).astype(np.float32))
    scale = om.softmax_scale(sh)
    cfg = mla.make_config(sh)
    refs = {}
    for h in heads:
        sl = slice(h, h + 1)
        k = np.concatenate([kv[:, sl, :128], kpe[:, None, :]], -1)
        o[:, sl] = mi.bf16_round(om.causal_varlen_attention(q[:, sl], k, kv[:, sl, 128:], scale, cu).astype(np.float32))
        r = ob.attention_core_backward(q[:, sl], kv[:, sl], kpe, scale, cu, dout[:, sl], 128, out=o[:, sl])
        c = conditioning(q[:, sl], k, kv[:, sl, 128:], dout[:, sl], o[:, sl].astype(np.float64), scale, cu, r[3])
        refs[h] = (r, c)
    dq = torch.full((n, H, 192), float("nan"), dtype=torch.float32, device=DEV)
    dkv = torch.full((n, H, 256), float("nan"), dtype=torch.float32, device=DEV)
    dkpe = torch.full((n, 64), float("nan"), dtype=torch.float32, device=DEV)
    ws = mla.attention_prefill_bwd(cfg, dev(q, torch.bfloat16), dev(kv, torch.bfloat16), dev(kpe, torch.bfloat16),
                                   torch.from_numpy(cu).to(DEV), cu, dev(o, torch.bfloat16), dev(dout, torch.bfloat16),
                                   dq, dkv, dkpe)
    torch.cuda.synchronize()
    off = 2 * (-(-n * H * 4 // 256) * 256)
    dkr = ws[off:off + n * H * 64 * 4].view(torch.float32).view(n, H, 64).cpu().numpy()
    g_dq, g_dkv, g_dkpe = dq.cpu().numpy(), dkv.cpu().numpy(), dkpe.cpu().numpy()
    assert np.all(np.isfinite(g_dq)) and np.all(np.isfinite(g_dkv)) and np.all(np.isfinite(g_dkpe))
    for h in heads:
        (rdq, rdkv, rdkr, _), (cq, ck, cv) = refs[h]
        for name, g, r, al in (("dq", g_dq[:, h], rdq[:, 0], cq[:, 0]),
                               ("dkv", g_dkv[:, h], rdkv[:, 0], np.concatenate([ck[:, 0, :128], cv[:, 0]], -1)),
                               ("dk_pe of the head", dkr[:, h], rdkr, ck[:, 0, 128:])):
            rms = float(np.sqrt(np.mean(r * r)))
            frac = float(np.max(np.abs(g - r) / (2 * U * al + 2.0 ** -12 * rms)))
            _say(f"  head {h} {name}: max-abs / RMS {np.max(np.abs(g - r)) / rms:.3e}, of the allowance {frac:.3f}")
            assert frac <= 1.0, (h, name, frac)
    # dkpe is the head sum of the per-head parts (fp32 sums in another order)
    s = dkr.astype(np.float64).sum(axis=1)
    err = np.max(np.abs(g_dkpe - s) / (1e-5 * np.abs(dkr).sum(axis=1) + 1e-30))
    _say(f"  dkpe vs the head sum of the per-head parts: {err:.3f} of 1e-5 sum |parts|")
    assert err <= 1.0
