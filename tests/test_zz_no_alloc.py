"""GPU: the allocation-free decode entry point against the one with a workspace.

mla_decode_absorbed_fwd_noalloc runs the same kernels on the library's static
scratch; on the same inputs its output must equal mla_decode_absorbed_fwd's
bit for bit, and both must meet the parity bound against the oracle.  Two
calls in a row, the second on a smaller batch (the scratch keeps the first
call's contents, which the second must not read).
"""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import mla as om
from test_gpu_parity import DEV, _say, bf16_check, dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import latent_attention_forward_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def _inputs(dc):
    b = lambda a: dev(a, torch.bfloat16)
    return (b(dc.w_kv_b), b(dc.q_nope), b(dc.q_pe), b(dc.cache), torch.from_numpy(dc.block_table).to(DEV),
            torch.from_numpy(dc.seq_lens).to(DEV), dc.seq_lens)


def test_noalloc_decode_matches_workspace_decode(mla):
    sh = mi.WORKLOADS["dsv3_decode_64"]
    cfg = mla.make_config(sh)
    cases = [("full DeepSeek-V3 decode, 64 sequences", mi.make_decode_case(sh)),
             ("smaller batch after it", mi.make_decode_case(sh, seq_lens=[5, 3000, 129, 64, 1], block_size=32))]
    for label, dc in cases:
        _say(f"case: no-alloc decode, {label}")
        args = _inputs(dc)
        B = len(dc.seq_lens)
        out_ws = torch.full((B, sh.num_heads, sh.v_head_dim), float("nan"), dtype=torch.bfloat16, device=DEV)
        out_na = torch.full_like(out_ws, float("nan"))
        mla.decode_absorbed_fwd_noalloc(cfg, *args, out_na)
        mla.decode_absorbed_fwd(cfg, *args, out_ws)
        torch.cuda.synchronize()
        a, b = out_na.float().cpu().numpy(), out_ws.float().cpu().numpy()
        assert np.array_equal(a, b)
        ref = om.decode_absorbed(sh, dc.w_kv_b, dc.q_nope, dc.q_pe, dc.cache, dc.block_table, dc.seq_lens,
                                 dc.block_size)
        bf16_check(ref.reshape(B, -1), a.reshape(B, -1), "no-alloc output vs oracle")


def test_noalloc_decode_refuses_a_batch_beyond_the_scratch(mla):
    sh = mi.WORKLOADS["dsv3_decode_64"]
    cfg = mla.make_config(sh)
    lens = np.full(300, 8192, np.int32)
    dc = mi.make_decode_case(sh, seq_lens=[64], block_size=64)
    w, qn, qp, cache, table, _, _ = _inputs(dc)
    qn, qp = qn.expand(300, -1, -1).contiguous(), qp.expand(300, -1, -1).contiguous()
    table = torch.zeros(300, 128, dtype=torch.int32, device=DEV)
    out = torch.empty(300, sh.num_heads, sh.v_head_dim, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mla.MLAError) as e:
        mla.decode_absorbed_fwd_noalloc(cfg, w, qn, qp, cache, table, torch.from_numpy(lens).to(DEV), lens, out)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
