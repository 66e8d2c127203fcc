"""HIP graph capture of the library calls.

A call of the library allocates nothing, copies nothing, clears nothing with a
memset and never synchronises: it only launches kernels on the stream it is
given.  So a whole prefill layer, a chunked prefill or an absorbed decode call
can be recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed.  Every
kernel is deterministic, so each replay must reproduce the eager result bit for
bit.  The replays are interleaved with eager work and synchronisations, every
replay is checked, and one input is changed in place between replays to show
that the graph reads the live buffers.
"""
import sys

import numpy as np
import pytest

import mla_inputs as mi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    import latent_attention_forward_amd as m
    m.load_library()
    return m


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(torch.bfloat16)


def _capture(call):
    """Warm up on a side stream, then record one call into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _replays(g, call, outs, mutate):
    """Replay four times against the eager result; after the second replay the
    input is changed in place and the eager result recomputed."""
    call()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    for i in range(4):
        if i == 2:
            mutate()
            call()
            torch.cuda.synchronize()
            refs = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float(i + 1))          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"replay {i}, output {k} differs from the eager call"
    return refs


def test_decode_graph_replays_match_eager(mla):
    _say("case: graph of mla_decode_absorbed_fwd, lens [700, 64, 1500, 33], block 64")
    sh = mi.WORKLOADS["dsv3_decode_64"]
    dc = mi.make_decode_case(sh, seq_lens=[700, 64, 1500, 33], block_size=64)
    cfg = mla.make_config(sh)
    w, qn, qp, cache = _bf(dc.w_kv_b), _bf(dc.q_nope), _bf(dc.q_pe), _bf(dc.cache)
    table = torch.from_numpy(dc.block_table).to(DEV)
    lens = torch.from_numpy(dc.seq_lens).to(DEV)
    ws = torch.empty(mla.decode_workspace_size(cfg, dc.seq_lens), dtype=torch.uint8, device=DEV)
    out = torch.empty(len(dc.seq_lens), sh.num_heads, sh.v_head_dim, dtype=torch.bfloat16, device=DEV)

    def call():
        mla.decode_absorbed_fwd(cfg, w, qn, qp, cache, table, lens, dc.seq_lens, out, workspace=ws)

    g = _capture(call)
    first = out.clone()
    refs = _replays(g, call, [out], lambda: qn.neg_())
    assert not torch.equal(refs[0], first), "negating q_nope must change the output"


def test_prefill_graph_replays_match_eager(mla):
    _say("case: graph of mla_prefill_fwd, DeepSeek-V3 layer at hidden 512, 4 heads, documents [70, 1, 131, 257]")
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=4, q_lora_rank=256)
    case = mi.make_prefill_case(sh, doc_lengths=[70, 1, 131, 257])
    cfg = mla.make_config(sh)
    W = {k: (None if v is None else _bf(v)) for k, v in case.w.items()}
    x = _bf(case.x)
    n = case.x.shape[0]
    cu = torch.from_numpy(case.cu_seqlens).to(DEV)
    cos, sin = mla.rope_table(cfg, int(np.max(np.diff(case.cu_seqlens))) + 1, DEV)
    out = torch.empty(n, sh.hidden, dtype=torch.bfloat16, device=DEV)
    lat = torch.empty(n, sh.kv_lora_rank + sh.qk_rope_dim, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(mla.prefill_workspace_size(cfg, n, len(case.cu_seqlens) - 1), dtype=torch.uint8, device=DEV)

    def call():
        mla.prefill_fwd(cfg, W, x, cu, case.cu_seqlens, out, latent_out=lat, rope_cos=cos, rope_sin=sin,
                        workspace=ws)

    g = _capture(call)
    _replays(g, call, [out, lat], lambda: x.mul_(0.5))


def test_chunk_graph_replays_match_eager(mla):
    _say("case: graph of mla_prefill_chunk_fwd, chunks [40, 7, 100] after prefixes [300, 0, 64], block 16")
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=4, q_lora_rank=256)
    cc = mi.make_chunk_case(sh, [40, 7, 100], [300, 0, 64], block_size=16)
    cfg = mla.make_config(sh)
    W = {k: (None if v is None else _bf(v)) for k, v in cc.w.items()}
    x = _bf(cc.x)
    n = cc.x.shape[0]
    cu = torch.from_numpy(cc.cu_seqlens).to(DEV)
    pre = torch.from_numpy(cc.prefix_lens).to(DEV)
    cache = _bf(cc.cache)
    table = torch.from_numpy(cc.block_table).to(DEV)
    longest = int(np.max(cc.prefix_lens + np.diff(cc.cu_seqlens)))
    cos, sin = mla.rope_table(cfg, longest, DEV)
    out = torch.empty(n, sh.hidden, dtype=torch.bfloat16, device=DEV)
    lat = torch.empty(n, sh.kv_lora_rank + sh.qk_rope_dim, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(mla.prefill_chunk_workspace_size(cfg, cc.cu_seqlens, cc.prefix_lens), dtype=torch.uint8,
                     device=DEV)

    def call():
        mla.prefill_chunk_fwd(cfg, W, x, cu, cc.cu_seqlens, pre, cc.prefix_lens, cache, table, out,
                              latent_out=lat, rope_cos=cos, rope_sin=sin, workspace=ws)

    g = _capture(call)
    _replays(g, call, [out, lat], lambda: cache.mul_(0.5))


def test_attention_forward_backward_graph_replays_match_eager(mla):
    """The attention core with its log-sum-exp output (16 heads, documents
    [1500, 700]: the paired one-round launch) and the backward given that
    log-sum-exp, recorded as one graph."""
    _say("case: graph of mla_attention_prefill (lse) + mla_attention_prefill_bwd, 16 heads, lens [1500, 700]")
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=16)
    cfg = mla.make_config(sh)
    lens = [1500, 700]
    n, H = sum(lens), 16
    cuh = np.array([0, 1500, 2200], np.int32)
    cu = torch.from_numpy(cuh).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(21)
    q = torch.randn(n, H, 192, device=DEV, generator=g).to(torch.bfloat16)
    kv = torch.randn(n, H, 256, device=DEV, generator=g).to(torch.bfloat16)
    kpe = torch.randn(n, 64, device=DEV, generator=g).to(torch.bfloat16)
    dout = torch.randn(n, H, 128, device=DEV, generator=g).to(torch.bfloat16)
    attn = torch.empty(n, H, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(H, n, dtype=torch.float32, device=DEV)
    dq = torch.empty(n, H, 192, dtype=torch.float32, device=DEV)
    dkv = torch.empty(n, H, 256, dtype=torch.float32, device=DEV)
    dkpe = torch.empty(n, 64, dtype=torch.float32, device=DEV)
    ws = torch.empty(mla.attention_bwd_workspace_size(cfg, n), dtype=torch.uint8, device=DEV)

    def call():
        mla.attention_prefill(cfg, q, kv, kpe, cu, cuh, attn, lse=lse)
        mla.attention_prefill_bwd(cfg, q, kv, kpe, cu, cuh, attn, dout, dq, dkv, dkpe, workspace=ws, lse=lse)

    graph = _capture(call)
    refs = _replays(graph, call, [attn, lse, dq, dkv, dkpe], lambda: dout.mul_(-0.5))
    assert all(bool(torch.isfinite(r).all()) for r in refs)
