"""GPU parity of the chunked prefill over a cached latent prefix
(``mla_prefill_chunk_fwd``) against the float64 oracle, through the C ABI.

Same bounds as the prefill tests: bf16 outputs within 2e-2 of the row RMS on
top of one bf16 ulp, fp32 within 1e-4 of the row RMS; the prefix-free chunk
is bit-identical to the plain prefill.
"""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import mla as om
from test_gpu_parity import BF16_TOL, F32_TOL, DEV, _say, bf16_check, dev, tdtype, run_prefill  # noqa: F401

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    import latent_attention_forward_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load_library()
    return m


def run_chunk(mla, sh, c, table=None, cache=None):
    dt = tdtype(sh)
    cfg = mla.make_config(sh)
    W = {k: dev(v, dt) for k, v in c.w.items()}
    x = dev(c.x, dt)
    n = c.x.shape[0]
    cu = torch.from_numpy(c.cu_seqlens).to(DEV)
    pre = torch.from_numpy(c.prefix_lens).to(DEV)
    cos = sin = None
    if sh.rope.kind != "none":
        longest = int(np.max(c.prefix_lens + np.diff(c.cu_seqlens)))
        cos, sin = mla.rope_table(cfg, longest + 1, DEV)
    out = torch.full((n, sh.hidden), float("nan"), dtype=dt, device=DEV)
    lat = torch.full((n, sh.kv_lora_rank + sh.qk_rope_dim), float("nan"), dtype=dt, device=DEV)
    kc = dev(c.cache if cache is None else cache, dt)
    bt = torch.from_numpy(c.block_table if table is None else table).to(DEV)
    mla.prefill_chunk_fwd(cfg, W, x, cu, c.cu_seqlens, pre, c.prefix_lens, kc, bt, out, latent_out=lat,
                          rope_cos=cos, rope_sin=sin)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lat.float().cpu().numpy()


def oracle(sh, c, rows=None):
    return om.mla_prefill_with_prefix(sh, c.w, c.x, c.cu_seqlens, c.prefix_lens, c.cache, c.block_table,
                                      c.block_size, rows=rows)


SMALL = {
    "v3_yarn": (mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=4, q_lora_rank=256),
                [70, 1, 131, 5], [0, 64, 300, 129], 64),
    "megatron_direct_q": (mi.WORKLOADS["megatron_2x2048"].replace(hidden=256, num_heads=2),
                          [128, 33], [256, 1], 16),
    "kimi_gate_nope": (mi.WORKLOADS["kimi_gated_varlen_8192"].replace(hidden=384, num_heads=3, q_lora_rank=128),
                       [33, 190], [200, 17], 32),
    # many sequences with mixed prefixes, 16-token blocks
    "v3_many_small_blocks": (mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=2, q_lora_rank=256),
                             [1, 2, 129, 64, 7, 300, 1, 50], [0, 1, 15, 16, 17, 1000, 4095, 127], 16),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_chunk_small(mla, name):
    sh, chunks, prefixes, bs = SMALL[name]
    _say(f"case: chunk over prefix {name} chunks={chunks} prefixes={prefixes} block={bs}")
    c = mi.make_chunk_case(sh, chunks, prefixes, block_size=bs)
    got, lat = run_chunk(mla, sh, c)
    ref = oracle(sh, c)
    bf16_check(ref["out"], got, "out")
    bf16_check(ref["latent"], lat, "latent of the new tokens")


def test_chunk_tiny_fp32(mla):
    sh = mi.WORKLOADS["tiny_fp32_t64"]
    _say("case: chunk over prefix, tiny fp32")
    c = mi.make_chunk_case(sh, [20, 7, 1], [44, 3, 0], block_size=16)
    got, lat = run_chunk(mla, sh, c)
    ref = oracle(sh, c)
    err = om.row_rel_error(ref["out"], got)
    _say(f"  err {err:.3e}")
    assert err <= F32_TOL
    assert om.row_rel_error(ref["latent"], lat) <= F32_TOL


def test_chunk_without_prefix_is_the_prefill(mla):
    """Every prefix 0: the same bits as mla_prefill_fwd on the same tokens."""
    sh, _, _, _ = SMALL["v3_yarn"]
    lens = [70, 1, 131, 0, 257]
    c = mi.make_chunk_case(sh, lens, [0] * len(lens), block_size=64)
    got, lat = run_chunk(mla, sh, c)
    case = mi.PrefillCase(shape=sh, x=c.x, w=c.w, cu_seqlens=c.cu_seqlens)
    want, want_lat = run_prefill(mla, sh, case, latent=True)
    assert np.array_equal(got, want) and np.array_equal(lat, want_lat)


def test_chunk_single_new_token_per_sequence(mla):
    """T = 1 (a decode step taken through the prefill path): every cached key is visible."""
    sh, _, _, _ = SMALL["v3_yarn"]
    c = mi.make_chunk_case(sh, [1, 1, 1], [1, 64, 1000], block_size=64)
    got, _ = run_chunk(mla, sh, c)
    bf16_check(oracle(sh, c)["out"], got, "out")


def test_chunk_bad_block_id_poisons_only_its_sequence(mla):
    sh, chunks, prefixes, bs = SMALL["v3_yarn"]
    c = mi.make_chunk_case(sh, chunks, prefixes, block_size=bs)
    table = c.block_table.copy()
    table[2, 1] = 10 ** 6                                  # sequence 2, a cached block
    got, _ = run_chunk(mla, sh, c, table=table)
    cu = c.cu_seqlens
    assert np.all(np.isnan(got[cu[2]:cu[3]]))
    ok = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in (0, 1, 3)])
    assert np.all(np.isfinite(got[ok]))
    bf16_check(oracle(sh, c, rows=ok)["out"], got[ok], "other sequences")


def test_prefill_then_chunk_continues_the_prefill(mla):
    """The latent rows a prefill returns, stored in a paged cache, let a chunk
    of the following tokens reproduce the whole-sequence layer (oracle) on
    those tokens."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(hidden=512, num_heads=8, q_lora_rank=256)
    P, T, bs = 300, 150, 64
    full = mi.make_prefill_case(sh, doc_lengths=[P + T])
    first = mi.PrefillCase(shape=sh, x=full.x[:P], w=full.w, cu_seqlens=np.array([0, P], np.int32))
    _, lat = run_prefill(mla, sh, first, latent=True)
    nblk = (P + bs - 1) // bs
    cache = np.full((nblk + 1, bs, lat.shape[1]), np.nan, np.float32)
    table = np.full((1, nblk + 2), -1, np.int32)
    table[0, :nblk] = np.random.default_rng(9).permutation(nblk + 1)[:nblk]
    for j in range(P):
        cache[table[0, j // bs], j % bs] = lat[j]
    c = mi.ChunkCase(shape=sh, x=full.x[P:], w=full.w, cu_seqlens=np.array([0, T], np.int32),
                     prefix_lens=np.array([P], np.int32), cache=cache, block_table=table, block_size=bs)
    got, _ = run_chunk(mla, sh, c)
    ref = om.mla_prefill_rows(sh, full.w, full.x, full.cu_seqlens, list(range(P, P + T)))
    bf16_check(ref["out"], got, "chunk after prefill vs whole-sequence oracle")


def test_chunk_full_size_sampled_rows(mla):
    """DeepSeek-V3 shape (128 heads, YaRN): two sequences continuing long cached prefixes."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"]
    chunks, prefixes = [512, 128], [3000, 700]
    _say(f"case: full-size chunk chunks={chunks} prefixes={prefixes}")
    c = mi.make_chunk_case(sh, chunks, prefixes, block_size=64)
    got, lat = run_chunk(mla, sh, c)
    cu = c.cu_seqlens
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 511, 512, 513, int(cu[-1]) - 1] + list(rng.integers(0, int(cu[-1]), 10))))
    ref = oracle(sh, c, rows=rows)
    bf16_check(ref["out"], got[rows], "out (sampled rows)")
    bf16_check(ref["latent"], lat, "latent (all new rows)")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("qlens,klens", [([1, 64, 200, 129], [1, 64, 700, 1000]), ([300, 5], [300, 4099])])
def test_attention_prefix_core(mla, qlens, klens):
    """The attention core alone, fp16 operands, ragged queries over longer keys."""
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=2)
    _say(f"case: attention over a prefix qlens={qlens} klens={klens}")
    rng = np.random.default_rng(5)
    f16 = lambda a: np.asarray(a, np.float16).astype(np.float32)
    n, nk = sum(qlens), sum(klens)
    q = f16(rng.standard_normal((n, 2, 192)))
    kv = f16(rng.standard_normal((nk, 2, 256)))
    kpe = f16(rng.standard_normal((nk, 64)))
    cq = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(klens)]).astype(np.int32)
    attn = torch.full((n, 2, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    mla.attention_prefix(mla.make_config(sh), dev(q, torch.float16), dev(kv, torch.float16), dev(kpe, torch.float16),
                         torch.from_numpy(cq).to(DEV), cq, torch.from_numpy(ck).to(DEV), ck, attn)
    torch.cuda.synchronize()
    got = attn.float().cpu().numpy()
    k = np.concatenate([kv[..., :128], np.broadcast_to(kpe[:, None, :], (nk, 2, 64))], -1)
    for d in range(len(qlens)):
        P = klens[d] - qlens[d]
        ref = om.prefix_causal_attention(q[cq[d]:cq[d + 1]], k[ck[d]:ck[d + 1]], kv[ck[d]:ck[d + 1], :, 128:],
                                         om.softmax_scale(sh), P)
        bf16_check(ref.reshape(-1, 128), got[cq[d]:cq[d + 1]].reshape(-1, 128), f"doc {d} (P={P})")


def test_attention_prefix_rejects_short_keys(mla):
    sh = mi.WORKLOADS["dsv3_prefill_4096"].replace(num_heads=2)
    t = torch.zeros(8, 2, 256, dtype=torch.float16, device=DEV)
    cq = np.array([0, 4], np.int32)
    ck = np.array([0, 3], np.int32)
    with pytest.raises(mla.MLAError):
        mla.attention_prefix(mla.make_config(sh), t[:, :, :192].contiguous(), t, t[:, 0, :64].contiguous(),
                             torch.from_numpy(cq).to(DEV), cq, torch.from_numpy(ck).to(DEV), ck,
                             torch.empty(4, 2, 128, dtype=torch.bfloat16, device=DEV))
