#!/usr/bin/env python3
"""Benchmark of the MLA forward hot path on one MI355X.

One step = one full MLA prefill layer (DeepSeek-V3 shape, 4096 tokens, 128
heads, YaRN) plus one weight-absorbed decode over the paged latent cache (64
sequences, lengths U[1024, 8192]).  Prints ONE JSON line.

Metric: "MLA prefill attn TFLOP/s + absorbed decode HBM GB/s, % of MI355X
peak".  ``value`` is the mean of the two fractions of peak, in percent:
  prefill attention: algorithmic FLOPs 2 (d_qk + d_v) H sum_d T_d (T_d + 1) / 2
      per launch / the attention kernel's mean launch time, against the dense
      bf16/fp16 MFMA peak (2516.6 TFLOP/s), on the DeepSeek-V3 workload with
      the layer's own (fp16) operand type;
  absorbed decode: algorithmic bytes sum_b L_b (r_kv + d_rope) 2 + W_kv_b + q +
      out + index arrays per call / the mean call time, against 8 TB/s.
Beside it: the attention kernel on the other two graded prefill workloads
(Megatron-shaped 2 x 2048, Kimi-shaped gated 8192 tokens in 4 documents),
with bf16 operands on the DeepSeek-V3 workload, the fused latent
norm + RoPE kernel's GB/s, and the chunked prefill over a cached prefix.

The attention operands are the workloads' own: q, kv and the shared k_pe are
computed from each workload's seeded x and weights with the library's
projection and norm/RoPE calls, then held in the operand type timed.
Kernel times are HIP events on the stream the kernels run on.  Between timed
decode calls a 512 MiB buffer is read, so the 256 MB Infinity Cache holds none
of the ~370 MB decode working set (a read leaves clean lines; overwriting the
buffer instead would charge the decode for writing back 256 MB of dirty
lines).
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA prefill attn TFLOP/s + absorbed decode HBM GB/s, % of MI355X peak"
PEAK_MFMA_TFLOPS = 2516.6      # dense bf16 / fp16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 << 20
# sources whose change invalidates a committed counter figure
KERNEL_SOURCES = {"flash": ["flash.hip", "mla_internal.hpp"],
                  "decode": ["decode.hip", "api.hip", "mla_internal.hpp"],
                  "decode_fp8": ["decode_fp8.hip", "decode.hip", "api.hip", "mla_internal.hpp"],
                  "chunk": ["flash.hip", "mla_internal.hpp"]}
# the graded prefill workloads whose attention kernel is timed
ATTN_WORKLOADS = ["megatron_2x2048", "dsv3_prefill_4096", "kimi_gated_varlen_8192"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill", default="dsv3_prefill_4096")
    ap.add_argument("--decode", default="dsv3_decode_64")
    ap.add_argument("--chunk", default="dsv3_chunk_4x1024_p4096",
                    help="chunked-prefill workload reported beside the metric ('none' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["full", "prefill", "prefill_bwd", "attention", "attention_bwd", "decode",
                                       "decode_fp8", "copy", "chunk", "chunk_attention", "norm"], default="full",
                    help="full: the JSON line; the others only run that part's timing loop (for profilers)")
    ap.add_argument("--attn-workload", default="dsv3_prefill_4096", choices=ATTN_WORKLOADS,
                    help="workload of --mode attention")
    ap.add_argument("--operand", default="f16", choices=["f16", "bf16"],
                    help="attention operand type of --mode attention / prefill")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for the CPU baseline")
    return ap.parse_args()


def attention_flops(shape, cu):
    s = 0
    for a, b in zip(cu[:-1], cu[1:]):
        t = int(b) - int(a)
        s += t * (t + 1) // 2
    return 2 * (shape.qk_head_dim + shape.v_head_dim) * shape.num_heads * s


def attention_bwd_flops(shape, cu):
    """Algorithmic FLOPs of the attention backward: per causal (query, key,
    head) pair the score recompute and dq, dk (2 d_qk each), dP and dv (2 d_v
    each), two FLOPs per multiply-add."""
    dqk, dv = shape.qk_head_dim, shape.v_head_dim
    return attention_flops(shape, cu) // (dqk + dv) * (3 * dqk + 2 * dv)


# Chunked prefill over a cached prefix: (layer shape, new tokens per sequence,
# cached tokens per sequence).  DeepSeek-V3 shape, four sequences each
# continuing 4096 cached tokens with a 1024-token chunk.
CHUNK_WORKLOADS = {"dsv3_chunk_4x1024_p4096": ("dsv3_prefill_4096", [1024] * 4, [4096] * 4)}


def prefix_attention_flops(shape, chunks, prefixes):
    s = 0
    for t, p in zip(chunks, prefixes):
        s += t * p + t * (t + 1) // 2          # query i sees p + i + 1 keys
    return 2 * (shape.qk_head_dim + shape.v_head_dim) * shape.num_heads * s


def layer_flops(shape, n, attn):
    H, dqk, dv, r, dr = shape.num_heads, shape.qk_head_dim, shape.v_head_dim, shape.kv_lora_rank, shape.qk_rope_dim
    f = 0
    if shape.q_lora_rank:
        f += 2 * n * shape.hidden * shape.q_lora_rank + 2 * n * shape.q_lora_rank * H * dqk
    else:
        f += 2 * n * shape.hidden * H * dqk
    f += 2 * n * shape.hidden * (r + dr) + 2 * n * r * H * (shape.qk_nope_dim + dv)
    if shape.output_gate:
        f += 2 * n * shape.hidden * H * dv
    if shape.o_groups:
        f += 2 * n * H * dv * shape.o_lora_rank + 2 * n * shape.o_groups * shape.o_lora_rank * shape.hidden
    else:
        f += 2 * n * H * dv * shape.hidden
    return f + attn


def layer_gemms(shape, n):
    """The prefill layer's projections in the order the library launches
    them: (name, flops)."""
    H, dqk, dv, r, dr = shape.num_heads, shape.qk_head_dim, shape.v_head_dim, shape.kv_lora_rank, shape.qk_rope_dim
    g = []
    if shape.q_lora_rank:
        g += [("q_a", 2 * n * shape.hidden * shape.q_lora_rank), ("q_b", 2 * n * shape.q_lora_rank * H * dqk)]
    else:
        g += [("q_proj", 2 * n * shape.hidden * H * dqk)]
    g += [("kv_a", 2 * n * shape.hidden * (r + dr)), ("kv_b", 2 * n * r * H * (shape.qk_nope_dim + dv))]
    if shape.output_gate:
        g += [("gate", 2 * n * shape.hidden * H * dv)]
    if shape.o_groups:
        g += [("o_a", 2 * n * H * dv * shape.o_lora_rank),
              ("o_b", 2 * n * shape.o_groups * shape.o_lora_rank * shape.hidden)]
    else:
        g += [("o_proj", 2 * n * H * dv * shape.hidden)]
    return g


def device_kernels(torch, fn, reps, between=None):
    """Device-side kernel durations (us) of `reps` calls of fn, from the torch
    profiler (it records every kernel dispatched in the process, the
    library's included); calls of `between` (not profiled work) are dropped
    by name.  Returns one list of (name, us) per call, in launch order."""
    from torch.profiler import profile, ProfilerActivity
    calls = []
    for _ in range(reps):
        if between is not None:
            between()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            fn()
            torch.cuda.synchronize()
        evs = sorted((e for e in prof.events() if e.device_type.name in ("CUDA", "HIP")),
                     key=lambda e: e.time_range.start)
        calls.append([(e.name, float(e.device_time)) for e in evs])
    return calls


def decode_bytes(shape, lens, max_blocks):
    H, r, dr, dn, dv = shape.num_heads, shape.kv_lora_rank, shape.qk_rope_dim, shape.qk_nope_dim, shape.v_head_dim
    B = len(lens)
    return (int(sum(lens)) * (r + dr) * 2 + H * (dn + dv) * r * 2 + B * H * (dn + dr) * 2 + B * H * dv * 2
            + B * max_blocks * 4 + B * 4)


def source_hash(name):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[name]:
        h.update(open(os.path.join(ROOT, "latent_attention_forward_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when it is missing or the kernel source changed since it was taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))[name]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256_16") != source_hash(name):
        return None
    return t.get("bytes_per_launch")


CPU_CODE = r'''
import json, sys, time, os, platform, io, contextlib
sys.path.insert(0, %(root)r)
import numpy as np
from threadpoolctl import threadpool_info
import mla_inputs as mi
from oracle import mla as om
heads_sample = %(heads)d

def best_of(fn, runs=3):
    fn()                                   # warm-up
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter(); fn(); ts.append(time.perf_counter() - t0)
    return min(ts)

# prefill attention: the 4096-token document of the DeepSeek-V3 workload at
# its head shape, on a sample of its 128 heads (the work per head is the same)
sh = mi.WORKLOADS[%(prefill)r]
T = sh.total_tokens
rng = np.random.default_rng(0)
q = rng.standard_normal((T, heads_sample, sh.qk_head_dim))
k = rng.standard_normal((T, heads_sample, sh.qk_head_dim))
v = rng.standard_normal((T, heads_sample, sh.v_head_dim))
scale = om.softmax_scale(sh)
tp = best_of(lambda: om.causal_varlen_attention(q, k, v, scale, [0, T]))
fp = 2 * (sh.qk_head_dim + sh.v_head_dim) * heads_sample * T * (T + 1) // 2
# absorbed decode over all 64 sequences; the non-absorbed form on 8 of them
dsh = mi.WORKLOADS[%(decode)r]
dc = mi.make_decode_case(dsh)
args = (dsh, dc.w_kv_b, dc.q_nope, dc.q_pe, dc.cache, dc.block_table, dc.seq_lens, dc.block_size)
td = best_of(lambda: om.decode_absorbed(*args))
B = len(dc.seq_lens)
H, r, dr, dn, dv = dsh.num_heads, dsh.kv_lora_rank, dsh.qk_rope_dim, dsh.qk_nope_dim, dsh.v_head_dim
dbytes = (int(dc.seq_lens.sum()) * (r + dr) * 2 + H * (dn + dv) * r * 2 + B * H * (dn + dr) * 2 + B * H * dv * 2
          + dc.block_table.size * 4 + B * 4)
sub = list(range(8))
t0 = time.perf_counter(); om.decode_naive(*args, batch_idx=sub); tn = time.perf_counter() - t0
nbytes = (int(dc.seq_lens[sub].sum()) * (r + dr) * 2 + H * (dn + dv) * r * 2 + 8 * H * (dn + dr + dv) * 2)
threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
cpu = platform.processor() or ""
try:
    for line in open("/proc/cpuinfo"):
        if line.startswith("model name"):
            cpu = line.split(":", 1)[1].strip(); break
except OSError:
    pass
buf = io.StringIO()
with contextlib.redirect_stdout(buf):
    np.show_config()
blas = " ".join(l.strip() for l in buf.getvalue().splitlines() if "name" in l.lower())[:300]
print(json.dumps({"prefill_tflops": fp / tp / 1e12, "prefill_T": T, "prefill_heads": heads_sample, "prefill_s": tp,
                  "decode_gbs": dbytes / td / 1e9, "decode_s": td, "decode_seqs": B,
                  "naive_gbs": nbytes / tn / 1e9, "naive_s": tn, "naive_seqs": len(sub),
                  "threads": threads, "affinity": len(os.sched_getaffinity(0)), "cpu": cpu, "blas": blas}))
'''


def cpu_baseline(prefill_name, decode_name, budget):
    """Time the float64 oracle on the host in a child process whose BLAS /
    OpenMP threads are set to the cores it may run on before NumPy loads:
    best of 3 runs after a warm-up for the prefill attention (the 4096-token
    DeepSeek-V3 document on a sample of its heads, sized so the whole leg
    takes about ``budget`` seconds) and the absorbed decode of all 64
    sequences; one run of the non-absorbed decode of 8 sequences."""
    cores = len(os.sched_getaffinity(0))
    env = dict(os.environ)
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        env[v] = str(cores)
    heads = 8 if budget >= 10 else 4
    code = CPU_CODE % dict(root=ROOT, heads=heads, prefill=prefill_name, decode=decode_name)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=900, env=env)
    if r.returncode != 0:
        raise RuntimeError("cpu baseline failed: " + r.stderr[-2000:])
    d = json.loads(r.stdout.strip().splitlines()[-1])
    frac = 0.5 * (d["prefill_tflops"] / PEAK_MFMA_TFLOPS + d["decode_gbs"] / PEAK_HBM_GBS) * 100
    return {
        "value": frac, "unit": "% of MI355X peak (same definition as value)", "cores": d["threads"],
        "kind": "oracle",
        "sample": (f"float64 oracle on {d['cpu']} ({d['affinity']} cores in the affinity mask, {d['threads']} BLAS "
                   f"threads): causal attention of the {d['prefill_T']}-token DeepSeek-V3 document on "
                   f"{d['prefill_heads']} of its heads, best of 3 after a warm-up ({d['prefill_s']:.2f} s, "
                   f"{d['prefill_tflops'] * 1e3:.2f} GFLOP/s); absorbed decode of all {d['decode_seqs']} sequences of "
                   f"{decode_name}, best of 3 ({d['decode_s']:.2f} s, {d['decode_gbs']:.3f} GB/s); non-absorbed "
                   f"decode of {d['naive_seqs']} sequences, one run ({d['naive_s']:.1f} s, {d['naive_gbs']:.3f} GB/s); "
                   f"numpy BLAS: {d['blas']}"),
        "prefill_attn_tflops": d["prefill_tflops"], "decode_gbs": d["decode_gbs"], "naive_decode_gbs": d["naive_gbs"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path runs on a single MI355X; sharding across GPUs is not built).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import latent_attention_forward_amd as mla
    import mla_inputs as mi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    mla.load_library()
    stream = torch.cuda.current_stream()
    tb = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)

    def timed(fn, k, warm=10):
        """Mean time of one call of fn in ms: HIP events around each call on
        the stream the library launches on, after `warm` untimed calls."""
        for _ in range(warm):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        for i in range(k):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / k

    def attention_operands(name):
        """q, kv and the shared k_pe of a prefill workload, computed from its
        seeded x and weights with the library's projection and norm/RoPE calls
        (bf16 intermediates), and a runner for the attention kernel on them."""
        sh = mi.WORKLOADS[name]
        case = mi.make_prefill_case(sh)
        cfg = mla.make_config(sh)
        n, H = case.x.shape[0], sh.num_heads
        cuh = case.cu_seqlens
        cu = torch.from_numpy(cuh).to(dev)
        x = tb(case.x)
        w = {k: tb(v) for k, v in case.w.items() if k in ("w_q_a", "q_a_gamma", "w_q_b", "w_q", "w_kv_a",
                                                          "kv_a_gamma", "w_kv_b")}
        del case
        lw = sh.kv_lora_rank + sh.qk_rope_dim
        rope = sh.rope.kind != "none"
        pos = torch.from_numpy(np.concatenate([np.arange(b - a) for a, b in zip(cuh[:-1], cuh[1:])]).astype(np.int32)).to(dev)
        cos = sin = None
        if rope:
            cos, sin = mla.rope_table(cfg, int(np.max(np.diff(cuh))), dev)
        q = torch.empty(n, H * sh.qk_head_dim, dtype=torch.bfloat16, device=dev)
        if sh.q_lora_rank:
            ql = torch.empty(n, sh.q_lora_rank, dtype=torch.bfloat16, device=dev)
            mla.linear(cfg, x, w["w_q_a"], ql)
            mla.latent_norm_rope(cfg, ql, n, sh.q_lora_rank, sh.q_lora_rank, w["q_a_gamma"], ql)
            mla.linear(cfg, ql, w["w_q_b"], q)
            del ql
        else:
            mla.linear(cfg, x, w["w_q"], q)
        if rope:
            mla.latent_norm_rope(cfg, q, n, H * sh.qk_head_dim, 0, None, q, rope_offset=sh.qk_nope_dim,
                                 rope_slices=H, rope_slice_stride=sh.qk_head_dim, rope_cos=cos, rope_sin=sin,
                                 positions=pos)
        ckv = torch.empty(n, lw, dtype=torch.bfloat16, device=dev)
        mla.linear(cfg, x, w["w_kv_a"], ckv)
        lat = torch.empty_like(ckv)
        mla.latent_norm_rope(cfg, ckv, n, lw, sh.kv_lora_rank, w["kv_a_gamma"], lat, rope_offset=sh.kv_lora_rank,
                             rope_slices=1 if rope else 0, rope_slice_stride=sh.qk_rope_dim, rope_cos=cos,
                             rope_sin=sin, positions=pos)
        kv = torch.empty(n, H * (sh.qk_nope_dim + sh.v_head_dim), dtype=torch.bfloat16, device=dev)
        mla.linear(cfg, lat[:, :sh.kv_lora_rank], w["w_kv_b"], kv)
        del x, w, ckv
        kpe = lat[:, sh.kv_lora_rank:].contiguous()
        del lat
        torch.cuda.synchronize()
        ops = {"bf16": (q.view(n, H, -1), kv.view(n, H, -1), kpe)}
        ops["f16"] = tuple(t.to(torch.float16) for t in ops["bf16"])
        attn = torch.empty(n, H, sh.v_head_dim, dtype=torch.bfloat16, device=dev)

        def runner(operand):
            qq, kk, pp = ops[operand]
            return lambda: mla.attention_prefill(cfg, qq, kk, pp, cu, cuh, attn)

        def backward():
            """The attention backward on the bf16 operands, with the forward's
            bf16 output and log-sum-exp and a seeded N(0, 1) output gradient."""
            qq, kk, pp = ops["bf16"]
            lse = torch.empty(H, n, dtype=torch.float32, device=dev)
            mla.attention_prefill(cfg, qq, kk, pp, cu, cuh, attn, lse=lse)
            o = attn.clone()
            g = torch.Generator(device=dev).manual_seed(7)
            do = torch.randn(o.shape, device=dev, generator=g).to(torch.bfloat16)
            dq = torch.empty(qq.shape, dtype=torch.float32, device=dev)
            dkv = torch.empty(kk.shape, dtype=torch.float32, device=dev)
            dkpe = torch.empty(pp.shape, dtype=torch.float32, device=dev)
            ws = torch.empty(mla.attention_bwd_workspace_size(cfg, n), dtype=torch.uint8, device=dev)
            return lambda: mla.attention_prefill_bwd(cfg, qq, kk, pp, cu, cuh, o, do, dq, dkv, dkpe, workspace=ws,
                                                     lse=lse)
        return {"shape": sh, "cu": cuh, "flops": attention_flops(sh, cuh), "run": runner, "ops": ops,
                "bwd": backward, "bwd_flops": attention_bwd_flops(sh, cuh)}

    # ------------------------------------------------------------------ prefill layer inputs
    sh = mi.WORKLOADS[args.prefill]
    case = mi.make_prefill_case(sh)
    cfg = mla.make_config(sh)
    if args.operand == "bf16":
        cfg.attn_operand = mla.MLA_ATTN_BF16
    W = {k: tb(v) for k, v in case.w.items()}
    x = tb(case.x)
    n = case.x.shape[0]
    cuh = case.cu_seqlens
    cu = torch.from_numpy(cuh).to(dev)
    maxlen = int(np.max(np.diff(cuh)))
    cos = sin = None
    if sh.rope.kind != "none":
        cos, sin = mla.rope_table(cfg, maxlen, dev)
    out = torch.empty(n, sh.hidden, dtype=torch.bfloat16, device=dev)
    lat = torch.empty(n, sh.kv_lora_rank + sh.qk_rope_dim, dtype=torch.bfloat16, device=dev)
    ws_p = torch.empty(mla.prefill_workspace_size(cfg, n, len(cuh) - 1), dtype=torch.uint8, device=dev)
    del case

    # ------------------------------------------------------------------ decode inputs
    dsh = mi.WORKLOADS[args.decode]
    dc = mi.make_decode_case(dsh)
    dcfg = mla.make_config(dsh)
    w_kvb, q_nope, q_pe, cache = tb(dc.w_kv_b), tb(dc.q_nope), tb(dc.q_pe), tb(dc.cache)
    table = torch.from_numpy(dc.block_table).to(dev)
    lens_d = torch.from_numpy(dc.seq_lens).to(dev)
    lens_h = dc.seq_lens.copy()
    B = len(lens_h)
    out_d = torch.empty(B, dsh.num_heads, dsh.v_head_dim, dtype=torch.bfloat16, device=dev)
    ws_d = torch.empty(mla.decode_workspace_size(dcfg, lens_h), dtype=torch.uint8, device=dev)
    max_blocks = dc.block_table.shape[1]
    del dc

    # the same cache in E4M3 (one scale), converted by the library
    FP8_SCALE = 1.0 / 32.0
    cache8 = torch.empty(cache.shape, dtype=torch.uint8, device=dev)
    mla.cache_quantize_fp8(cache, FP8_SCALE, cache8)
    ws_d8 = torch.empty(mla.decode_fp8_workspace_size(dcfg, lens_h), dtype=torch.uint8, device=dev)

    def prefill():
        mla.prefill_fwd(cfg, W, x, cu, cuh, out, latent_out=lat, rope_cos=cos, rope_sin=sin, workspace=ws_p)

    def decode_fp8():
        mla.decode_absorbed_fp8_fwd(dcfg, w_kvb, q_nope, q_pe, cache8, FP8_SCALE, table, lens_d, lens_h, out_d,
                                    workspace=ws_d8)

    def decode():
        mla.decode_absorbed_fwd(dcfg, w_kvb, q_nope, q_pe, cache, table, lens_d, lens_h, out_d, workspace=ws_d)

    # the fused latent norm + RoPE (a5) on the layer's [N, r_kv + d_rope] rows
    norm_src = torch.randn(n, sh.kv_lora_rank + sh.qk_rope_dim, device=dev).to(torch.bfloat16)
    norm_dst = torch.empty_like(norm_src)
    norm_pos = torch.from_numpy(np.concatenate([np.arange(b - a) for a, b in zip(cuh[:-1], cuh[1:])]).astype(np.int32)).to(dev)

    def norm_rope():
        mla.latent_norm_rope(cfg, norm_src, n, sh.kv_lora_rank + sh.qk_rope_dim, sh.kv_lora_rank, W["kv_a_gamma"],
                             norm_dst, rope_offset=sh.kv_lora_rank, rope_slices=1 if cos is not None else 0,
                             rope_slice_stride=sh.qk_rope_dim, rope_cos=cos, rope_sin=sin, positions=norm_pos)

    # ------------------------------------------------------------------ chunked prefill inputs
    chunk = None
    if args.chunk != "none" and args.mode in ("full", "chunk", "chunk_attention"):
        cname, cch, cpre = CHUNK_WORKLOADS[args.chunk]
        csh = mi.WORKLOADS[cname]
        cc = mi.make_chunk_case(csh, cch, cpre, block_size=64)
        ccfg = mla.make_config(csh)
        cW = W if cname == args.prefill else {k: tb(v) for k, v in cc.w.items()}
        c_n = cc.x.shape[0]
        ccu_h, cpre_h = cc.cu_seqlens, cc.prefix_lens
        ccos, csin = cos, sin
        longest = int(np.max(cpre_h + np.diff(ccu_h)))
        if csh.rope.kind != "none":
            ccos, csin = mla.rope_table(ccfg, longest, dev)
        chunk = dict(
            name=args.chunk, sh=csh, cfg=ccfg, W=cW, x=tb(cc.x), cu=torch.from_numpy(ccu_h).to(dev), cu_h=ccu_h,
            pre=torch.from_numpy(cpre_h).to(dev), pre_h=cpre_h, cache=tb(cc.cache),
            table=torch.from_numpy(cc.block_table).to(dev), cos=ccos, sin=csin, chunks=cch, prefixes=cpre,
            out=torch.empty(c_n, csh.hidden, dtype=torch.bfloat16, device=dev),
            lat=torch.empty(c_n, csh.kv_lora_rank + csh.qk_rope_dim, dtype=torch.bfloat16, device=dev),
            ws=torch.empty(mla.prefill_chunk_workspace_size(ccfg, ccu_h, cpre_h), dtype=torch.uint8, device=dev))
        del cc

    def chunk_layer():
        c = chunk
        mla.prefill_chunk_fwd(c["cfg"], c["W"], c["x"], c["cu"], c["cu_h"], c["pre"], c["pre_h"], c["cache"],
                              c["table"], c["out"], latent_out=c["lat"], rope_cos=c["cos"], rope_sin=c["sin"],
                              workspace=c["ws"])

    def chunk_attention_operands():
        # fp16 operands of the chunk layer's attention shapes (keys = context rows)
        c = chunk
        csh = c["sh"]
        ck_h = np.concatenate([[0], np.cumsum(np.asarray(c["prefixes"]) + np.asarray(c["chunks"]))]).astype(np.int32)
        g = torch.Generator(device=dev).manual_seed(1)
        Hc, nq, nk = csh.num_heads, int(c["cu_h"][-1]), int(ck_h[-1])
        qa = torch.randn(nq, Hc, csh.qk_head_dim, device=dev, generator=g).to(torch.float16)
        kva = torch.randn(nk, Hc, csh.qk_nope_dim + csh.v_head_dim, device=dev, generator=g).to(torch.float16)
        kpe = torch.randn(nk, csh.qk_rope_dim, device=dev, generator=g).to(torch.float16)
        attn = torch.empty(nq, Hc, csh.v_head_dim, dtype=torch.bfloat16, device=dev)
        ck = torch.from_numpy(ck_h).to(dev)
        return lambda: mla.attention_prefix(c["cfg"], qa, kva, kpe, c["cu"], c["cu_h"], ck, ck_h, attn)

    # the layer backward on the same layer (seeded N(0, 1) output gradient)
    lbw = {}

    def prefill_bwd():
        if not lbw:
            g = torch.Generator(device=dev).manual_seed(11)
            lbw["dout"] = torch.randn(n, sh.hidden, device=dev, generator=g).to(torch.bfloat16)
            lbw["dx"] = torch.empty(n, sh.hidden, dtype=torch.float32, device=dev)
            lbw["grads"] = {k: torch.empty(v.shape, dtype=torch.float32, device=dev) for k, v in W.items()
                            if v is not None and not (k == "w_o" and sh.o_groups)}
            lbw["ws"] = torch.empty(mla.prefill_bwd_workspace_size(cfg, n), dtype=torch.uint8, device=dev)
        mla.prefill_bwd(cfg, W, x, cu, cuh, lbw["dout"], lbw["dx"], lbw["grads"], rope_cos=cos, rope_sin=sin,
                        workspace=lbw["ws"])

    def step():
        prefill()
        decode()

    if args.mode != "full":
        # profiler runs: only the requested part, warmup + steps launches, no JSON line
        if args.mode == "attention":
            fn = attention_operands(args.attn_workload)["run"](args.operand)
        elif args.mode == "attention_bwd":
            fn = attention_operands(args.attn_workload)["bwd"]()
        elif args.mode == "chunk_attention":
            fn = chunk_attention_operands()
        elif args.mode == "chunk":
            fn = chunk_layer
        elif args.mode == "norm":
            fn = norm_rope
        elif args.mode == "copy":
            # known-size device copy: calibrates the FETCH_SIZE / WRITE_SIZE counters
            src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            fn = lambda: dst.copy_(src)
        elif args.mode == "decode_fp8":
            fn = decode_fp8
        elif args.mode == "prefill_bwd":
            fn = prefill_bwd
        else:
            fn = prefill if args.mode == "prefill" else decode
        flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev) if args.mode in ("decode", "decode_fp8") else None
        sink = torch.zeros(1, dtype=torch.int64, device=dev)
        for i in range(args.warmup + args.steps):
            if flush is not None:
                sink.copy_(flush.view(torch.int64).sum())
            fn()
        torch.cuda.synchronize()
        print(f"{args.mode}: {args.warmup + args.steps} launches done", flush=True)
        return

    # ------------------------------------------------------------------ whole steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_wall = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        pe[i][0].record(stream)
        prefill()
        pe[i][1].record(stream)
        decode()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = e0.elapsed_time(e1) / args.steps
    prefill_ms = sum(a.elapsed_time(b) for a, b in pe) / args.steps
    print(f"steps done: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------ the same layer with the grouped low-rank
    # output projection (8 groups x 1024, the guide's grouping), seeded N(0, 0.02) W_o_a / W_o_b
    grouped_rec = None
    if sh.o_groups == 0 and (sh.num_heads * sh.v_head_dim) % 8 == 0:
        gsh = sh.replace(o_groups=8, o_lora_rank=1024)
        gcfg = mla.make_config(gsh)
        gcfg.attn_operand = cfg.attn_operand
        gg = torch.Generator(device=dev).manual_seed(13)
        fg = sh.num_heads * sh.v_head_dim // 8
        Wg = dict(W)
        Wg["w_o"] = None
        Wg["w_o_a"] = (0.02 * torch.randn(8 * 1024, fg, device=dev, generator=gg)).to(torch.bfloat16)
        Wg["w_o_b"] = (0.02 * torch.randn(sh.hidden, 8 * 1024, device=dev, generator=gg)).to(torch.bfloat16)
        ws_g = torch.empty(mla.prefill_workspace_size(gcfg, n, len(cuh) - 1), dtype=torch.uint8, device=dev)
        grouped = lambda: mla.prefill_fwd(gcfg, Wg, x, cu, cuh, out, latent_out=lat, rope_cos=cos, rope_sin=sin,
                                          workspace=ws_g)
        g_ms = timed(grouped, args.steps, warm=5)
        g_fl = layer_flops(gsh, n, attention_flops(sh, cuh))
        grouped_rec = {"workload": f"{args.prefill} with the output projection as 8 groups x 1024 (W_o_a, W_o_b)",
                       "layer_ms": round(g_ms, 4), "layer_tflops": round(g_fl / (g_ms * 1e-3) / 1e12, 2)}
        try:
            gc = device_kernels(torch, grouped, 3)
            gl = layer_gemms(gsh, n)
            gem = [[us for nm, us in c if "gemm" in nm] for c in gc]
            if all(len(c) == len(gl) for c in gem):
                for i, (nm, fl) in enumerate(gl):
                    if nm in ("o_a", "o_b"):
                        us = sum(c[i] for c in gem) / len(gem)
                        grouped_rec[nm] = {"us": round(us, 1), "tflops": round(fl / (us * 1e-6) / 1e12, 1),
                                           "frac": round(fl / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4)}
        except Exception as ex:
            grouped_rec["breakdown_error"] = f"{type(ex).__name__}: {ex}"[:200]
        del Wg, ws_g
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ attention kernel alone, graded workloads
    # warm-up launches bring the GPU to the kernel's steady state after the
    # layer steps (power and clock state, caches)
    attn_rec = {}
    bwd_rec = None
    for name in ATTN_WORKLOADS:
        ao = attention_operands(name)
        for operand in (("f16", "bf16") if name == args.prefill else ("f16",)):
            ms = timed(ao["run"](operand), args.steps, warm=max(20, args.warmup))
            tf = ao["flops"] / (ms * 1e-3) / 1e12
            attn_rec[f"{name}/{operand}"] = {"ms": round(ms, 4), "tflops": round(tf, 2),
                                              "frac": round(tf / PEAK_MFMA_TFLOPS, 4), "flops": ao["flops"]}
        if name == args.prefill:
            # the attention backward on the same workload (bf16 operands, fp32 gradients)
            b_ms = timed(ao["bwd"](), args.steps, warm=10)
            b_tf = ao["bwd_flops"] / (b_ms * 1e-3) / 1e12
            bwd_rec = {"workload": f"{name}, bf16 operands, fp32 dq / dkv / dkpe", "ms": round(b_ms, 4),
                       "tflops": round(b_tf, 2), "frac": round(b_tf / PEAK_MFMA_TFLOPS, 4),
                       "flops_per_launch": ao["bwd_flops"],
                       "kernel": "mla_attention_prefill_bwd with the forward's log-sum-exp (dq pass forming D, "
                                 "dk/dv pass, k_pe head sum)"}
        del ao
        torch.cuda.empty_cache()
        print(f"attention {name} done", file=sys.stderr, flush=True)
    head = attn_rec[f"{args.prefill}/f16"]
    attn_ms, attn_tflops, a_flops = head["ms"], head["tflops"], head["flops"]

    # ------------------------------------------------------------------ layer backward (recompute + chain rule)
    lb_ms = timed(prefill_bwd, max(3, args.steps // 4), warm=2)
    lb_flops = 2 * layer_flops(sh, n, 0) + attention_bwd_flops(sh, cuh)
    lbw.clear()
    torch.cuda.empty_cache()
    layer_bwd_rec = {"workload": f"{args.prefill}, bf16, fp32 dx and weight gradients", "ms": round(lb_ms, 3),
                     "tflops": round(lb_flops / (lb_ms * 1e-3) / 1e12, 2),
                     "frac": round(lb_flops / (lb_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                     "flops_per_call": lb_flops,
                     "flops_counted": "dX and dW of every projection (twice the forward's) + the attention backward; "
                                      "the forward recompute inside the call is not counted"}

    # ------------------------------------------------------------------ fused query up-projection + RoPE + MXFP8
    mxq = None
    if sh.q_lora_rank > 0:
        Hq, dqk = sh.num_heads, sh.qk_nope_dim + sh.qk_rope_dim
        g = torch.Generator(device=dev).manual_seed(5)
        qlat = torch.randn(n, sh.q_lora_rank, device=dev, generator=g).to(torch.bfloat16)
        qc = torch.empty(n, Hq * dqk, dtype=torch.uint8, device=dev)
        qs = torch.empty(n, Hq * dqk // 32, dtype=torch.uint8, device=dev)
        qpos = torch.from_numpy(np.concatenate([np.arange(b - a) for a, b in zip(cuh[:-1], cuh[1:])]).astype(np.int32)).to(dev)
        mx_ms = timed(lambda: mla.q_uproj_rope_mxfp8(cfg, qlat, W["w_q_b"], qpos if cos is not None else None, cos,
                                                     sin, qc, qs), args.steps, warm=10)
        mx_flops = 2.0 * n * sh.q_lora_rank * Hq * dqk
        mxq = {"workload": f"{args.prefill} query latent [{n}, {sh.q_lora_rank}] -> [{n}, {Hq * dqk}] E4M3 + E8M0",
               "us": round(mx_ms * 1e3, 1), "tflops": round(mx_flops / (mx_ms * 1e-3) / 1e12, 1),
               "frac": round(mx_flops / (mx_ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4), "flops": mx_flops}
        del qlat, qc, qs

    # ------------------------------------------------------------------ fused latent norm + RoPE (a5)
    norm_ms = timed(norm_rope, 50, warm=20)
    lw = sh.kv_lora_rank + sh.qk_rope_dim
    norm_bytes = n * lw * 2 * 2 + n * 4 + n * sh.qk_rope_dim * 4 + sh.kv_lora_rank * 2   # rows in/out, positions, cos/sin rows, gain
    norm_gbs = norm_bytes / (norm_ms * 1e-3) / 1e9

    # ------------------------------------------------------------------ decode call alone (cold Infinity Cache)
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int64, device=dev)
    de = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # decode in its own steady state: 20 warm-up calls, each after the flush as
    # the timed ones
    for _ in range(20):
        sink.copy_(flush.view(torch.int64).sum())
        decode()
    for i in range(args.steps):
        sink.copy_(flush.view(torch.int64).sum())
        de[i][0].record(stream)
        decode()
        de[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = sum(a.elapsed_time(b) for a, b in de) / args.steps
    # the decode over the E4M3 copy of the cache, timed the same way
    for _ in range(20):
        sink.copy_(flush.view(torch.int64).sum())
        decode_fp8()
    for i in range(args.steps):
        sink.copy_(flush.view(torch.int64).sum())
        de[i][0].record(stream)
        decode_fp8()
        de[i][1].record(stream)
    torch.cuda.synchronize()
    dec8_ms = sum(a.elapsed_time(b) for a, b in de) / args.steps
    del flush

    # ------------------------------------------------------------------ chunked prefill (reported beside the metric)
    chunk_rec = None
    if chunk is not None:
        c_layer_ms = timed(chunk_layer, args.steps)
        c_attn_ms = timed(chunk_attention_operands(), args.steps)
        csh = chunk["sh"]
        c_aflops = prefix_attention_flops(csh, chunk["chunks"], chunk["prefixes"])
        c_tflops = c_aflops / (c_attn_ms * 1e-3) / 1e12
        # layer FLOPs: the new tokens' projections, the up-projection of every context row, the attention
        n_new, n_ctx = int(chunk["cu_h"][-1]), int(sum(chunk["chunks"]) + sum(chunk["prefixes"]))
        c_lflops = (layer_flops(csh, n_new, c_aflops)
                    + 2 * (n_ctx - n_new) * csh.kv_lora_rank * csh.num_heads * (csh.qk_nope_dim + csh.v_head_dim))
        chunk_rec = {"workload": chunk["name"], "new_tokens": n_new, "context_tokens": n_ctx,
                     "layer_ms": round(c_layer_ms, 4), "layer_tflops": round(c_lflops / (c_layer_ms * 1e-3) / 1e12, 2),
                     "attn_ms": round(c_attn_ms, 4), "attn_tflops": round(c_tflops, 2),
                     "roofline": {"bound": "mfma", "achieved": round(c_tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(c_tflops / PEAK_MFMA_TFLOPS, 4),
                                  "traffic": traffic_for("chunk"),
                                  "kernel": "flash_mfma_kernel<fp16> (queries over cached + new keys)",
                                  "flops_per_launch": c_aflops}}
        del chunk

    # ------------------------------------------------------------------ per-kernel breakdown (profiler device times)
    breakdown = None
    try:
        reps = 3
        lcalls = device_kernels(torch, prefill, reps)
        gl = layer_gemms(sh, n)
        gem = [[us for nm, us in c if "gemm" in nm] for c in lcalls]
        per_gemm = None
        if all(len(c) == len(gl) for c in gem):
            per_gemm = {}
            for i, (nm, fl) in enumerate(gl):
                us = sum(c[i] for c in gem) / reps
                per_gemm[nm] = {"us": round(us, 1), "tflops": round(fl / (us * 1e-6) / 1e12, 1),
                                "frac": round(fl / (us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4)}
        layer_kernel_us = sum(us for c in lcalls for _, us in c) / reps
        flush_b = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        sink_b = torch.zeros(1, dtype=torch.int64, device=dev)
        dcalls = device_kernels(torch, decode, reps, between=lambda: sink_b.copy_(flush_b.view(torch.int64).sum()))
        del flush_b
        ncalls = device_kernels(torch, norm_rope, reps)
        norm_dev_us = sum(us for c in ncalls for _, us in c) / reps
        dk = {}
        for key in ("absorb_q", "decode_split", "decode_combine"):
            t = [sum(us for nm, us in c if key in nm) for c in dcalls]
            dk[key] = sum(t) / reps
        keys_tot = int(lens_h.sum())
        cache_b = keys_tot * (dsh.kv_lora_rank + dsh.qk_rope_dim) * 2
        sp_flops = keys_tot * dsh.num_heads * 2 * ((dsh.kv_lora_rank + dsh.qk_rope_dim) + dsh.kv_lora_rank)
        sp_us = dk["decode_split"]
        breakdown = {
            "source": "torch.profiler device durations, mean of 3 calls (the decode after a 512 MiB flush)",
            "prefill_layer_kernels_us": round(layer_kernel_us, 1),
            "prefill_gemms": per_gemm,
            "latent_norm_rope_kernel": {"us": round(norm_dev_us, 2),
                                        "gbs": round(norm_bytes / (norm_dev_us * 1e-6) / 1e9, 1),
                                        "frac": round(norm_bytes / (norm_dev_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
            "decode_kernels_us": {k: round(v, 1) for k, v in dk.items()},
            "decode_split_kernel": {"us": round(sp_us, 1), "cache_bytes": cache_b,
                                    "cache_gbs": round(cache_b / (sp_us * 1e-6) / 1e9, 1),
                                    "frac_hbm": round(cache_b / (sp_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                                    "tflops": round(sp_flops / (sp_us * 1e-6) / 1e12, 1),
                                    "frac_mfma": round(sp_flops / (sp_us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS, 4)},
        }
    except Exception as ex:                      # the profiler is optional: report why it is missing
        breakdown = {"error": f"{type(ex).__name__}: {ex}"[:200]}

    # ------------------------------------------------------------------ figures
    layer_tflops = layer_flops(sh, n, a_flops) / (prefill_ms * 1e-3) / 1e12
    d_bytes = decode_bytes(dsh, lens_h, max_blocks)
    dec_gbs = d_bytes / (dec_ms * 1e-3) / 1e9
    d8_bytes = d_bytes - int(lens_h.sum()) * (dsh.kv_lora_rank + dsh.qk_rope_dim)   # one byte per cached value
    dec8_gbs = d8_bytes / (dec8_ms * 1e-3) / 1e9
    value = 0.5 * (attn_tflops / PEAK_MFMA_TFLOPS + dec_gbs / PEAK_HBM_GBS) * 100

    rec = {
        "metric": METRIC, "value": round(value, 3),
        "unit": "% of MI355X peak (mean of prefill-attention MFMA and absorbed-decode HBM fractions)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 MFMA (prefill attention operands) + bf16 MFMA (decode); fp32 accumulate and softmax; bf16 I/O",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights, bf16)",
        "config": {"workload": f"{args.prefill} + {args.decode}", "prefill_tokens": n, "prefill_docs": len(cuh) - 1,
                   "heads": sh.num_heads, "hidden": sh.hidden, "q_lora_rank": sh.q_lora_rank,
                   "kv_lora_rank": sh.kv_lora_rank, "decode_batch": B, "decode_keys": int(lens_h.sum()),
                   "decode_block": 64, "prefill_attn_operand": args.operand},
        "prefill_attn_tflops": round(attn_tflops, 2), "prefill_attn_ms": round(attn_ms, 4),
        "prefill_layer_ms": round(prefill_ms, 4), "prefill_layer_tflops": round(layer_tflops, 2),
        "decode_ms": round(dec_ms, 4), "decode_hbm_gbs": round(dec_gbs, 1),
        "attention_by_workload": attn_rec,
        "latent_norm_rope": {"workload": f"{args.prefill} latent rows [{n}, {lw}] bf16, norm 512 + RoPE 64",
                             "us": round(norm_ms * 1e3, 2), "gbs": round(norm_gbs, 1),
                             "frac": round(norm_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": norm_bytes},
        "wall_s_timed": round(t_wall, 3),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4), "traffic": traffic_for("flash"),
                     "kernel": "flash_mfma_kernel<fp16> (prefill attention)", "flops_per_launch": a_flops},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for("decode"),
                            "kernel": "mla_decode_absorbed_fwd (query absorption + split-KV attention + fused combine and un-absorb)",
                            "bytes_per_call": d_bytes},
    }
    if mxq is not None:
        rec["q_uproj_rope_mxfp8"] = mxq
    rec["decode_fp8_cache"] = {
        "workload": f"{args.decode} with the cache in E4M3 (scale {FP8_SCALE}), mla_decode_absorbed_fp8_fwd",
        "ms": round(dec8_ms, 4), "speedup_vs_bf16_cache": round(dec_ms / dec8_ms, 3),
        "roofline": {"bound": "hbm", "achieved": round(dec8_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dec8_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for("decode_fp8"),
                     "bytes_per_call": d8_bytes}}
    if chunk_rec is not None:
        rec["chunked_prefill"] = chunk_rec
    rec["kernel_breakdown"] = breakdown
    if grouped_rec is not None:
        rec["grouped_o_proj_layer"] = grouped_rec
    if bwd_rec is not None:
        rec["attention_backward"] = bwd_rec
    rec["layer_backward"] = layer_bwd_rec
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.prefill, args.decode, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
