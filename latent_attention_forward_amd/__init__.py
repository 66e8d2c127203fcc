"""Python binding of libmla (MLA forward for MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmla.so``.  PyTorch provides device memory and the current stream.  The
names follow the C ABI in ``include/mla.h``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_MISALIGNED, MLA_ERR_HIP = range(6)
MLA_BF16, MLA_F32, MLA_F16 = 0, 1, 2
MLA_ROPE_NONE, MLA_ROPE_PLAIN, MLA_ROPE_YARN = 0, 1, 2


class MLAError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func} failed with status {status}: {msg}")
        self.status = status


class MlaConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("q_lora_rank", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32), ("qk_nope_dim", ctypes.c_int32), ("qk_rope_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_kind", ctypes.c_int32),
        ("yarn_original_max_pos", ctypes.c_int32), ("output_gate", ctypes.c_int32),
        ("norm_eps", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("rope_theta", ctypes.c_double), ("yarn_factor", ctypes.c_double), ("yarn_beta_fast", ctypes.c_double),
        ("yarn_beta_slow", ctypes.c_double), ("yarn_mscale", ctypes.c_double), ("yarn_mscale_all_dim", ctypes.c_double),
        ("rope_interleave", ctypes.c_int32), ("o_groups", ctypes.c_int32), ("o_lora_rank", ctypes.c_int32),
    ]


class MlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_q_a", "q_a_gamma", "w_q_b", "w_q", "w_kv_a", "kv_a_gamma", "w_kv_b", "w_o", "w_g", "w_o_a",
                 "w_o_b")]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_CFG = ctypes.POINTER(MlaConfig)

_SIGNATURES = {
    "mla_abi_version": (_I32, []),
    "mla_validate_config": (_I32, [_CFG]),
    "mla_softmax_scale": (ctypes.c_float, [_CFG]),
    "mla_rope_table": (_I32, [_CFG, _I32, _P, _P]),
    "mla_prefill_workspace_size": (_SZ, [_CFG, _I32, _I32]),
    "mla_decode_workspace_size": (_SZ, [_CFG, _P, _I32]),
    "mla_status_string": (ctypes.c_char_p, [_I32]),
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_latent_norm_rope": (_I32, [_CFG, _P, _I64, _I32, _I32, _I32, _P, _I32, _I32, _I32, _P, _P, _I32, _P,
                                    _P, _I64, _P, _I64, _P]),
    "mla_linear": (_I32, [_CFG, _P, _I64, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "mla_attention_prefill": (_I32, [_CFG, _I32, _P, _P, _P, _I64, _P, _P, _I32, _P, _P, _SZ, _P]),
    "mla_prefill_fwd": (_I32, [_CFG, ctypes.POINTER(MlaWeights), _P, _P, _P, _I32, _P, _P, _P, _I32, _P, _P,
                               _P, _SZ, _P]),
    "mla_decode_absorbed_fwd": (_I32, [_CFG, _P, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _P, _SZ, _P]),
    "mla_prefill_chunk_workspace_size": (_SZ, [_CFG, _P, _P, _I32]),
    "mla_attention_prefix": (_I32, [_CFG, _I32, _P, _P, _P, _I64, _P, _P, _P, _P, _I32, _P, _P]),
    "mla_prefill_chunk_fwd": (_I32, [_CFG, ctypes.POINTER(MlaWeights), _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P,
                                     _I32, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
}

_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmla.so (built in-tree by ``latent_attention_forward_amd.build``).
    Raises when it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmla.so not found at {p}; build it with "
                           "`python -m latent_attention_forward_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return list(_SIGNATURES)


def _check(status: int, func: str):
    if status != MLA_OK:
        msg = load_library().mla_last_error().decode()
        raise MLAError(status, func, msg)


# --------------------------------------------------------------------------- config
def make_config(shape=None, *, softmax_scale: float = 0.0, **kw) -> MlaConfig:
    """Build an ``MlaConfig`` from any object with the attribute names of
    ``mla_inputs.MLAShape`` (hidden, num_heads, q_lora_rank, kv_lora_rank,
    qk_nope_dim, qk_rope_dim, v_head_dim, dtype "bf16"/"f32", rope (kind,
    theta, factor, original_max_pos, beta_fast, beta_slow, mscale,
    mscale_all_dim), output_gate, norm_eps, and optionally rope_interleave,
    o_groups, o_lora_rank), or from keyword arguments."""
    c = MlaConfig()
    if shape is not None:
        r = shape.rope
        c.hidden, c.num_heads, c.q_lora_rank = shape.hidden, shape.num_heads, shape.q_lora_rank
        c.kv_lora_rank, c.qk_nope_dim, c.qk_rope_dim = shape.kv_lora_rank, shape.qk_nope_dim, shape.qk_rope_dim
        c.v_head_dim = shape.v_head_dim
        c.dtype = MLA_BF16 if shape.dtype == "bf16" else MLA_F32
        c.rope_kind = {"none": MLA_ROPE_NONE, "plain": MLA_ROPE_PLAIN, "yarn": MLA_ROPE_YARN}[r.kind]
        c.rope_theta, c.yarn_factor = r.theta, r.factor
        c.yarn_original_max_pos, c.yarn_beta_fast, c.yarn_beta_slow = r.original_max_pos, r.beta_fast, r.beta_slow
        c.yarn_mscale, c.yarn_mscale_all_dim = r.mscale, r.mscale_all_dim
        c.output_gate = int(shape.output_gate)
        c.norm_eps = shape.norm_eps
        c.rope_interleave = int(getattr(shape, "rope_interleave", False))
        c.o_groups = int(getattr(shape, "o_groups", 0))
        c.o_lora_rank = int(getattr(shape, "o_lora_rank", 0))
    for k, v in kw.items():
        setattr(c, k, v)
    c.softmax_scale = softmax_scale
    return c


def softmax_scale(cfg: MlaConfig) -> float:
    return float(load_library().mla_softmax_scale(ctypes.byref(cfg)))


def validate_config(cfg: MlaConfig) -> None:
    _check(load_library().mla_validate_config(ctypes.byref(cfg)), "mla_validate_config")


def rope_table_host(cfg: MlaConfig, max_pos: int):
    """(cos, sin) as float32 numpy arrays [max_pos, d_rope/2], built by the library."""
    import numpy as np
    half = cfg.qk_rope_dim // 2
    cos = np.empty((max_pos, half), np.float32)
    sin = np.empty((max_pos, half), np.float32)
    _check(load_library().mla_rope_table(ctypes.byref(cfg), max_pos, cos.ctypes.data, sin.ctypes.data),
           "mla_rope_table")
    return cos, sin


def rope_table(cfg: MlaConfig, max_pos: int, device="cuda"):
    import torch
    cos, sin = rope_table_host(cfg, max_pos)
    return torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device)


def prefill_workspace_size(cfg: MlaConfig, num_tokens: int, num_seqs: int) -> int:
    return int(load_library().mla_prefill_workspace_size(ctypes.byref(cfg), num_tokens, num_seqs))


def decode_workspace_size(cfg: MlaConfig, seq_lens_host) -> int:
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    return int(load_library().mla_decode_workspace_size(ctypes.byref(cfg), lens.ctypes.data, len(lens)))


# --------------------------------------------------------------------------- device calls
def _ptr(t, rows: bool = False) -> Optional[int]:
    """Device address of a tensor argument.  The library takes raw device
    pointers, so a host tensor, or a layout the call does not describe, is
    refused here rather than read wrongly: the tensor must live on a GPU and
    be contiguous (with ``rows``, only its last dimension must be contiguous:
    the call takes the row stride as an argument)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments of the library calls must be GPU tensors")
    if rows:
        if t.dim() > 0 and t.stride(-1) != 1:
            raise ValueError("a row-strided tensor argument needs a contiguous last dimension")
    elif not t.is_contiguous():
        raise ValueError("tensor arguments of the library calls must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, workspace=None):
    import torch
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def latent_norm_rope(cfg: MlaConfig, src, n_rows: int, row_width: int, norm_dim: int, gamma, dst,
                     rope_offset: int = 0, rope_slices: int = 0, rope_slice_stride: int = 0,
                     rope_cos=None, rope_sin=None, positions=None, slot_mapping=None, num_slots: int = 0,
                     src_row_stride: Optional[int] = None, dst_row_stride: Optional[int] = None, stream=None):
    lib = load_library()
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    st = lib.mla_latent_norm_rope(
        ctypes.byref(cfg), _ptr(src, rows=True), src.stride(0) if src_row_stride is None else src_row_stride, n_rows,
        row_width, norm_dim, _ptr(gamma), rope_offset, rope_slices, rope_slice_stride, _ptr(rope_cos),
        _ptr(rope_sin), table_len, _ptr(positions), _ptr(dst, rows=True),
        dst.stride(0) if dst_row_stride is None else dst_row_stride, _ptr(slot_mapping), num_slots, _stream(stream))
    _check(st, "mla_latent_norm_rope")


def linear(cfg: MlaConfig, x, w, y, stream=None):
    lib = load_library()
    m, k = x.shape
    n = w.shape[0]
    _check(lib.mla_linear(ctypes.byref(cfg), _ptr(x, rows=True), x.stride(0), _ptr(w), _ptr(y, rows=True), y.stride(0), m, n, k,
                          _stream(stream)), "mla_linear")


def attention_prefill(cfg: MlaConfig, q, kv, kpe, cu_seqlens_dev, cu_seqlens_host: Sequence[int], attn,
                      kpe_stride: Optional[int] = None, stream=None):
    """Attention core.  ``kpe`` is a view whose row r is the shared rope key of
    token r (e.g. ``latent[:, r_kv:]``); its dtype (bf16 / fp16 / fp32) sets
    the operand type."""
    import numpy as np
    import torch
    lib = load_library()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    op = {torch.bfloat16: MLA_BF16, torch.float16: MLA_F16, torch.float32: MLA_F32}[q.dtype]
    _check(lib.mla_attention_prefill(ctypes.byref(cfg), op, _ptr(q), _ptr(kv), _ptr(kpe, rows=True),
                                     kpe.stride(0) if kpe_stride is None else kpe_stride,
                                     _ptr(cu_seqlens_dev), cuh.ctypes.data, len(cuh) - 1, _ptr(attn), None, 0,
                                     _stream(stream)), "mla_attention_prefill")


def attention_prefix(cfg: MlaConfig, q, kv, kpe, cu_q_dev, cu_q_host: Sequence[int], cu_k_dev,
                     cu_k_host: Sequence[int], attn, kpe_stride: Optional[int] = None, stream=None):
    """Attention core of new queries over longer key sequences (aligned at
    the end).  ``q`` rows follow ``cu_q``, ``kv`` and ``kpe`` rows ``cu_k``."""
    import numpy as np
    import torch
    lib = load_library()
    cqh = np.ascontiguousarray(np.asarray(cu_q_host, dtype=np.int32))
    ckh = np.ascontiguousarray(np.asarray(cu_k_host, dtype=np.int32))
    op = {torch.bfloat16: MLA_BF16, torch.float16: MLA_F16, torch.float32: MLA_F32}[q.dtype]
    _check(lib.mla_attention_prefix(ctypes.byref(cfg), op, _ptr(q), _ptr(kv), _ptr(kpe, rows=True),
                                    kpe.stride(0) if kpe_stride is None else kpe_stride, _ptr(cu_q_dev),
                                    cqh.ctypes.data, _ptr(cu_k_dev), ckh.ctypes.data, len(cqh) - 1, _ptr(attn),
                                    _stream(stream)), "mla_attention_prefix")


def make_weights(w: Dict[str, object]) -> MlaWeights:
    mw = MlaWeights()
    for name, _ in MlaWeights._fields_:
        t = w.get(name)
        setattr(mw, name, _ptr(t))
    return mw


def prefill_fwd(cfg: MlaConfig, weights: Dict[str, object], x, cu_seqlens_dev, cu_seqlens_host: Sequence[int],
                out, latent_out=None, positions=None, rope_cos=None, rope_sin=None, workspace=None, stream=None):
    """The full prefill layer.  ``weights`` maps the ``MlaWeights`` field names
    to device tensors (None for absent ones)."""
    import numpy as np
    lib = load_library()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    n, s = int(cuh[-1]), len(cuh) - 1
    ws_bytes = prefill_workspace_size(cfg, n, s)
    ws = _workspace(ws_bytes, x.device, workspace)
    mw = make_weights(weights)
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib.mla_prefill_fwd(ctypes.byref(cfg), ctypes.byref(mw), _ptr(x), _ptr(cu_seqlens_dev), cuh.ctypes.data,
                               s, _ptr(positions), _ptr(rope_cos), _ptr(rope_sin), table_len, _ptr(out),
                               _ptr(latent_out), _ptr(ws), ws.numel(), _stream(stream)), "mla_prefill_fwd")
    return ws


def decode_absorbed_fwd(cfg: MlaConfig, w_kv_b, q_nope, q_pe, kv_cache, block_table, seq_lens_dev,
                        seq_lens_host: Sequence[int], out, workspace=None, stream=None):
    import numpy as np
    lib = load_library()
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    ws_bytes = decode_workspace_size(cfg, lens)
    ws = _workspace(ws_bytes, q_nope.device, workspace)
    num_blocks, block_size = kv_cache.shape[0], kv_cache.shape[1]
    _check(lib.mla_decode_absorbed_fwd(ctypes.byref(cfg), _ptr(w_kv_b), _ptr(q_nope), _ptr(q_pe), _ptr(kv_cache),
                                       num_blocks, block_size, _ptr(block_table), block_table.shape[1],
                                       _ptr(seq_lens_dev), lens.ctypes.data, len(lens), _ptr(out), _ptr(ws),
                                       ws.numel(), _stream(stream)), "mla_decode_absorbed_fwd")
    return ws


def prefill_chunk_workspace_size(cfg: MlaConfig, cu_seqlens_host: Sequence[int], prefix_lens_host: Sequence[int]) -> int:
    import numpy as np
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    pre = np.ascontiguousarray(np.asarray(prefix_lens_host, dtype=np.int32))
    return int(load_library().mla_prefill_chunk_workspace_size(ctypes.byref(cfg), cuh.ctypes.data, pre.ctypes.data,
                                                                len(cuh) - 1))


def prefill_chunk_fwd(cfg: MlaConfig, weights: Dict[str, object], x, cu_seqlens_dev, cu_seqlens_host: Sequence[int],
                      prefix_lens_dev, prefix_lens_host: Sequence[int], kv_cache, block_table, out,
                      latent_out=None, rope_cos=None, rope_sin=None, workspace=None, stream=None):
    """Prefill of new tokens over a cached latent prefix.  ``kv_cache`` is
    [num_blocks, block_size, r_kv + d_rope] (or None when every prefix is 0),
    ``block_table`` [num_seqs, max_blocks] int32."""
    import numpy as np
    lib = load_library()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    pre = np.ascontiguousarray(np.asarray(prefix_lens_host, dtype=np.int32))
    s = len(cuh) - 1
    ws = _workspace(prefill_chunk_workspace_size(cfg, cuh, pre), x.device, workspace)
    mw = make_weights(weights)
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    nb, bs = (0, 0) if kv_cache is None else (kv_cache.shape[0], kv_cache.shape[1])
    mb = 0 if block_table is None else block_table.shape[1]
    _check(lib.mla_prefill_chunk_fwd(ctypes.byref(cfg), ctypes.byref(mw), _ptr(x), _ptr(cu_seqlens_dev),
                                     cuh.ctypes.data, s, _ptr(prefix_lens_dev), pre.ctypes.data, _ptr(kv_cache), nb,
                                     bs, _ptr(block_table), mb, _ptr(rope_cos), _ptr(rope_sin), table_len, _ptr(out),
                                     _ptr(latent_out), _ptr(ws), ws.numel(), _stream(stream)),
           "mla_prefill_chunk_fwd")
    return ws
