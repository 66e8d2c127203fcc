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
MLA_ATTN_F16, MLA_ATTN_BF16 = 0, 1


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
        ("attn_operand", ctypes.c_int32),
    ]


class MlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_q_a", "q_a_gamma", "w_q_b", "w_q", "w_kv_a", "kv_a_gamma", "w_kv_b", "w_o", "w_g", "w_o_a",
                 "w_o_b")]


class MlaWeightGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n, _ in MlaWeights._fields_]


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
    "mla_attention_prefill": (_I32, [_CFG, _I32, _P, _P, _P, _I64, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "mla_prefill_fwd": (_I32, [_CFG, ctypes.POINTER(MlaWeights), _P, _P, _P, _I32, _P, _P, _P, _I32, _P, _P,
                               _P, _SZ, _P]),
    "mla_decode_absorbed_fwd": (_I32, [_CFG, _P, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _P, _SZ, _P]),
    "mla_decode_absorbed_fwd_noalloc": (_I32, [_CFG, _P, _P, _P, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _P]),
    "mla_prefill_chunk_workspace_size": (_SZ, [_CFG, _P, _P, _I32]),
    "mla_decode_fp8_workspace_size": (_SZ, [_CFG, _P, _I32]),
    "mla_attention_bwd_workspace_size": (_SZ, [_CFG, _I32]),
    "mla_prefill_bwd_workspace_size": (_SZ, [_CFG, _I32]),
    "mla_prefill_bwd": (_I32, [_CFG, ctypes.POINTER(MlaWeights), _P, _P, _P, _I32, _P, _P, _P, _I32, _P, _P,
                               ctypes.POINTER(MlaWeightGrads), _P, _SZ, _P]),
    "mla_attention_prefill_bwd": (_I32, [_CFG, _P, _P, _P, _I64, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mla_q_uproj_rope_mxfp8": (_I32, [_CFG, _P, _I64, _I32, _P, _P, _P, _P, _I32, _P, _P, _P]),
    "mla_cache_quantize_fp8": (_I32, [_P, _I64, _I64, _I32, ctypes.c_float, _P, _I64, _P]),
    "mla_decode_absorbed_fp8_fwd": (_I32, [_CFG, _P, _P, _P, _P, ctypes.c_float, _I32, _I32, _P, _I32, _P, _P, _I32,
                                           _P, _P, _SZ, _P]),
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
    o_groups, o_lora_rank, attn_operand "f16"/"bf16"), or from keyword
    arguments."""
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
        c.attn_operand = MLA_ATTN_BF16 if getattr(shape, "attn_operand", "f16") == "bf16" else MLA_ATTN_F16
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
def _ptr(t, rows: bool = False, dtype=None, name: str = "tensor") -> Optional[int]:
    """Device address of a tensor argument.  The library takes raw device
    pointers, so a host tensor, an element type other than the one the call
    reads (``dtype``), or a layout the call does not describe, is refused here
    rather than read wrongly: the tensor must live on a GPU and be contiguous
    (with ``rows``, only its last dimension must be contiguous: the call takes
    the row stride as an argument)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments of the library calls must be GPU tensors")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
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


def _i32():
    import torch
    return torch.int32


def _act(cfg: MlaConfig):
    """Element type of the activations, weights and outputs of a config."""
    import torch
    return torch.bfloat16 if cfg.dtype == MLA_BF16 else torch.float32


def _workspace(nbytes: int, device, workspace=None, stream=None):
    """The caller's workspace, or a new one.  A new workspace is allocated on
    torch's current stream; when the kernels run on another stream it is
    recorded there, so the caching allocator does not hand the memory out
    again while they may still use it."""
    import torch
    if workspace is not None:
        return workspace
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def _f32():
    import torch
    return torch.float32


def _resolve_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def latent_norm_rope(cfg: MlaConfig, src, n_rows: int, row_width: int, norm_dim: int, gamma, dst,
                     rope_offset: int = 0, rope_slices: int = 0, rope_slice_stride: int = 0,
                     rope_cos=None, rope_sin=None, positions=None, slot_mapping=None, num_slots: int = 0,
                     src_row_stride: Optional[int] = None, dst_row_stride: Optional[int] = None, stream=None):
    lib = load_library()
    act, i32, f32 = _act(cfg), _i32(), _f32()
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    st = lib.mla_latent_norm_rope(
        ctypes.byref(cfg), _ptr(src, True, act, "src"), src.stride(0) if src_row_stride is None else src_row_stride,
        n_rows, row_width, norm_dim, _ptr(gamma, dtype=act, name="gamma"), rope_offset, rope_slices,
        rope_slice_stride, _ptr(rope_cos, dtype=f32, name="rope_cos"), _ptr(rope_sin, dtype=f32, name="rope_sin"),
        table_len, _ptr(positions, dtype=i32, name="positions"), _ptr(dst, True, act, "dst"),
        dst.stride(0) if dst_row_stride is None else dst_row_stride,
        _ptr(slot_mapping, dtype=i32, name="slot_mapping"), num_slots, _stream(stream))
    _check(st, "mla_latent_norm_rope")


def linear(cfg: MlaConfig, x, w, y, stream=None):
    lib = load_library()
    act = _act(cfg)
    m, k = x.shape
    n = w.shape[0]
    _check(lib.mla_linear(ctypes.byref(cfg), _ptr(x, True, act, "x"), x.stride(0), _ptr(w, dtype=act, name="w"),
                          _ptr(y, True, act, "y"), y.stride(0), m, n, k, _stream(stream)), "mla_linear")


def _operand_type(cfg: MlaConfig, q, kv, kpe):
    """Operand type code of an attention call: q, kv and kpe must share one
    element type (bf16 or fp16 for a bf16 config, fp32 for an fp32 config)."""
    import torch
    codes = {torch.bfloat16: MLA_BF16, torch.float16: MLA_F16, torch.float32: MLA_F32}
    if q.dtype not in codes:
        raise ValueError(f"attention operands must be bf16, fp16 or fp32, got {q.dtype}")
    for name, t in (("kv", kv), ("kpe", kpe)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have the dtype of q ({q.dtype}), got {t.dtype}")
    return codes[q.dtype]


def attention_prefill(cfg: MlaConfig, q, kv, kpe, cu_seqlens_dev, cu_seqlens_host: Sequence[int], attn,
                      kpe_stride: Optional[int] = None, stream=None, lse=None):
    """Attention core.  ``kpe`` is a view whose row r is the shared rope key of
    token r (e.g. ``latent[:, r_kv:]``); its dtype (bf16 / fp16 / fp32, the
    same as q and kv) sets the operand type.  ``lse``: optional fp32 [H, N]
    receiving the base-2 log-sum-exp for ``attention_prefill_bwd``."""
    import numpy as np
    lib = load_library()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    op = _operand_type(cfg, q, kv, kpe)
    _check(lib.mla_attention_prefill(ctypes.byref(cfg), op, _ptr(q), _ptr(kv), _ptr(kpe, rows=True),
                                     kpe.stride(0) if kpe_stride is None else kpe_stride,
                                     _ptr(cu_seqlens_dev, dtype=_i32(), name="cu_seqlens_dev"), cuh.ctypes.data,
                                     len(cuh) - 1, _ptr(attn, dtype=_act(cfg), name="attn"),
                                     None if lse is None else _ptr(lse, dtype=_f32(), name="lse"), None, 0,
                                     _stream(stream)), "mla_attention_prefill")


def attention_prefix(cfg: MlaConfig, q, kv, kpe, cu_q_dev, cu_q_host: Sequence[int], cu_k_dev,
                     cu_k_host: Sequence[int], attn, kpe_stride: Optional[int] = None, stream=None):
    """Attention core of new queries over longer key sequences (aligned at
    the end).  ``q`` rows follow ``cu_q``, ``kv`` and ``kpe`` rows ``cu_k``."""
    import numpy as np
    lib = load_library()
    cqh = np.ascontiguousarray(np.asarray(cu_q_host, dtype=np.int32))
    ckh = np.ascontiguousarray(np.asarray(cu_k_host, dtype=np.int32))
    op = _operand_type(cfg, q, kv, kpe)
    i32 = _i32()
    _check(lib.mla_attention_prefix(ctypes.byref(cfg), op, _ptr(q), _ptr(kv), _ptr(kpe, rows=True),
                                    kpe.stride(0) if kpe_stride is None else kpe_stride,
                                    _ptr(cu_q_dev, dtype=i32, name="cu_q_dev"), cqh.ctypes.data,
                                    _ptr(cu_k_dev, dtype=i32, name="cu_k_dev"), ckh.ctypes.data, len(cqh) - 1,
                                    _ptr(attn, dtype=_act(cfg), name="attn"), _stream(stream)),
           "mla_attention_prefix")


def make_weights(w: Dict[str, object], dtype=None) -> MlaWeights:
    """``MlaWeights`` from a dict of device tensors (absent names are NULL);
    with ``dtype`` every weight must have that element type."""
    mw = MlaWeights()
    for name, _ in MlaWeights._fields_:
        t = w.get(name)
        setattr(mw, name, _ptr(t, dtype=dtype, name=name))
    return mw


def prefill_fwd(cfg: MlaConfig, weights: Dict[str, object], x, cu_seqlens_dev, cu_seqlens_host: Sequence[int],
                out, latent_out=None, positions=None, rope_cos=None, rope_sin=None, workspace=None, stream=None):
    """The full prefill layer.  ``weights`` maps the ``MlaWeights`` field names
    to device tensors (None for absent ones)."""
    import numpy as np
    lib = load_library()
    act, i32, f32 = _act(cfg), _i32(), _f32()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    n, s = int(cuh[-1]), len(cuh) - 1
    ws_bytes = prefill_workspace_size(cfg, n, s)
    st = _resolve_stream(stream)
    ws = _workspace(ws_bytes, x.device, workspace, st)
    mw = make_weights(weights, act)
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib.mla_prefill_fwd(ctypes.byref(cfg), ctypes.byref(mw), _ptr(x, dtype=act, name="x"),
                               _ptr(cu_seqlens_dev, dtype=i32, name="cu_seqlens_dev"), cuh.ctypes.data, s,
                               _ptr(positions, dtype=i32, name="positions"),
                               _ptr(rope_cos, dtype=f32, name="rope_cos"), _ptr(rope_sin, dtype=f32, name="rope_sin"),
                               table_len, _ptr(out, dtype=act, name="out"),
                               _ptr(latent_out, dtype=act, name="latent_out"), _ptr(ws), ws.numel(),
                               st.cuda_stream), "mla_prefill_fwd")
    return ws


def prefill_bwd_workspace_size(cfg: MlaConfig, num_tokens: int) -> int:
    """Bytes of workspace ``mla_prefill_bwd`` needs for N tokens."""
    return int(load_library().mla_prefill_bwd_workspace_size(ctypes.byref(cfg), int(num_tokens)))


def prefill_bwd(cfg: MlaConfig, weights: Dict[str, object], x, cu_seqlens_dev, cu_seqlens_host: Sequence[int],
                dout, dx, grads: Dict[str, object], positions=None, rope_cos=None, rope_sin=None, workspace=None,
                stream=None):
    """Backward of the prefill layer (``mla_prefill_bwd``): bf16 x, dout
    [N, hidden] and weights as for ``prefill_fwd``; fp32 dx [N, hidden] and
    ``grads``, a dict of fp32 device tensors named and shaped as the weights
    the configuration uses."""
    import numpy as np
    lib = load_library()
    act, i32, f32 = _act(cfg), _i32(), _f32()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    n, s = int(cuh[-1]), len(cuh) - 1
    st = _resolve_stream(stream)
    ws = _workspace(prefill_bwd_workspace_size(cfg, n), x.device, workspace, st)
    mw = make_weights(weights, act)
    mg = MlaWeightGrads()
    for name, _ in MlaWeightGrads._fields_:
        setattr(mg, name, _ptr(grads.get(name), dtype=f32, name="d" + name))
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib.mla_prefill_bwd(ctypes.byref(cfg), ctypes.byref(mw), _ptr(x, dtype=act, name="x"),
                               _ptr(cu_seqlens_dev, dtype=i32, name="cu_seqlens_dev"), cuh.ctypes.data, s,
                               _ptr(positions, dtype=i32, name="positions"),
                               _ptr(rope_cos, dtype=f32, name="rope_cos"), _ptr(rope_sin, dtype=f32, name="rope_sin"),
                               table_len, _ptr(dout, dtype=act, name="dout"), _ptr(dx, dtype=f32, name="dx"),
                               ctypes.byref(mg), _ptr(ws), ws.numel(), st.cuda_stream), "mla_prefill_bwd")
    return ws


def decode_absorbed_fwd(cfg: MlaConfig, w_kv_b, q_nope, q_pe, kv_cache, block_table, seq_lens_dev,
                        seq_lens_host: Sequence[int], out, workspace=None, stream=None):
    import numpy as np
    lib = load_library()
    act, i32 = _act(cfg), _i32()
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    ws_bytes = decode_workspace_size(cfg, lens)
    st = _resolve_stream(stream)
    ws = _workspace(ws_bytes, q_nope.device, workspace, st)
    num_blocks, block_size = kv_cache.shape[0], kv_cache.shape[1]
    _check(lib.mla_decode_absorbed_fwd(ctypes.byref(cfg), _ptr(w_kv_b, dtype=act, name="w_kv_b"),
                                       _ptr(q_nope, dtype=act, name="q_nope"), _ptr(q_pe, dtype=act, name="q_pe"),
                                       _ptr(kv_cache, dtype=act, name="kv_cache"), num_blocks, block_size,
                                       _ptr(block_table, dtype=i32, name="block_table"), block_table.shape[1],
                                       _ptr(seq_lens_dev, dtype=i32, name="seq_lens_dev"), lens.ctypes.data,
                                       len(lens), _ptr(out, dtype=act, name="out"), _ptr(ws), ws.numel(),
                                       st.cuda_stream), "mla_decode_absorbed_fwd")
    return ws


def decode_absorbed_fwd_noalloc(cfg: MlaConfig, w_kv_b, q_nope, q_pe, kv_cache, block_table, seq_lens_dev,
                                seq_lens_host: Sequence[int], out, stream=None):
    """``decode_absorbed_fwd`` with the library's static scratch instead of a
    workspace: allocates nothing (see ``mla_decode_absorbed_fwd_noalloc``)."""
    import numpy as np
    lib = load_library()
    act, i32 = _act(cfg), _i32()
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    num_blocks, block_size = kv_cache.shape[0], kv_cache.shape[1]
    _check(lib.mla_decode_absorbed_fwd_noalloc(ctypes.byref(cfg), _ptr(w_kv_b, dtype=act, name="w_kv_b"),
                                               _ptr(q_nope, dtype=act, name="q_nope"),
                                               _ptr(q_pe, dtype=act, name="q_pe"),
                                               _ptr(kv_cache, dtype=act, name="kv_cache"), num_blocks, block_size,
                                               _ptr(block_table, dtype=i32, name="block_table"), block_table.shape[1],
                                               _ptr(seq_lens_dev, dtype=i32, name="seq_lens_dev"), lens.ctypes.data,
                                               len(lens), _ptr(out, dtype=act, name="out"), _stream(stream)),
           "mla_decode_absorbed_fwd_noalloc")


def decode_fp8_workspace_size(cfg: MlaConfig, seq_lens_host) -> int:
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    return int(load_library().mla_decode_fp8_workspace_size(ctypes.byref(cfg), lens.ctypes.data, len(lens)))


def cache_quantize_fp8(src, scale: float, dst, stream=None):
    """E4M3 codes of the bf16 rows of ``src`` ([..., width], row-strided
    along the first dimensions as one contiguous block of rows) into ``dst``
    (uint8, same shape); see ``mla_cache_quantize_fp8``."""
    import torch
    if src.shape != dst.shape:
        raise ValueError("src and dst must have the same shape")
    width = src.shape[-1]
    rows = src.numel() // width if width else 0
    _check(load_library().mla_cache_quantize_fp8(_ptr(src, dtype=torch.bfloat16, name="src"), width, rows, width,
                                                 float(scale), _ptr(dst, dtype=torch.uint8, name="dst"), width,
                                                 _stream(stream)), "mla_cache_quantize_fp8")


def attention_bwd_workspace_size(cfg: MlaConfig, num_tokens: int) -> int:
    """Bytes of workspace ``mla_attention_prefill_bwd`` needs for N tokens."""
    return int(load_library().mla_attention_bwd_workspace_size(ctypes.byref(cfg), int(num_tokens)))


def attention_prefill_bwd(cfg: MlaConfig, q, kv, kpe, cu_seqlens_dev, cu_seqlens_host: Sequence[int], out, dout,
                          dq, dkv, dkpe, workspace=None, stream=None, lse=None):
    """Backward of the attention core (``mla_attention_prefill_bwd``): bf16
    q [N, H, 192], kv [N, H, 256], kpe [N, 64] (row-strided), out and dout
    [N, H, 128]; fp32 dq [N, H, 192], dkv [N, H, 256], dkpe [N, 64]; ``lse``:
    optional fp32 [H, N] from ``attention_prefill`` (statistics not
    recomputed)."""
    import numpy as np
    import torch
    lib = load_library()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    n = int(cuh[-1])
    st = _resolve_stream(stream)
    ws = _workspace(int(lib.mla_attention_bwd_workspace_size(ctypes.byref(cfg), n)), q.device, workspace, st)
    bf, f32 = torch.bfloat16, torch.float32
    _check(lib.mla_attention_prefill_bwd(
        ctypes.byref(cfg), _ptr(q, dtype=bf, name="q"), _ptr(kv, dtype=bf, name="kv"),
        _ptr(kpe, rows=True, dtype=bf, name="kpe"), kpe.stride(0), _ptr(cu_seqlens_dev, dtype=_i32(), name="cu"),
        cuh.ctypes.data, len(cuh) - 1, _ptr(out, dtype=bf, name="out"),
        None if lse is None else _ptr(lse, dtype=f32, name="lse"), _ptr(dout, dtype=bf, name="dout"),
        _ptr(dq, dtype=f32, name="dq"), _ptr(dkv, dtype=f32, name="dkv"), _ptr(dkpe, dtype=f32, name="dkpe"),
        _ptr(ws), ws.numel(), st.cuda_stream), "mla_attention_prefill_bwd")
    return ws


def q_uproj_rope_mxfp8(cfg: MlaConfig, q_latent, w_q_b, positions, rope_cos, rope_sin, q_codes, q_scales,
                       stream=None):
    """Fused query up-projection + RoPE + MXFP8 (``mla_q_uproj_rope_mxfp8``):
    q_latent [N, q_lora_rank] bf16, w_q_b bf16, positions int32 [N] (None
    without RoPE), q_codes uint8 [N, H d_qk], q_scales uint8 [N, H d_qk / 32]."""
    import torch
    act, i32 = _act(cfg), _i32()
    n = q_latent.shape[0]
    table_len = rope_cos.shape[0] if rope_cos is not None else 0
    _check(load_library().mla_q_uproj_rope_mxfp8(
        ctypes.byref(cfg), _ptr(q_latent, rows=True, dtype=act, name="q_latent"), q_latent.stride(0), n,
        _ptr(w_q_b, dtype=act, name="w_q_b"), _ptr(positions, dtype=i32, name="positions"),
        _ptr(rope_cos, dtype=torch.float32, name="rope_cos"), _ptr(rope_sin, dtype=torch.float32, name="rope_sin"),
        table_len, _ptr(q_codes, dtype=torch.uint8, name="q_codes"), _ptr(q_scales, dtype=torch.uint8, name="q_scales"),
        _stream(stream)), "mla_q_uproj_rope_mxfp8")


def decode_absorbed_fp8_fwd(cfg: MlaConfig, w_kv_b, q_nope, q_pe, kv_cache_fp8, cache_scale: float, block_table,
                            seq_lens_dev, seq_lens_host: Sequence[int], out, workspace=None, stream=None):
    """``decode_absorbed_fwd`` over an E4M3 cache (uint8 codes
    [num_blocks, block_size, r_kv + d_rope], value = code * cache_scale)."""
    import numpy as np
    import torch
    lib = load_library()
    act, i32 = _act(cfg), _i32()
    lens = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    ws_bytes = decode_fp8_workspace_size(cfg, lens)
    st = _resolve_stream(stream)
    ws = _workspace(ws_bytes, q_nope.device, workspace, st)
    num_blocks, block_size = kv_cache_fp8.shape[0], kv_cache_fp8.shape[1]
    _check(lib.mla_decode_absorbed_fp8_fwd(ctypes.byref(cfg), _ptr(w_kv_b, dtype=act, name="w_kv_b"),
                                           _ptr(q_nope, dtype=act, name="q_nope"),
                                           _ptr(q_pe, dtype=act, name="q_pe"),
                                           _ptr(kv_cache_fp8, dtype=torch.uint8, name="kv_cache_fp8"),
                                           float(cache_scale), num_blocks, block_size,
                                           _ptr(block_table, dtype=i32, name="block_table"), block_table.shape[1],
                                           _ptr(seq_lens_dev, dtype=i32, name="seq_lens_dev"), lens.ctypes.data,
                                           len(lens), _ptr(out, dtype=act, name="out"), _ptr(ws), ws.numel(),
                                           st.cuda_stream), "mla_decode_absorbed_fp8_fwd")
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
    act, i32, f32 = _act(cfg), _i32(), _f32()
    cuh = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
    pre = np.ascontiguousarray(np.asarray(prefix_lens_host, dtype=np.int32))
    s = len(cuh) - 1
    st = _resolve_stream(stream)
    ws = _workspace(prefill_chunk_workspace_size(cfg, cuh, pre), x.device, workspace, st)
    mw = make_weights(weights, act)
    table_len = 0 if rope_cos is None else rope_cos.shape[0]
    nb, bs = (0, 0) if kv_cache is None else (kv_cache.shape[0], kv_cache.shape[1])
    mb = 0 if block_table is None else block_table.shape[1]
    _check(lib.mla_prefill_chunk_fwd(ctypes.byref(cfg), ctypes.byref(mw), _ptr(x, dtype=act, name="x"),
                                     _ptr(cu_seqlens_dev, dtype=i32, name="cu_seqlens_dev"), cuh.ctypes.data, s,
                                     _ptr(prefix_lens_dev, dtype=i32, name="prefix_lens_dev"), pre.ctypes.data,
                                     _ptr(kv_cache, dtype=act, name="kv_cache"), nb, bs,
                                     _ptr(block_table, dtype=i32, name="block_table"), mb,
                                     _ptr(rope_cos, dtype=f32, name="rope_cos"),
                                     _ptr(rope_sin, dtype=f32, name="rope_sin"), table_len,
                                     _ptr(out, dtype=act, name="out"), _ptr(latent_out, dtype=act, name="latent_out"),
                                     _ptr(ws), ws.numel(), st.cuda_stream),
           "mla_prefill_chunk_fwd")
    return ws
