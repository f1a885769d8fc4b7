"""ctypes binding of libolk.so (the C ABI declared in include/olk.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libolk.  PyTorch provides device memory and the current stream.
Importing this module raises if libolk.so has not been built: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from .workloads import Problem, present_shape, y_shape

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libolk.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m transformer_attention_fwd_amd.build_lib` "
        "(or __graft_entry__.build()); the attention path has no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)

OLK_OK, OLK_E_NULL, OLK_E_ATTR, OLK_E_SHAPE, OLK_E_UNSUPPORTED, OLK_E_WORKSPACE, OLK_E_HIP = range(7)
OLK_F32, OLK_F16, OLK_BF16 = 0, 1, 2
OLK_OP_GQA, OLK_OP_MHA, OLK_OP_ATTENTION = 0, 1, 2
OLK_KERNEL_AUTO, OLK_KERNEL_GENERIC, OLK_KERNEL_TILED = 0, 1, 2

_OPS = {"gqa": OLK_OP_GQA, "mha": OLK_OP_MHA, "attention": OLK_OP_ATTENTION}
_DTYPES = {"f32": OLK_F32, "f16": OLK_F16, "bf16": OLK_BF16}
KERNELS = {"auto": OLK_KERNEL_AUTO, "generic": OLK_KERNEL_GENERIC, "tiled": OLK_KERNEL_TILED}


class olk_attn_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "op", "dtype", "batch", "q_seq", "kv_seq", "past_seq", "q_num_heads",
        "kv_num_heads", "head_size", "v_head_size", "q_rank", "kv_rank", "causal",
        "local_window_size", "has_scale")] + [
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
        ("mask_filter_value", ctypes.c_float),
        ("bias_b", ctypes.c_int32), ("bias_h", ctypes.c_int32),
        ("kv_inplace", ctypes.c_int32), ("kernel", ctypes.c_int32)] + [
        (n, ctypes.c_int32) for n in ("do_rotary", "rotary_interleaved", "rotary_dim",
                                      "rotary_max_pos", "bias_s", "bias_t", "mask_kind",
                                      "mask_b", "mask_h", "mask_s", "mask_t", "seqlens_i64",
                                      "qk_mode")]


class olk_attn_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "v", "past_k", "past_v", "seqlens", "attn_bias", "head_sink",
        "proj_bias", "y", "present_k", "present_v", "cos_cache", "sin_cache", "attn_mask",
        "qk_out")]


class olk_attn_bwd_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "v", "seqlens", "dy", "dq", "dk", "dv")]


_P = ctypes.POINTER
_lib.olk_validate.argtypes = [_P(olk_attn_desc), _P(olk_attn_io)]
_lib.olk_validate.restype = ctypes.c_int
_lib.olk_workspace_bytes.argtypes = [_P(olk_attn_desc)]
_lib.olk_workspace_bytes.restype = ctypes.c_size_t
_lib.olk_attention_fwd.argtypes = [_P(olk_attn_desc), _P(olk_attn_io), ctypes.c_void_p]
_lib.olk_attention_fwd.restype = ctypes.c_int
_lib.olk_attention_decode.argtypes = [_P(olk_attn_desc), _P(olk_attn_io), ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
_lib.olk_attention_decode.restype = ctypes.c_int
_lib.olk_attention_decode_noalloc.argtypes = [_P(olk_attn_desc), _P(olk_attn_io),
                                              ctypes.c_void_p]
_lib.olk_attention_decode_noalloc.restype = ctypes.c_int
_lib.olk_bwd_workspace_bytes.argtypes = [_P(olk_attn_desc)]
_lib.olk_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.olk_attention_bwd.argtypes = [_P(olk_attn_desc), _P(olk_attn_bwd_io), ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
_lib.olk_attention_bwd.restype = ctypes.c_int
_lib.olk_status_str.argtypes = [ctypes.c_int]
_lib.olk_status_str.restype = ctypes.c_char_p
_lib.olk_last_kernel_name.argtypes = []
_lib.olk_last_kernel_name.restype = ctypes.c_char_p

EXPORTED = ("olk_validate", "olk_workspace_bytes", "olk_attention_fwd", "olk_attention_decode",
            "olk_attention_decode_noalloc", "olk_bwd_workspace_bytes", "olk_attention_bwd",
            "olk_status_str", "olk_last_kernel_name")


class OlkError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"olk status {status}: {olk_status_str(status)}")


# ---- the C entry points, same names ---------------------------------------

def _ref(x):
    return None if x is None else ctypes.byref(x)


def olk_validate(desc: olk_attn_desc, io: olk_attn_io) -> int:
    return _lib.olk_validate(_ref(desc), _ref(io))


def olk_workspace_bytes(desc: olk_attn_desc) -> int:
    return _lib.olk_workspace_bytes(ctypes.byref(desc))


def olk_attention_fwd(desc: olk_attn_desc, io: olk_attn_io, stream: int) -> int:
    return _lib.olk_attention_fwd(ctypes.byref(desc), ctypes.byref(io), stream)


def olk_attention_decode(desc: olk_attn_desc, io: olk_attn_io, workspace: int,
                         workspace_bytes: int, stream: int) -> int:
    return _lib.olk_attention_decode(ctypes.byref(desc), ctypes.byref(io), workspace,
                                     workspace_bytes, stream)


def olk_attention_decode_noalloc(desc: olk_attn_desc, io: olk_attn_io, stream: int) -> int:
    return _lib.olk_attention_decode_noalloc(ctypes.byref(desc), ctypes.byref(io), stream)


NOALLOC_SCRATCH_BYTES = 32 << 20


def olk_bwd_workspace_bytes(desc: olk_attn_desc) -> int:
    return _lib.olk_bwd_workspace_bytes(ctypes.byref(desc))


def olk_attention_bwd(desc: olk_attn_desc, io: olk_attn_bwd_io, workspace: int,
                      workspace_bytes: int, stream: int) -> int:
    return _lib.olk_attention_bwd(ctypes.byref(desc), ctypes.byref(io), workspace,
                                  workspace_bytes, stream)


def olk_status_str(status: int) -> str:
    return _lib.olk_status_str(status).decode()


def olk_last_kernel_name() -> str:
    return _lib.olk_last_kernel_name().decode()


# ---- marshalling helpers ---------------------------------------------------

def make_desc(p: Problem, kernel: str = "auto", kv_inplace: bool = False) -> olk_attn_desc:
    bb, bh = p.bias_bh if p.bias_bh is not None else (1, 1)
    return olk_attn_desc(
        op=_OPS[p.op], dtype=_DTYPES[p.dtype], batch=p.B, q_seq=p.S, kv_seq=p.L,
        past_seq=p.P, q_num_heads=p.Hq, kv_num_heads=p.Hkv, head_size=p.D,
        v_head_size=p.Dv, q_rank=p.q_rank, kv_rank=p.kv_rank, causal=p.causal,
        local_window_size=p.window, has_scale=0 if p.scale is None else 1,
        scale=0.0 if p.scale is None else p.scale, softcap=p.softcap,
        mask_filter_value=p.mask_filter_value, bias_b=bb, bias_h=bh,
        kv_inplace=1 if kv_inplace else 0, kernel=KERNELS[kernel],
        do_rotary=p.rotary, rotary_interleaved=p.rotary_interleaved,
        rotary_dim=p.rotary_dim, rotary_max_pos=p.max_pos if p.rotary else 0,
        bias_s=1 if p.bias_s_bcast else 0, bias_t=p.bias_cols,
        mask_kind={"": 0, "bool": 1, "int32": 2}[p.mask_kind],
        mask_b=p.mask_bhs[0] if p.mask_bhs else 0, mask_h=p.mask_bhs[1] if p.mask_bhs else 0,
        mask_s=(1 if p.mask_bhs[2] == 1 else 0) if p.mask_bhs else 0, mask_t=p.mask_cols,
        seqlens_i64=1 if p.lens_i64 else 0, qk_mode=p.qk_mode if p.qk_mode is not None else 0)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def make_io(tensors: Dict[str, torch.Tensor], y: torch.Tensor,
            present_k: Optional[torch.Tensor] = None,
            present_v: Optional[torch.Tensor] = None,
            qk_out: Optional[torch.Tensor] = None) -> olk_attn_io:
    g = tensors.get
    return olk_attn_io(q=_ptr(g("q")), k=_ptr(g("k")), v=_ptr(g("v")),
                       past_k=_ptr(g("past_k")), past_v=_ptr(g("past_v")),
                       seqlens=_ptr(g("lens")), attn_bias=_ptr(g("bias")),
                       head_sink=_ptr(g("sink")), proj_bias=_ptr(g("proj_bias")),
                       y=_ptr(y), present_k=_ptr(present_k), present_v=_ptr(present_v),
                       cos_cache=_ptr(g("cos_cache")), sin_cache=_ptr(g("sin_cache")),
                       attn_mask=_ptr(g("mask")), qk_out=_ptr(qk_out))


def current_stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Call:
    """One prepared call: descriptor, device outputs and (for decode) workspace.

    Allocation happens here, once; ``launch()`` only calls the C entry point,
    so timing loops measure the kernels alone.
    """

    def __init__(self, p: Problem, dev: Dict[str, torch.Tensor], *, mode: str = "fwd",
                 kernel: str = "auto", want_present: bool = True, kv_inplace: bool = False,
                 present_k: Optional[torch.Tensor] = None,
                 present_v: Optional[torch.Tensor] = None,
                 y: Optional[torch.Tensor] = None):
        self.p = p
        self.mode = mode
        self.dev = dict(dev)
        device = dev["q"].device
        self.y = y if y is not None else torch.empty(y_shape(p), dtype=p.torch_dtype,
                                                     device=device)
        if want_present or kv_inplace:
            self.present_k = present_k if present_k is not None else torch.empty(
                present_shape(p, False), dtype=p.torch_dtype, device=device)
            self.present_v = present_v if present_v is not None else torch.empty(
                present_shape(p, True), dtype=p.torch_dtype, device=device)
        else:
            self.present_k = self.present_v = None
        if kv_inplace:
            self.dev.pop("past_k", None)
            self.dev.pop("past_v", None)
        self.qk = (torch.empty((p.B, p.Hq, p.S, p.T), dtype=torch.float32, device=device)
                   if p.qk_mode is not None else None)
        self.desc = make_desc(p, kernel=kernel, kv_inplace=kv_inplace)
        self.io = make_io(self.dev, self.y, self.present_k, self.present_v, self.qk)
        self.ws_bytes = olk_workspace_bytes(self.desc) if mode == "decode" else 0
        self.ws = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
                   if self.ws_bytes else None)
        st = olk_validate(self.desc, self.io)
        if st != OLK_OK:
            raise OlkError(st)

    def launch(self, stream: Optional[int] = None) -> None:
        s = current_stream() if stream is None else stream
        if self.mode == "decode":
            st = olk_attention_decode(self.desc, self.io, _ptr(self.ws), self.ws_bytes, s)
        else:
            st = olk_attention_fwd(self.desc, self.io, s)
        if st != OLK_OK:
            raise OlkError(st)


def attention(p: Problem, dev: Dict[str, torch.Tensor], **kw):
    """Runs one call and returns (y, present_k, present_v) device tensors."""
    c = Call(p, dev, **kw)
    c.launch()
    return c.y, c.present_k, c.present_v


class BwdCall:
    """One prepared backward call: descriptor, gradient outputs and workspace."""

    def __init__(self, p: Problem, dev: Dict[str, torch.Tensor], dy: torch.Tensor):
        device = dev["q"].device
        self.p = p
        self.dy = dy
        self.dq = torch.empty_like(dev["q"])
        self.dk = torch.empty_like(dev["k"])
        self.dv = torch.empty_like(dev["v"])
        self.desc = make_desc(p)
        self.io = olk_attn_bwd_io(q=_ptr(dev["q"]), k=_ptr(dev["k"]), v=_ptr(dev["v"]),
                                  seqlens=_ptr(dev.get("lens")), dy=_ptr(dy), dq=_ptr(self.dq),
                                  dk=_ptr(self.dk), dv=_ptr(self.dv))
        self.ws_bytes = olk_bwd_workspace_bytes(self.desc)
        self.ws = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
                   if self.ws_bytes else None)

    def launch(self, stream: Optional[int] = None) -> None:
        s = current_stream() if stream is None else stream
        st = olk_attention_bwd(self.desc, self.io, _ptr(self.ws), self.ws_bytes, s)
        if st != OLK_OK:
            raise OlkError(st)
