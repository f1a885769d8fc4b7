"""Python front end of the oracle (``olk_ref.c``).  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg import this
module.  It marshals host tensors (torch CPU tensors from the seeded input
generators) into the oracle's own plain structs and returns float64 results.
It imports nothing from the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "olk_ref.c")
_LIB = os.path.join(_HERE, "libolk_ref.so")

_OPS = {"gqa": 0, "mha": 1, "attention": 2}
_DT = {"f32": 0, "f16": 1, "bf16": 2}


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "op", "dtype", "batch", "q_seq", "kv_seq", "past_seq", "q_heads",
        "kv_heads", "head_size", "v_head_size", "q_rank", "kv_rank", "causal",
        "window", "has_scale")] + [
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
        ("mask_filter_value", ctypes.c_float),
        ("bias_b", ctypes.c_int32), ("bias_h", ctypes.c_int32)] + [
        (n, ctypes.c_int32) for n in ("do_rotary", "rotary_interleaved", "rotary_dim",
                                      "rotary_max_pos", "bias_s", "bias_t", "mask_kind",
                                      "mask_b", "mask_h", "mask_s", "mask_t", "seqlens_i64")]


class _Inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q", "k", "v", "past_k", "past_v", "lens", "bias", "sink", "proj_bias",
        "cos_cache", "sin_cache", "mask")]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (float64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        # -ffp-contract=off: the rotary arithmetic (R18) is float32 with exactly
        # the roundings written in the source
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                        _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.POINTER
        _lib.olk_ref_attention.argtypes = [P(_Desc), P(_Inputs), ctypes.c_void_p, ctypes.c_int]
        _lib.olk_ref_attention_rows.argtypes = [P(_Desc), P(_Inputs), ctypes.c_void_p,
                                                ctypes.c_long, ctypes.c_void_p, ctypes.c_int]
        _lib.olk_ref_row_weights.argtypes = [P(_Desc), P(_Inputs), ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib.olk_ref_row_weights.restype = ctypes.c_long
        _lib.olk_ref_present.argtypes = [P(_Desc), P(_Inputs), ctypes.c_void_p, ctypes.c_void_p]
        _lib.olk_ref_qk.argtypes = [P(_Desc), P(_Inputs), ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_int]
        _lib.olk_ref_attention_bwd.argtypes = [P(_Desc), P(_Inputs), ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return _lib


def _desc(p) -> _Desc:
    bb, bh = p.bias_bh if p.bias_bh is not None else (1, 1)
    return _Desc(op=_OPS[p.op], dtype=_DT[p.dtype], batch=p.B, q_seq=p.S, kv_seq=p.L,
                 past_seq=p.P, q_heads=p.Hq, kv_heads=p.Hkv, head_size=p.D,
                 v_head_size=p.Dv, q_rank=p.q_rank, kv_rank=p.kv_rank,
                 causal=p.causal, window=p.window,
                 has_scale=0 if p.scale is None else 1,
                 scale=0.0 if p.scale is None else p.scale, softcap=p.softcap,
                 mask_filter_value=p.mask_filter_value, bias_b=bb, bias_h=bh,
                 do_rotary=p.rotary, rotary_interleaved=p.rotary_interleaved,
                 rotary_dim=p.rotary_dim, rotary_max_pos=p.max_pos,
                 bias_s=1 if p.bias_s_bcast else 0, bias_t=p.bias_cols,
                 mask_kind={"": 0, "bool": 1, "int32": 2}[p.mask_kind],
                 mask_b=p.mask_bhs[0] if p.mask_bhs else 1,
                 mask_h=p.mask_bhs[1] if p.mask_bhs else 1,
                 mask_s=(1 if p.mask_bhs[2] == 1 else 0) if p.mask_bhs else 0,
                 mask_t=p.mask_cols, seqlens_i64=1 if p.lens_i64 else 0)


class _Bound:
    """Keeps contiguous host copies alive while the oracle reads them."""

    def __init__(self, inputs: Dict[str, torch.Tensor]):
        self.keep = {}
        ptrs = {}
        for name in ("q", "k", "v", "past_k", "past_v", "lens", "bias", "sink", "proj_bias",
                     "cos_cache", "sin_cache", "mask"):
            t = inputs.get(name)
            if t is None:
                ptrs[name] = None
                continue
            t = t.detach().to("cpu").contiguous()
            self.keep[name] = t
            ptrs[name] = t.data_ptr() if t.numel() else None
        self.s = _Inputs(**ptrs)


def attention(p, inputs: Dict[str, torch.Tensor], threads: int = 0) -> np.ndarray:
    """Y of every row, float64, shaped (B, S, Hq, Dv)."""
    b = _Bound(inputs)
    y = np.zeros((p.B, p.S, p.Hq, p.Dv), dtype=np.float64)
    rc = lib().olk_ref_attention(ctypes.byref(_desc(p)), ctypes.byref(b.s),
                                 y.ctypes.data, threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return y


def attention_rows(p, inputs: Dict[str, torch.Tensor], rows: np.ndarray,
                   threads: int = 0) -> np.ndarray:
    """Y of selected rows; ``rows`` is int (n, 3) of (b, h, i).  Returns (n, Dv)."""
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    b = _Bound(inputs)
    out = np.zeros((rows.shape[0], p.Dv), dtype=np.float64)
    rc = lib().olk_ref_attention_rows(ctypes.byref(_desc(p)), ctypes.byref(b.s),
                                      rows.ctypes.data, rows.shape[0], out.ctypes.data,
                                      threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem or a row index")
    return out


def row_weights(p, inputs: Dict[str, torch.Tensor], b: int, h: int, i: int
                ) -> Tuple[np.ndarray, float]:
    """Softmax weights of row (b, h, i) over its concatenated keys, and the
    share taken by the head sink (0 without one)."""
    bd = _Bound(inputs)
    w = np.zeros(p.P + p.L + 1, dtype=np.float64)
    sw = ctypes.c_double(0.0)
    n = lib().olk_ref_row_weights(ctypes.byref(_desc(p)), ctypes.byref(bd.s), b, h, i,
                                  w.ctypes.data, ctypes.byref(sw))
    if n < 0:
        raise ValueError("oracle rejected the problem")
    return w[:n].copy(), sw.value


def present(p, inputs: Dict[str, torch.Tensor], fill: Optional[float] = None
            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Expected present_key / present_value (B, Hkv, P+L, D|Dv).  Positions
    beyond each batch's total length keep ``fill`` (NaN by default)."""
    bd = _Bound(inputs)
    shape_k = (p.B, p.Hkv, p.P + p.L, p.D)
    shape_v = (p.B, p.Hkv, p.P + p.L, p.Dv)
    f = float("nan") if fill is None else fill
    pk = torch.full(shape_k, f, dtype=p.torch_dtype)
    pv = torch.full(shape_v, f, dtype=p.torch_dtype)
    rc = lib().olk_ref_present(ctypes.byref(_desc(p)), ctypes.byref(bd.s),
                               pk.data_ptr() if pk.numel() else None,
                               pv.data_ptr() if pv.numel() else None)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return pk, pv


def qk(p, inputs: Dict[str, torch.Tensor], mode: int, threads: int = 0) -> np.ndarray:
    """qk_matmul_output of ai.onnx Attention in float64, (B, Hq, S, T)."""
    b = _Bound(inputs)
    out = np.zeros((p.B, p.Hq, p.S, p.T), dtype=np.float64)
    rc = lib().olk_ref_qk(ctypes.byref(_desc(p)), ctypes.byref(b.s), mode, out.ctypes.data,
                          threads)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return out


def attention_bwd(p, inputs: Dict[str, torch.Tensor], dy: torch.Tensor):
    """R22 gradients of the GroupQueryAttention forward (no past): float64
    dq (B, S, Hq, D), dk (B, S, Hkv, D), dv (B, S, Hkv, Dv)."""
    b = _Bound(inputs)
    dyc = dy.detach().to("cpu").contiguous()
    dq = np.zeros((p.B, p.S, p.Hq, p.D))
    dk = np.zeros((p.B, p.S, p.Hkv, p.D))
    dv = np.zeros((p.B, p.S, p.Hkv, p.Dv))
    rc = lib().olk_ref_attention_bwd(ctypes.byref(_desc(p)), ctypes.byref(b.s), dyc.data_ptr(),
                                     dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return dq, dk, dv
