"""Seeded synthetic inputs for the attention forward.

This module holds no attention arithmetic: it only describes problems (shapes,
attributes) and draws their input tensors from a seeded generator.  Both the
oracle (``oracle/``) and the HIP path take their inputs from here, so the two
see bit-identical data.

Tensor layouts (all row-major, element type = ``dtype`` unless stated):

* ``q``        rank 3: (B, S, Hq*D)          rank 4: (B, Hq, S, D)
* ``k``/``v``  rank 3: (B, L, Hkv*D|Dv)      rank 4: (B, Hkv, L, D|Dv)
* ``past_k``/``past_v``: (B, Hkv, P, D|Dv)
* ``lens``  int32 (B,): GroupQueryAttention ``seqlens_k`` (total length - 1),
  MultiHeadAttention key-padding lengths, ai.onnx Attention non-padding lengths
* ``bias``  (bias_b, bias_h, S, P+L) additive attention bias
* ``sink``  (Hq,) per-head virtual logit (GroupQueryAttention ``head_sink``)
* ``proj_bias`` (2*Hq*D + Hq*Dv,) MultiHeadAttention projection bias [q | k | v]
* ``cos_cache``/``sin_cache`` (max_pos, R/2) rotary tables (GroupQueryAttention
  with ``rotary``); deterministic, not drawn
* ``mask`` (mask_b, mask_h, mask_s, cols) bool or int32 attention mask, drawn
  after ``proj_bias`` as uniform [0, 1) < mask_p

Draw order inside one problem is fixed: q, k, v, past_k, past_v, lens, bias,
sink, proj_bias (absent tensors are skipped).  Normals are drawn as float32 from
``numpy.random.Generator(PCG64(seed))``, multiplied by sigma in float32 and
rounded to the element type with round-to-nearest-even (torch ``.to``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
OPS = ("gqa", "mha", "attention")


@dataclass(frozen=True)
class Problem:
    """Shapes and attributes of one attention call."""

    op: str = "gqa"              # "gqa" | "mha" | "attention"
    dtype: str = "bf16"          # "f32" | "f16" | "bf16"
    B: int = 1                   # batch
    S: int = 1                   # query length
    L: int = 1                   # new key/value length (GroupQueryAttention: L == S)
    P: int = 0                   # past buffer length (0: no past inputs)
    Hq: int = 1
    Hkv: int = 1
    D: int = 64
    Dv: int = 64
    q_rank: int = 3
    kv_rank: int = 3
    causal: int = 1
    window: int = -1             # local_window_size
    scale: Optional[float] = None  # None: 1/sqrt(D)
    softcap: float = 0.0
    mask_filter_value: float = -10000.0
    bias_bh: Optional[Tuple[int, int]] = None  # (bias_b, bias_h) or None
    has_sink: bool = False
    has_lens: bool = True        # GroupQueryAttention always has seqlens_k
    has_proj_bias: bool = False
    # how the seeded draw fills lens (ignored for GroupQueryAttention prefill
    # without past, where seqlens_k = S - 1 is implied)
    lens_range: Optional[Tuple[int, int]] = None
    sigma_qkv: float = 1.0
    sigma_bias: float = 0.1
    sigma_sink: float = 1.0
    sigma_proj: float = 0.02
    # rotary embedding (GroupQueryAttention do_rotary): cos/sin caches of
    # rotary_max_pos rows (0: P + L) and R/2 columns, R = rotary_dim (0: D)
    rotary: int = 0
    rotary_interleaved: int = 0
    rotary_dim: int = 0
    rotary_max_pos: int = 0
    rotary_base: float = 10000.0
    # attn_bias extents beyond (bias_b, bias_h): one row for every query
    # (bias_s_bcast) and a short last dimension (bias_cols < P+L, ai.onnx Attention)
    bias_s_bcast: bool = False
    bias_cols: int = 0
    # attn_mask: "" none, "bool" (ai.onnx Attention, uint8, true = attend) or
    # "int32" (MultiHeadAttention binary key-padding mask, nonzero = attend);
    # extents (mask_b, mask_h, mask_s) with mask_s 1 or S, mask_cols 0 = P+L
    mask_kind: str = ""
    mask_bhs: Optional[Tuple[int, int, int]] = None
    mask_cols: int = 0
    mask_p: float = 0.8          # probability that a mask element attends
    lens_i64: bool = False       # ai.onnx Attention nonpad_kv_seqlen as int64
    qk_mode: Optional[int] = None  # ai.onnx Attention qk_matmul_output_mode

    @property
    def T(self) -> int:
        """Present length / key columns of the bias: P + L."""
        return self.P + self.L

    @property
    def R(self) -> int:
        return self.rotary_dim if self.rotary_dim > 0 else self.D

    @property
    def max_pos(self) -> int:
        return self.rotary_max_pos if self.rotary_max_pos > 0 else self.P + self.L

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)


# The workloads.  Sizes and distributions follow the workload list of the
# attention-forward study; each is named by what it is.
WORKLOADS: Dict[str, Problem] = {
    # fp32 GQA prefill, tiny: B=1 S=16, 4 q heads / 2 kv heads, D=32, causal
    "gqa_prefill_tiny_f32": Problem(
        op="gqa", dtype="f32", B=1, S=16, L=16, P=0, Hq=4, Hkv=2, D=32, Dv=32,
        causal=1, window=-1, scale=float(np.float32(1.0 / math.sqrt(32)))),
    # bf16 GQA causal prefill: B=4 S=2048, 32/8 heads, D=128
    "gqa_prefill_causal_bf16": Problem(
        op="gqa", dtype="bf16", B=4, S=2048, L=2048, P=0, Hq=32, Hkv=8, D=128,
        Dv=128, causal=1, window=-1),
    # bf16 GQA sliding-window prefill with sinks and softcap: B=2 S=4096, W=512
    "gqa_prefill_window_sink_bf16": Problem(
        op="gqa", dtype="bf16", B=2, S=4096, L=4096, P=0, Hq=32, Hkv=8, D=128,
        Dv=128, causal=1, window=512, softcap=50.0, has_sink=True),
    # fp16 GQA decode against an 8192-slot KV cache, valid past in [512, 8192]
    "gqa_decode_f16": Problem(
        op="gqa", dtype="f16", B=64, S=1, L=1, P=8192, Hq=32, Hkv=8, D=128,
        Dv=128, causal=1, window=-1, lens_range=(512, 8192)),
    # fp16 MHA (Whisper-style) cross-attention with key padding and bias
    "mha_cross_f16": Problem(
        op="mha", dtype="f16", B=8, S=448, L=1500, P=0, Hq=20, Hkv=20, D=64,
        Dv=64, kv_rank=4, causal=0, window=-1, bias_bh=(1, 20),
        has_lens=True, lens_range=(1000, 1500), has_proj_bias=True),
    # the bf16 causal prefill with rotary embedding fused in (do_rotary, split
    # halves over the full head): Q/K rotated at positions 0..S-1
    "gqa_prefill_rope_bf16": Problem(
        op="gqa", dtype="bf16", B=4, S=2048, L=2048, P=0, Hq=32, Hkv=8, D=128,
        Dv=128, causal=1, window=-1, rotary=1),
    # ai.onnx Attention over (B, 1, 1, T) BOOL key masks, 80% of keys attended
    "attention_boolmask_bf16": Problem(
        op="attention", dtype="bf16", B=4, S=2048, L=2048, P=0, Hq=32, Hkv=8, D=128,
        Dv=128, causal=0, window=-1, has_lens=False, mask_kind="bool",
        mask_bhs=(4, 1, 1)),
}

WORKLOAD_ORDER = [
    "gqa_prefill_tiny_f32",
    "gqa_prefill_causal_bf16",
    "gqa_prefill_window_sink_bf16",
    "gqa_decode_f16",
    "mha_cross_f16",
    "gqa_prefill_rope_bf16",
    "attention_boolmask_bf16",
]


def workload_seed(name: str) -> int:
    """Seed of a named workload: 1000 + its 1-based position in the list."""
    return 1000 + WORKLOAD_ORDER.index(name) + 1


def _normal(rng: np.random.Generator, shape, sigma: float, dtype: torch.dtype,
            chunk_rows: int = 1) -> torch.Tensor:
    """Draw N(0, sigma^2) float32 values chunk by chunk along dim 0 and round
    them to ``dtype``.  Chunking bounds the float32 temporaries for the big
    KV-cache tensors; the stream of draws does not depend on the chunking."""
    out = torch.empty(shape, dtype=dtype)
    if out.numel() == 0:
        return out
    flat = out.view(shape[0], -1)
    per = flat.shape[1]
    rows = max(1, chunk_rows)
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        x = rng.standard_normal(size=(r1 - r0) * per, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        flat[r0:r1] = torch.from_numpy(x).view(r1 - r0, per).to(dtype)
    return out


def q_shape(p: Problem):
    return (p.B, p.S, p.Hq * p.D) if p.q_rank == 3 else (p.B, p.Hq, p.S, p.D)


def kv_shape(p: Problem, dv: bool):
    d = p.Dv if dv else p.D
    return (p.B, p.L, p.Hkv * d) if p.kv_rank == 3 else (p.B, p.Hkv, p.L, d)


def y_shape(p: Problem):
    return (p.B, p.S, p.Hq * p.Dv) if p.q_rank == 3 else (p.B, p.Hq, p.S, p.Dv)


def present_shape(p: Problem, dv: bool):
    return (p.B, p.Hkv, p.P + p.L, p.Dv if dv else p.D)


def make_inputs(p: Problem, seed: int, lens: Optional[np.ndarray] = None
                ) -> Dict[str, torch.Tensor]:
    """Draw every input tensor of problem ``p`` (host tensors).

    ``lens`` overrides the drawn lengths (still int32 (B,)).  For
    GroupQueryAttention the lengths are ``seqlens_k`` = total length - 1; when
    ``lens_range`` is set they are drawn as the valid past length P_b (so
    seqlens_k[b] = P_b + S - 1); otherwise a prefill without past uses S - 1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = p.torch_dtype
    big = 1 if (p.B * p.S * p.Hq * p.D) > (1 << 22) else p.B
    out: Dict[str, torch.Tensor] = {}
    out["q"] = _normal(rng, q_shape(p), p.sigma_qkv, dt, chunk_rows=big)
    out["k"] = _normal(rng, kv_shape(p, False), p.sigma_qkv, dt, chunk_rows=big)
    out["v"] = _normal(rng, kv_shape(p, True), p.sigma_qkv, dt, chunk_rows=big)
    if p.P > 0:
        out["past_k"] = _normal(rng, (p.B, p.Hkv, p.P, p.D), p.sigma_qkv, dt, 1)
        out["past_v"] = _normal(rng, (p.B, p.Hkv, p.P, p.Dv), p.sigma_qkv, dt, 1)
    if p.op == "gqa" or p.has_lens:
        if lens is not None:
            l32 = np.asarray(lens, dtype=np.int32)
        elif p.lens_range is not None:
            lo, hi = p.lens_range
            l32 = rng.integers(lo, hi, size=p.B, endpoint=True, dtype=np.int32)
            if p.op == "gqa":
                l32 = (l32 + np.int32(p.S - 1)).astype(np.int32)
        else:
            if p.op == "gqa":
                l32 = np.full(p.B, p.P + p.S - 1, dtype=np.int32)
            else:
                l32 = np.full(p.B, p.T, dtype=np.int32)
        out["lens"] = torch.from_numpy(np.ascontiguousarray(l32))
    if p.bias_bh is not None:
        bb, bh = p.bias_bh
        rows = 1 if p.bias_s_bcast else p.S
        cols = p.bias_cols if p.bias_cols > 0 else p.T
        out["bias"] = _normal(rng, (bb, bh, rows, cols), p.sigma_bias, dt, 1)
    if p.has_sink:
        out["sink"] = _normal(rng, (p.Hq,), p.sigma_sink, dt, 1)
    if p.has_proj_bias:
        out["proj_bias"] = _normal(rng, (2 * p.Hq * p.D + p.Hq * p.Dv,),
                                   p.sigma_proj, dt, 1)
    if p.mask_kind:
        mb, mh, ms = p.mask_bhs
        cols = p.mask_cols if p.mask_cols > 0 else p.T
        bits = rng.random(size=(mb, mh, ms, cols)) < p.mask_p
        out["mask"] = torch.from_numpy(bits.astype(np.uint8 if p.mask_kind == "bool"
                                                    else np.int32))
        if p.mask_kind == "bool":
            out["mask"] = out["mask"].to(torch.bool)
    if p.rotary:
        out["cos_cache"], out["sin_cache"] = rotary_tables(p)
    if p.lens_i64 and "lens" in out:
        out["lens"] = out["lens"].to(torch.int64)
    return out


def rotary_tables(p: Problem) -> Tuple[torch.Tensor, torch.Tensor]:
    """cos/sin caches (max_pos, R/2) with the usual frequency schedule
    base^(-2k/R), computed in float64 and rounded to the element type.  They
    are inputs of the operator (no random draws)."""
    half = p.R // 2
    pos = np.arange(p.max_pos, dtype=np.float64)[:, None]
    inv = p.rotary_base ** (-2.0 * np.arange(half, dtype=np.float64) / p.R)
    ang = pos * inv[None, :]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a.astype(np.float32))).to(p.torch_dtype)
    return to(np.cos(ang)), to(np.sin(ang))


def workload(name: str) -> Tuple[Problem, Dict[str, torch.Tensor]]:
    p = WORKLOADS[name]
    return p, make_inputs(p, workload_seed(name))


def valid_lengths(p: Problem, inputs: Dict[str, torch.Tensor]) -> np.ndarray:
    """Per-batch count of key positions that hold real data: for
    GroupQueryAttention seqlens_k + 1, otherwise the key-padding / non-padding
    length clamped to [0, P+L] (P+L when absent).  Bookkeeping only."""
    if p.op == "gqa":
        return inputs["lens"].numpy().astype(np.int64) + 1
    if "lens" in inputs:
        return np.clip(inputs["lens"].numpy().astype(np.int64), 0, p.T)
    return np.full(p.B, p.T, dtype=np.int64)
