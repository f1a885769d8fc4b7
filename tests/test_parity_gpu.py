"""GPU parity: the HIP path through the C ABI against the oracle.

Every problem, the full-size workloads included, is compared element by
element over the whole of Y (pre-filled with NaN, so a tile no workgroup wrote
fails) and present_key/present_value bit for bit.  The full-size workloads run
in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import olk_ref
from tests.parity import assert_close, assert_present_exact, to_dev, y_logical
from transformer_attention_fwd_amd.workloads import (WORKLOAD_ORDER, WORKLOADS, Problem,
                                                     make_inputs, workload, y_shape)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from transformer_attention_fwd_amd import olk


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


# Small problems spanning every feature: several 64-key tiles plus ragged tails.
SMALL = {
    "gqa_causal_bf16": Problem(op="gqa", dtype="bf16", B=2, S=197, L=197, Hq=8, Hkv=2,
                               D=128, Dv=128, causal=1),
    "gqa_causal_f16_d64": Problem(op="gqa", dtype="f16", B=2, S=150, L=150, Hq=4, Hkv=4,
                                  D=64, Dv=64, causal=1),
    "gqa_window_sink_softcap_bf16": Problem(op="gqa", dtype="bf16", B=2, S=300, L=300, Hq=8,
                                            Hkv=2, D=128, Dv=128, causal=1, window=70,
                                            softcap=2.0, has_sink=True),
    # a large softcap (30) at head size 128 with sinks: tanh far from saturation
    "gqa_softcap30_sink_bf16": Problem(op="gqa", dtype="bf16", B=2, S=260, L=260, Hq=8, Hkv=2,
                                       D=128, Dv=128, causal=1, softcap=30.0, has_sink=True),
    "gqa_past_f16": Problem(op="gqa", dtype="f16", B=3, S=37, L=37, P=200, Hq=8, Hkv=2, D=128,
                            Dv=128, causal=1, lens_range=(0, 200)),
    "gqa_decode_f16": Problem(op="gqa", dtype="f16", B=5, S=1, L=1, P=700, Hq=8, Hkv=2,
                              D=128, Dv=128, causal=1, lens_range=(0, 700)),
    "gqa_decode_sink_window_bf16": Problem(op="gqa", dtype="bf16", B=3, S=2, L=2, P=300,
                                           Hq=4, Hkv=1, D=64, Dv=64, causal=1, window=100,
                                           has_sink=True, lens_range=(50, 300)),
    # head-size-128 decode with 8 and 16 row slots per KV head (PV on the
    # matrix cores): window + sink, short and long pasts
    "gqa_decode_rows8_bf16": Problem(op="gqa", dtype="bf16", B=3, S=2, L=2, P=333, Hq=16,
                                     Hkv=4, D=128, Dv=128, causal=1, window=150,
                                     has_sink=True, lens_range=(1, 333)),
    "gqa_decode_rows16_f16": Problem(op="gqa", dtype="f16", B=2, S=1, L=1, P=1500, Hq=32,
                                     Hkv=2, D=128, Dv=128, causal=1, lens_range=(0, 1500)),
    # 8192 keys: split counts that are multiples of 8 (8 decode splits, 16
    # tiled splits), the case the split-major workgroup order is for
    "gqa_decode_8k_bf16": Problem(op="gqa", dtype="bf16", B=2, S=1, L=1, P=8191, Hq=8,
                                  Hkv=2, D=128, Dv=128, causal=1, lens_range=(3000, 8191)),
    "gqa_decode_8k_rows32_f16": Problem(op="gqa", dtype="f16", B=1, S=2, L=2, P=8190,
                                        Hq=16, Hkv=1, D=128, Dv=128, causal=1,
                                        lens_range=(5000, 8190)),
    "gqa_noncausal_f32": Problem(op="gqa", dtype="f32", B=2, S=40, L=40, Hq=4, Hkv=2, D=32,
                                 Dv=32, causal=0),
    "gqa_softcap_small_f32": Problem(op="gqa", dtype="f32", B=1, S=50, L=50, Hq=2, Hkv=1,
                                     D=48, Dv=48, causal=1, softcap=0.5, has_sink=True),
    "mha_cross_f16": Problem(op="mha", dtype="f16", B=2, S=70, L=333, Hq=4, Hkv=4, D=64,
                             Dv=64, kv_rank=4, causal=0, bias_bh=(1, 4), has_lens=True,
                             lens_range=(100, 333), has_proj_bias=True),
    # unidirectional with S != L (query i sits at P + i: every cached key and
    # the new keys 0..i), with and without a past; key padding beyond lengths
    "mha_unidir_cross_f16": Problem(op="mha", dtype="f16", B=2, S=70, L=150, Hq=4, Hkv=4, D=64,
                                    Dv=64, kv_rank=4, causal=1, has_lens=True,
                                    lens_range=(60, 150), bias_bh=(1, 4)),
    "mha_unidir_past_bf16": Problem(op="mha", dtype="bf16", B=2, S=90, L=40, P=70, Hq=2, Hkv=2,
                                    D=128, Dv=128, kv_rank=3, causal=1, has_lens=True,
                                    lens_range=(80, 110)),
    # additive bias with a power-of-two scale (Q pre-scaled, the bias in the
    # QK^T accumulator): head size 128 with an explicit scale, causal with a
    # past; MultiHeadAttention with a small filter value (added, not skipped)
    "attention_bias_pow2_scale_bf16": Problem(op="attention", dtype="bf16", B=2, S=90, L=150,
                                              P=20, Hq=8, Hkv=2, D=128, Dv=128, causal=1,
                                              has_lens=True, lens_range=(60, 170),
                                              bias_bh=(2, 8), scale=0.0625),
    "mha_filter_bias_f16": Problem(op="mha", dtype="f16", B=2, S=70, L=200, Hq=2, Hkv=2, D=64,
                                   Dv=64, kv_rank=4, causal=0, has_lens=True,
                                   lens_range=(50, 200), bias_bh=(1, 2), mask_filter_value=-3.0,
                                   has_proj_bias=True),
    "mha_self_bias_f32": Problem(op="mha", dtype="f32", B=2, S=33, L=33, P=20, Hq=3, Hkv=3,
                                 D=40, Dv=24, kv_rank=3, causal=1, bias_bh=(2, 3),
                                 has_lens=False),
    "mha_small_filter_bf16": Problem(op="mha", dtype="bf16", B=2, S=20, L=90, Hq=2, Hkv=2,
                                     D=64, Dv=64, kv_rank=4, causal=0, has_lens=True,
                                     lens_range=(10, 60), mask_filter_value=-2.0),
    "attention_rank4_bf16": Problem(op="attention", dtype="bf16", B=2, S=65, L=129, P=31,
                                    Hq=4, Hkv=2, D=128, Dv=128, q_rank=4, kv_rank=4, causal=1,
                                    has_lens=True, lens_range=(1, 160), bias_bh=(2, 4),
                                    softcap=10.0),
    "attention_dv_ne_d_f16": Problem(op="attention", dtype="f16", B=1, S=40, L=70, Hq=2,
                                     Hkv=1, D=96, Dv=160, causal=0, has_lens=False,
                                     scale=0.05),
    "gqa_headsize256_f32": Problem(op="gqa", dtype="f32", B=1, S=20, L=20, Hq=2, Hkv=1,
                                   D=256, Dv=256, causal=1),
    # rotary embedding (do_rotary): split halves, interleaved with a partial
    # rotary dimension and a past, and the fp32 path
    "gqa_rope_bf16": Problem(op="gqa", dtype="bf16", B=2, S=130, L=130, Hq=8, Hkv=2, D=128,
                             Dv=128, causal=1, rotary=1),
    "gqa_rope_past_interleaved_f16": Problem(op="gqa", dtype="f16", B=3, S=20, L=20, P=100,
                                             Hq=4, Hkv=2, D=64, Dv=64, causal=1,
                                             lens_range=(0, 100), rotary=1,
                                             rotary_interleaved=1, rotary_dim=32),
    "gqa_rope_window_f32": Problem(op="gqa", dtype="f32", B=2, S=17, L=17, P=40, Hq=4, Hkv=1,
                                   D=48, Dv=48, causal=1, window=9, lens_range=(5, 40),
                                   rotary=1, rotary_dim=16, rotary_max_pos=50),
    "gqa_rope_dim12_f16": Problem(op="gqa", dtype="f16", B=2, S=33, L=33, P=8, Hq=4, Hkv=2,
                                  D=64, Dv=64, causal=1, lens_range=(0, 8), rotary=1,
                                  rotary_dim=12),
    # split halves over part of the head (the pre-pass rotates Q too, and
    # copies the channels past the rotary dimension), rows not a multiple of
    # the pre-pass's 8-row workgroups, a past
    "gqa_rope_partial_split_bf16": Problem(op="gqa", dtype="bf16", B=2, S=37, L=37, P=12,
                                           Hq=8, Hkv=2, D=128, Dv=128, causal=1,
                                           lens_range=(3, 12), rotary=1, rotary_dim=64),
    # mask surface: BOOL masks (broadcast, short), FLOAT masks broadcast over
    # queries with a short last dimension (tiled path), int64 nonpad lengths,
    # MultiHeadAttention binary masks
    "attention_bool_mask_bf16": Problem(op="attention", dtype="bf16", B=2, S=65, L=130, Hq=4,
                                        Hkv=2, D=64, Dv=64, causal=0, has_lens=False,
                                        mask_kind="bool", mask_bhs=(2, 1, 1), mask_cols=100),
    "attention_bool_mask_full_f32": Problem(op="attention", dtype="f32", B=2, S=20, L=37, P=5,
                                            Hq=4, Hkv=1, D=32, Dv=32, causal=1, has_lens=True,
                                            lens_range=(10, 42), lens_i64=True,
                                            mask_kind="bool", mask_bhs=(1, 4, 20), softcap=3.0),
    "attention_float_mask_short_bf16": Problem(op="attention", dtype="bf16", B=2, S=70, L=200,
                                               Hq=8, Hkv=2, D=128, Dv=128, causal=0,
                                               has_lens=False, bias_bh=(1, 1),
                                               bias_s_bcast=True, bias_cols=170),
    "mha_binary_mask_bt_f16": Problem(op="mha", dtype="f16", B=3, S=30, L=90, Hq=4, Hkv=4,
                                      D=64, Dv=64, kv_rank=4, causal=0, has_lens=False,
                                      mask_kind="int32", mask_bhs=(3, 1, 1), bias_bh=(1, 4)),
    "mha_binary_mask_bst_f16": Problem(op="mha", dtype="f16", B=2, S=17, L=40, Hq=2, Hkv=2,
                                       D=64, Dv=64, kv_rank=4, causal=0, has_lens=False,
                                       mask_kind="int32", mask_bhs=(2, 1, 17)),
    # binary masks with few ones under a causal mask: many rows are all zeros
    # (a uniform shift that leaves the softmax as without the mask); rows of
    # 100 int32 elements take word loads up to the ragged last key tile
    "mha_binary_mask_sparse_causal_bf16": Problem(op="mha", dtype="bf16", B=2, S=100, L=100,
                                                  Hq=4, Hkv=4, D=128, Dv=128, kv_rank=4,
                                                  causal=1, has_lens=False, mask_kind="int32",
                                                  mask_bhs=(2, 1, 100), mask_p=0.05),
    # a small filter value: masked keys keep weight, so the added offset shows
    "mha_binary_mask_small_filter_f16": Problem(op="mha", dtype="f16", B=2, S=50, L=64, Hq=4,
                                                Hkv=4, D=64, Dv=64, kv_rank=4, causal=0,
                                                has_lens=False, mask_kind="int32",
                                                mask_bhs=(2, 1, 1), mask_p=0.5,
                                                mask_filter_value=-2.0, bias_bh=(2, 4)),
    # head size 128 without bias or mask: two query heads per KV head with a
    # variable past and a window; MultiHeadAttention cross-attention with one
    # head per group and ragged query and key ends; ai.onnx Attention with a
    # cache, nonpad lengths, softcap and few key tiles
    "gqa_gh2_past_window_f16": Problem(op="gqa", dtype="f16", B=2, S=150, L=150, P=90, Hq=4,
                                       Hkv=2, D=128, Dv=128, causal=1, window=100,
                                       lens_range=(10, 90)),
    "mha_cross_d128_bf16": Problem(op="mha", dtype="bf16", B=2, S=300, L=333, Hq=2, Hkv=2,
                                   D=128, Dv=128, kv_rank=4, causal=0, has_lens=False),
    "attention_cache_softcap_f16": Problem(op="attention", dtype="f16", B=2, S=65, L=60,
                                           P=31, Hq=8, Hkv=2, D=128, Dv=128, causal=1,
                                           has_lens=True, lens_range=(40, 91), softcap=5.0),
    # more head-size-128 cases without bias or mask: two query heads per KV
    # head with a window and a ragged end (no past), MultiHeadAttention
    # cross-attention with key-padding lengths (excluded), ai.onnx Attention
    # with nonpad lengths under a causal mask
    "gqa_gh2_window_f16": Problem(op="gqa", dtype="f16", B=2, S=150, L=150, Hq=4, Hkv=2,
                                  D=128, Dv=128, causal=1, window=100),
    "mha_cross_lens_d128_f16": Problem(op="mha", dtype="f16", B=2, S=90, L=200, Hq=4, Hkv=4,
                                       D=128, Dv=128, kv_rank=4, causal=0, has_lens=True,
                                       lens_range=(50, 200)),
    "attention_nonpad_d128_bf16": Problem(op="attention", dtype="bf16", B=2, S=100, L=130,
                                          Hq=8, Hkv=2, D=128, Dv=128, causal=1, has_lens=True,
                                          lens_range=(60, 130)),
    # MultiHeadAttention rank-3 self-attention with k / v projection-bias
    # segments, unidirectional with a past
    "mha_self_projbias_past_f16": Problem(op="mha", dtype="f16", B=2, S=40, L=40, P=30, Hq=4,
                                          Hkv=4, D=64, Dv=64, kv_rank=3, causal=1,
                                          has_lens=True, lens_range=(20, 70),
                                          has_proj_bias=True, sigma_proj=0.3),
    "mha_self_projbias_bf16": Problem(op="mha", dtype="bf16", B=2, S=100, L=100, Hq=4, Hkv=4,
                                      D=128, Dv=128, kv_rank=3, causal=0, has_lens=False,
                                      has_proj_bias=True, sigma_proj=0.3, bias_bh=(2, 1)),
    # decode-sized calls (at most 16 rows per KV head) through the decode
    # kernel's general score pipeline: a short BOOL mask over a cache, bias +
    # softcap with nonpad lengths at head size 64, a MultiHeadAttention int32
    # binary mask with projection bias and a past, softcap + sink + window
    "attention_decode_boolmask_bf16": Problem(op="attention", dtype="bf16", B=3, S=1, L=1,
                                              P=300, Hq=8, Hkv=2, D=128, Dv=128, causal=0,
                                              has_lens=False, mask_kind="bool",
                                              mask_bhs=(3, 1, 1), mask_cols=250),
    "attention_decode_bias_softcap_f16": Problem(op="attention", dtype="f16", B=2, S=2, L=2,
                                                 P=200, Hq=8, Hkv=2, D=64, Dv=64, causal=1,
                                                 has_lens=True, lens_range=(100, 202),
                                                 bias_bh=(2, 8), softcap=5.0),
    "mha_decode_binary_mask_projbias_f16": Problem(op="mha", dtype="f16", B=2, S=3, L=3, P=120,
                                                   Hq=4, Hkv=4, D=128, Dv=128, kv_rank=3,
                                                   causal=1, has_lens=False, mask_kind="int32",
                                                   mask_bhs=(2, 1, 1), mask_p=0.5,
                                                   mask_filter_value=-3.0, has_proj_bias=True,
                                                   sigma_proj=0.3),
    "gqa_decode_softcap_sink_bf16": Problem(op="gqa", dtype="bf16", B=3, S=1, L=1, P=500, Hq=16,
                                            Hkv=2, D=128, Dv=128, causal=1, window=200,
                                            softcap=30.0, has_sink=True, lens_range=(1, 500)),
    # head size 256 in the prefill kernel (one wavefront per SIMD): causal GQA
    # with ragged tiles, Attention with a cache, nonpad lengths, bias and
    # softcap, and a BOOL mask per query row
    "gqa_d256_causal_bf16": Problem(op="gqa", dtype="bf16", B=2, S=150, L=150, Hq=8, Hkv=2,
                                    D=256, Dv=256, causal=1),
    "attention_d256_bias_softcap_f16": Problem(op="attention", dtype="f16", B=2, S=70, L=100,
                                               P=20, Hq=4, Hkv=2, D=256, Dv=256, causal=1,
                                               has_lens=True, lens_range=(50, 120),
                                               bias_bh=(2, 4), softcap=8.0),
    "attention_d256_boolmask_bf16": Problem(op="attention", dtype="bf16", B=1, S=65, L=90, Hq=4,
                                            Hkv=1, D=256, Dv=256, causal=0, has_lens=False,
                                            mask_kind="bool", mask_bhs=(1, 1, 65)),
    # head size 256 in the decode kernel: a variable past, and bias + softcap
    "gqa_decode_d256_bf16": Problem(op="gqa", dtype="bf16", B=3, S=1, L=1, P=700, Hq=8, Hkv=2,
                                    D=256, Dv=256, causal=1, lens_range=(0, 700)),
    "attention_decode_d256_softcap_f16": Problem(op="attention", dtype="f16", B=2, S=2, L=2,
                                                 P=300, Hq=8, Hkv=2, D=256, Dv=256, causal=1,
                                                 has_lens=False, bias_bh=(2, 8), softcap=5.0),
    # head-size-64 softcap prefill without bias or mask (four wavefronts per
    # SIMD): window + sink with bf16 (fixed exponent offset), a cache and
    # nonpad lengths with f16 (running max)
    "gqa_d64_window_sink_softcap_bf16": Problem(op="gqa", dtype="bf16", B=2, S=200, L=200, Hq=8,
                                                Hkv=2, D=64, Dv=64, causal=1, window=90,
                                                softcap=3.0, has_sink=True),
    "attention_d64_cache_softcap_f16": Problem(op="attention", dtype="f16", B=2, S=150, L=150,
                                               P=40, Hq=4, Hkv=2, D=64, Dv=64, causal=1,
                                               has_lens=True, lens_range=(60, 191), softcap=5.0),
    # BOOL masks at head size 128 over several key tiles: with softcap and no
    # bias (the mask-only form), and with a bias and no softcap
    "attention_boolmask_softcap_bf16": Problem(op="attention", dtype="bf16", B=2, S=140, L=200,
                                               P=20, Hq=4, Hkv=2, D=128, Dv=128, causal=1,
                                               has_lens=True, lens_range=(120, 221),
                                               mask_kind="bool", mask_bhs=(2, 4, 140),
                                               softcap=4.0),
    "attention_boolmask_bias_f16": Problem(op="attention", dtype="f16", B=2, S=130, L=190,
                                           Hq=4, Hkv=2, D=128, Dv=128, causal=0, has_lens=False,
                                           mask_kind="bool", mask_bhs=(1, 1, 130),
                                           bias_bh=(2, 1)),
}


def _run(p, dev, **kw):
    c = olk.Call(p, dev, **kw)
    c.launch()
    torch.cuda.synchronize()
    return c


def tiled_capable(p, mode="fwd"):
    # attn_mask (BOOL and binary) runs in the prefill kernel and, for calls of
    # at most 16 rows per KV head, in the decode kernel, not in the tiled
    # split-KV partials; the qk output goes to the generic kernels
    if p.qk_mode is not None:
        return False
    if p.mask_kind and mode == "decode" and (p.Hq // p.Hkv) * p.S > 16:
        return False
    # head size 256 in decode: the decode kernel (up to 16 rows per KV head);
    # the tiled split partials take 64 / 128 only
    if p.D == 256 and mode == "decode" and (p.Hq // p.Hkv) * p.S > 16:
        return False
    return p.dtype in ("f16", "bf16") and p.D == p.Dv and p.D in (64, 128, 256)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("mode,kernel", [("fwd", "generic"), ("fwd", "tiled"),
                                         ("decode", "generic"), ("decode", "tiled"),
                                         ("fwd", "auto")])
def test_small_parity(name, mode, kernel):
    p = SMALL[name]
    if kernel == "tiled" and not tiled_capable(p, mode):
        pytest.skip("the matrix-core kernels cover f16/bf16 at head size 64, 128 or 256; "
                    "split-KV calls with attn_mask or head size 256 need at most 16 rows "
                    "per KV head")
    inp = make_inputs(p, 500 + list(SMALL).index(name))
    _say(f"[parity] {name} mode={mode} kernel={kernel}")
    c = _run(p, to_dev(inp), mode=mode, kernel=kernel)
    name_ran = olk.olk_last_kernel_name()
    if kernel != "generic" and tiled_capable(p, mode):
        assert "generic" not in name_ran, name_ran
        if mode == "decode" and (p.Hq // p.Hkv) * p.S <= 16 and (p.scale is None or p.scale > 0):
            # up to 16 rows per KV head: the decode kernel, bias / softcap /
            # masks through its general score pipeline
            assert name_ran == "olk_decode_split+combine", name_ran
    want = olk_ref.attention(p, inp)
    assert_close(p, y_logical(p, c.y), want)
    assert_present_exact(p, inp, c.present_k, c.present_v)


def _nan_y(p):
    return torch.full(y_shape(p), float("nan"), dtype=p.torch_dtype, device="cuda")


_ORACLE_Y = {}


def _oracle_y(name, p, inp):
    # one full oracle pass per workload and session (the largest takes ~15 s)
    if name not in _ORACLE_Y:
        _ORACLE_Y[name] = olk_ref.attention(p, inp)
    return _ORACLE_Y[name]


@pytest.mark.parametrize("name", WORKLOAD_ORDER)
def test_workload_parity(name):
    # the benchmark's launch configuration: prefill writes present only for
    # GroupQueryAttention; decode appends to a KV cache that already holds the past
    p, inp = workload(name)
    dev = to_dev(inp)
    y = _nan_y(p)
    if p.S == 1:
        pk = dev["past_k"].new_empty((p.B, p.Hkv, p.P + p.L, p.D))
        pv = dev["past_v"].new_empty((p.B, p.Hkv, p.P + p.L, p.Dv))
        pk[:, :, : p.P] = dev.pop("past_k")
        pv[:, :, : p.P] = dev.pop("past_v")
        _say(f"[parity] workload {name} decode in place")
        c = _run(p, dev, mode="decode", kv_inplace=True, present_k=pk, present_v=pv, y=y)
        mode = "decode"
    else:
        _say(f"[parity] workload {name} fwd")
        c = _run(p, dev, mode="fwd", want_present=(p.op == "gqa"), y=y)
        mode = "fwd"
    _say(f"[parity] {name} kernel={olk.olk_last_kernel_name()}")
    if tiled_capable(p, mode):
        assert "generic" not in olk.olk_last_kernel_name()
    assert_close(p, y_logical(p, c.y), _oracle_y(name, p, inp))
    if p.op == "gqa":
        assert_present_exact(p, inp, c.present_k, c.present_v)


def test_decode_workload_out_of_place():
    # the decode workload with present written out of place (past copied)
    name = "gqa_decode_f16"
    p, inp = workload(name)
    _say(f"[parity] workload {name} decode out of place")
    c = _run(p, to_dev(inp), mode="decode", y=_nan_y(p))
    assert_close(p, y_logical(p, c.y), _oracle_y(name, p, inp))
    assert_present_exact(p, inp, c.present_k, c.present_v)


@pytest.mark.parametrize("name", ["gqa_decode_f16", "gqa_decode_rows8_bf16",
                                  "gqa_decode_rows16_f16", "gqa_decode_8k_bf16",
                                  "gqa_decode_d256_bf16"])
def test_small_decode_inplace(name):
    # in-place KV cache at head size 128: the decode kernel appends the new
    # rows itself; Y against the oracle, present bit-exact over [0, total_b)
    p = SMALL[name]
    inp = make_inputs(p, 700 + list(SMALL).index(name))
    dev = to_dev(inp)
    pk = dev["past_k"].new_zeros((p.B, p.Hkv, p.T, p.D))
    pv = dev["past_v"].new_zeros((p.B, p.Hkv, p.T, p.Dv))
    pk[:, :, : p.P] = dev.pop("past_k")
    pv[:, :, : p.P] = dev.pop("past_v")
    _say(f"[parity] {name} decode in place")
    c = _run(p, dev, mode="decode", kv_inplace=True, present_k=pk, present_v=pv)
    assert olk.olk_last_kernel_name() == "olk_decode_split+combine"
    assert_close(p, y_logical(p, c.y), olk_ref.attention(p, inp))
    assert_present_exact(p, inp, c.present_k, c.present_v)


def test_fwd_equals_decode_and_is_deterministic():
    p = SMALL["gqa_past_f16"]
    inp = make_inputs(p, 77)
    dev = to_dev(inp)
    ys = []
    for mode in ("fwd", "fwd", "decode", "decode"):
        ys.append(_run(p, dev, mode=mode).y.clone())
    assert torch.equal(ys[0], ys[1])
    assert torch.equal(ys[2], ys[3])
    np.testing.assert_allclose(y_logical(p, ys[0]), y_logical(p, ys[2]), atol=2e-2)


def test_decode_kernel_poisoned_cache_tail():
    # In-place KV cache whose slots from each batch's past length on hold NaN
    # (the new step overwrites the first of them).  The decode kernel reads
    # only the key rows of its splits, so Y is finite, equal to the clean
    # cache's Y and to the oracle's.
    p = SMALL["gqa_decode_f16"]
    inp = make_inputs(p, 92)
    dev = to_dev(inp)
    lens = inp["lens"].numpy()

    def cache(poison):
        pk = torch.zeros((p.B, p.Hkv, p.T, p.D), dtype=p.torch_dtype, device="cuda")
        pv = torch.zeros((p.B, p.Hkv, p.T, p.Dv), dtype=p.torch_dtype, device="cuda")
        pk[:, :, : p.P] = dev["past_k"]
        pv[:, :, : p.P] = dev["past_v"]
        if poison:
            for b in range(p.B):
                past = int(lens[b]) + 1 - p.S
                pk[b, :, past:] = float("nan")
                pv[b, :, past:] = float("nan")
        return pk, pv

    run = {k: v for k, v in dev.items() if k not in ("past_k", "past_v")}
    ys = []
    for poison in (False, True):
        pk, pv = cache(poison)
        _say(f"[parity] decode kernel, poisoned cache tail={poison}")
        c = _run(p, run, mode="decode", kv_inplace=True, present_k=pk, present_v=pv)
        assert olk.olk_last_kernel_name() == "olk_decode_split+combine"
        ys.append(c.y.clone())
    assert torch.isfinite(ys[1].float()).all()
    assert torch.equal(ys[0], ys[1])
    assert_close(p, y_logical(p, ys[1]), olk_ref.attention(p, inp))


def test_poisoned_padding_and_guard_bands():
    # Cache slots beyond each batch's valid past hold NaN; outputs sit inside
    # guard bands.  Y must stay finite and equal the clean run; nothing may be
    # written outside the outputs or past each batch's total length.
    p = SMALL["gqa_past_f16"]
    inp = make_inputs(p, 91)
    clean = _run(p, to_dev(inp)).y.clone()
    lens = inp["lens"].numpy()
    for b in range(p.B):
        past = int(lens[b]) + 1 - p.S
        inp["past_k"][b, :, past:] = float("nan")
        inp["past_v"][b, :, past:] = float("nan")
    dev = to_dev(inp)
    guard = 4096
    # a value every element type represents exactly
    sentinel = -777.0 if p.dtype != "bf16" else -776.0

    def banded(shape):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * guard,), sentinel, dtype=p.torch_dtype, device="cuda")
        return buf, buf[guard: guard + n].view(shape)

    from transformer_attention_fwd_amd.workloads import present_shape, y_shape
    for mode in ("fwd", "decode"):
        by, y = banded(y_shape(p))
        bk, pk = banded(present_shape(p, False))
        bv, pv = banded(present_shape(p, True))
        pk.fill_(sentinel)
        pv.fill_(sentinel)
        c = _run(p, dev, mode=mode, y=y, present_k=pk, present_v=pv)
        assert torch.isfinite(c.y.float()).all()
        if mode == "fwd":
            assert torch.equal(c.y, clean)
        for buf in (by, bk, bv):
            assert (buf[:guard].float() == sentinel).all() and (buf[-guard:].float() == sentinel).all()
        for b in range(p.B):  # the tail beyond total_b is untouched
            total = int(lens[b]) + 1
            assert (pk[b, :, total:].float() == sentinel).all()
            assert (pv[b, :, total:].float() == sentinel).all()


def test_empty_and_degenerate_shapes():
    # no batch, no query rows, and a row with no allowed key (zeros)
    for p in (Problem(op="gqa", dtype="bf16", B=0, S=16, L=16, Hq=4, Hkv=2, D=64, Dv=64),
              Problem(op="attention", dtype="f16", B=2, S=0, L=16, Hq=2, Hkv=2, D=64, Dv=64,
                      has_lens=False)):
        inp = make_inputs(p, 5)
        c = _run(p, to_dev(inp))
        assert c.y.numel() == 0
    p = Problem(op="attention", dtype="bf16", B=2, S=5, L=40, Hq=2, Hkv=1, D=64, Dv=64,
                causal=0, has_lens=True)
    inp = make_inputs(p, 6, lens=np.array([0, 17]))
    for mode in ("fwd", "decode"):
        c = _run(p, to_dev(inp), mode=mode)
        y = y_logical(p, c.y)
        assert (y[0] == 0).all()
        assert_close(p, y, olk_ref.attention(p, inp))


def test_first_token_decode_and_full_cache():
    # past_b = 0 (first step) and past_b = P (cache full) in one batch
    p = Problem(op="gqa", dtype="bf16", B=2, S=1, L=1, P=256, Hq=8, Hkv=2, D=128, Dv=128,
                causal=1)
    inp = make_inputs(p, 8, lens=np.array([0, 256]))
    for mode in ("fwd", "decode"):
        c = _run(p, to_dev(inp), mode=mode)
        assert_close(p, y_logical(p, c.y), olk_ref.attention(p, inp))
        assert_present_exact(p, inp, c.present_k, c.present_v)


def test_rotary_decode_inplace_cache_append():
    # KV-cache decode with rotary: the cache holds rotated keys; the new key is
    # rotated at position past_b and appended in place
    p = Problem(op="gqa", dtype="bf16", B=4, S=1, L=1, P=300, Hq=8, Hkv=2, D=128, Dv=128,
                causal=1, lens_range=(0, 300), rotary=1)
    inp = make_inputs(p, 123)
    dev = to_dev(inp)
    pk = dev["past_k"].new_empty((p.B, p.Hkv, p.P + 1, p.D))
    pv = dev["past_v"].new_empty((p.B, p.Hkv, p.P + 1, p.Dv))
    pk[:, :, : p.P] = dev.pop("past_k")
    pv[:, :, : p.P] = dev.pop("past_v")
    for mode in ("decode", "fwd"):
        k0, v0 = pk.clone(), pv.clone()
        c = _run(p, dev, mode=mode, kv_inplace=True, present_k=k0, present_v=v0)
        _say(f"[parity] rotary inplace {mode} kernel={olk.olk_last_kernel_name()}")
        assert_close(p, y_logical(p, c.y), olk_ref.attention(p, inp))
        assert_present_exact(p, inp, c.present_k, c.present_v)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_qk_matmul_output(mode, dtype):
    # every stage of the score pipeline, with past, causal, nonpad lengths, a
    # BOOL mask, a FLOAT mask and softcap; Y must not change with the qk output
    p = Problem(op="attention", dtype=dtype, B=2, S=24, L=40, P=9, Hq=4, Hkv=2, D=64, Dv=64,
                causal=1, has_lens=True, lens_range=(20, 49), mask_kind="bool",
                mask_bhs=(2, 1, 24), bias_bh=(1, 4), softcap=4.0, qk_mode=mode)
    _check_qk(p, 700 + mode, ("fwd", "decode"))


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("D", [128, 256])
def test_qk_matmul_output_tiles(mode, D):
    # head sizes 128 and 256, several key tiles with T a multiple of 4 (16-byte
    # rows) and more than one 128-row query tile, through the matrix-core qk
    # kernel and the generic one
    p = Problem(op="attention", dtype="f16", B=2, S=150, L=130, P=30, Hq=4, Hkv=2, D=D,
                Dv=D, causal=1, has_lens=True, lens_range=(100, 160), mask_kind="bool",
                mask_bhs=(2, 4, 150), bias_bh=(2, 1), softcap=6.0, qk_mode=mode)
    _check_qk(p, 720 + mode, ("fwd", "decode", "fwd-generic"))


def _check_qk(p, seed, runs):
    inp = make_inputs(p, seed)
    for run in runs:
        mode_ = "decode" if run == "decode" else "fwd"
        kernel = "generic" if run.endswith("generic") else "auto"
        _say(f"[parity] qk mode={p.qk_mode} dtype={p.dtype} D={p.D} {run}")
        c = _run(p, to_dev(inp), mode=mode_, kernel=kernel)
        name = olk.olk_last_kernel_name()
        if p.dtype in ("f16", "bf16") and p.D in (64, 128, 256) and kernel != "generic":
            assert name.endswith("+olk_qk_mfma"), name
        else:
            assert name.endswith("+olk_qk"), name
        mode = p.qk_mode
        got = c.qk.detach().cpu().double().numpy()
        want = olk_ref.qk(p, inp, mode)
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin)
        tol = 1e-4 if mode == 3 else (2e-4 if p.dtype == "f32" else 2e-3)
        np.testing.assert_allclose(got[fin], want[fin], rtol=0, atol=tol)
        assert_close(p, y_logical(p, c.y), olk_ref.attention(p, inp))
