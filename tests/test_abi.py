"""The C-ABI library on the host: it loads, exports every declared symbol,
its ctypes mirror matches the C struct layout, and olk_validate rejects each
invalid input with its status code.  No GPU is touched (olk_validate only
reads host memory; the pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

from transformer_attention_fwd_amd import olk
from transformer_attention_fwd_amd.workloads import WORKLOADS, Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "olk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(olk_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(olk.EXPORTED)
    lib = ctypes.CDLL(olk.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", olk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (olk_[a-z_]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_ctypes_structs_match_c_layout(tmp_path):
    fields_d = [f[0] for f in olk.olk_attn_desc._fields_]
    fields_i = [f[0] for f in olk.olk_attn_io._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){",
            'printf("%zu %zu\\n", sizeof(olk_attn_desc), sizeof(olk_attn_io));']
    for f in fields_d:
        prog.append(f'printf("%zu\\n", offsetof(olk_attn_desc, {f}));')
    for f in fields_i:
        prog.append(f'printf("%zu\\n", offsetof(olk_attn_io, {f}));')
    prog.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-o", str(exe), str(src)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(olk.olk_attn_desc)
    assert vals[1] == ctypes.sizeof(olk.olk_attn_io)
    offs = vals[2:]
    want = [getattr(olk.olk_attn_desc, f).offset for f in fields_d] + \
           [getattr(olk.olk_attn_io, f).offset for f in fields_i]
    assert offs == want


# Fake, distinct, well-separated "device" addresses: validation compares and
# range-checks them but never dereferences them.
_BASE = 1 << 40


def fake_io(p: Problem, **over):
    names = ["q", "k", "v", "past_k", "past_v", "seqlens", "attn_bias", "head_sink",
             "proj_bias", "y", "present_k", "present_v", "cos_cache", "sin_cache"]
    ptr = {n: _BASE + (i + 1) * (1 << 36) for i, n in enumerate(names)}
    if p.P == 0:
        ptr["past_k"] = ptr["past_v"] = None
    if p.bias_bh is None:
        ptr["attn_bias"] = None
    if not p.has_sink:
        ptr["head_sink"] = None
    if not p.has_proj_bias:
        ptr["proj_bias"] = None
    if p.op != "gqa" and not p.has_lens:
        ptr["seqlens"] = None
    if not p.rotary:
        ptr["cos_cache"] = ptr["sin_cache"] = None
    if p.mask_kind:
        ptr["attn_mask"] = _BASE + 50 * (1 << 36)
    ptr.update(over)
    return olk.olk_attn_io(**ptr)


def status(p, kernel="auto", kv_inplace=False, **io_over):
    d = olk.make_desc(p, kernel=kernel, kv_inplace=kv_inplace)
    return olk.olk_validate(d, fake_io(p, **io_over))


GQA = WORKLOADS["gqa_prefill_causal_bf16"]
DEC = WORKLOADS["gqa_decode_f16"]
MHA = WORKLOADS["mha_cross_f16"]


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workloads_validate(name):
    assert status(WORKLOADS[name]) == olk.OLK_OK


def test_window_rules():
    # local_window_size: -1 or positive; 0 and below -1 rejected; needs causal
    assert status(GQA.with_(window=-1)) == olk.OLK_OK
    assert status(GQA.with_(window=1)) == olk.OLK_OK
    assert status(GQA.with_(window=2**31 - 1)) == olk.OLK_OK
    assert status(GQA.with_(window=0)) == olk.OLK_E_ATTR
    assert status(GQA.with_(window=-2)) == olk.OLK_E_ATTR
    assert status(GQA.with_(window=512, causal=0)) == olk.OLK_E_ATTR
    assert status(MHA.with_(window=16, causal=1)) == olk.OLK_E_ATTR


def test_head_rules():
    assert status(GQA.with_(Hq=30)) == olk.OLK_E_SHAPE  # 30 % 8 != 0
    assert status(GQA.with_(Hkv=0)) == olk.OLK_E_SHAPE
    assert status(MHA.with_(Hkv=10)) == olk.OLK_E_SHAPE  # MHA has one head count
    assert status(GQA.with_(D=0)) == olk.OLK_E_SHAPE
    assert status(GQA.with_(D=512, Dv=512)) == olk.OLK_E_UNSUPPORTED


def test_operator_specific_rejections():
    assert status(GQA.with_(L=GQA.S + 1)) == olk.OLK_E_SHAPE        # GQA: L == S
    assert status(GQA.with_(kv_rank=4)) == olk.OLK_E_SHAPE
    assert status(GQA, seqlens=None) == olk.OLK_E_NULL               # seqlens_k required
    assert status(MHA.with_(has_sink=True)) == olk.OLK_E_ATTR        # sink is GQA-only
    assert status(MHA.with_(softcap=5.0)) == olk.OLK_E_ATTR
    assert status(MHA.with_(kv_rank=3)) == olk.OLK_OK                # rank-3 K/V bias segments
    # their biased rows are written to present: present is required then
    assert status(MHA.with_(kv_rank=3), present_k=None, present_v=None) == olk.OLK_E_UNSUPPORTED
    att = Problem(op="attention", dtype="bf16", B=2, S=8, L=8, Hq=4, Hkv=2, D=64, Dv=64)
    assert status(att) == olk.OLK_OK
    assert status(att.with_(has_proj_bias=True)) == olk.OLK_E_ATTR
    assert status(att, kv_inplace=True) == olk.OLK_E_ATTR
    assert status(MHA.with_(mask_filter_value=float("inf"))) == olk.OLK_E_ATTR


def test_attribute_values():
    assert status(GQA.with_(scale=float("nan"))) == olk.OLK_E_ATTR
    assert status(GQA.with_(softcap=-1.0)) == olk.OLK_E_ATTR
    assert status(GQA.with_(softcap=float("nan"))) == olk.OLK_E_ATTR
    d = olk.make_desc(GQA)
    d.causal = 2
    assert olk.olk_validate(d, fake_io(GQA)) == olk.OLK_E_ATTR
    d = olk.make_desc(GQA)
    d.dtype = 7
    assert olk.olk_validate(d, fake_io(GQA)) == olk.OLK_E_ATTR
    d = olk.make_desc(GQA)
    d.op = 9
    assert olk.olk_validate(d, fake_io(GQA)) == olk.OLK_E_ATTR


def test_required_pointers():
    for n in ("q", "k", "v", "y"):
        assert status(GQA, **{n: None}) == olk.OLK_E_NULL, n
    assert status(DEC, past_k=None) == olk.OLK_E_NULL
    assert olk.olk_validate(None, fake_io(GQA)) == olk.OLK_E_NULL


def test_bias_extents():
    assert status(MHA.with_(bias_bh=(8, 20))) == olk.OLK_OK
    assert status(MHA.with_(bias_bh=(3, 20))) == olk.OLK_E_SHAPE
    assert status(MHA.with_(bias_bh=(1, 7))) == olk.OLK_E_SHAPE


def test_inplace_rules():
    # present holds the past: past pointers absent or equal to present
    assert status(DEC, kv_inplace=True, past_k=None, past_v=None) == olk.OLK_OK
    io = fake_io(DEC)
    d = olk.make_desc(DEC, kv_inplace=True)
    io.past_k, io.past_v = io.present_k, io.present_v
    assert olk.olk_validate(d, io) == olk.OLK_OK
    assert status(DEC, kv_inplace=True) == olk.OLK_E_SHAPE  # distinct past buffer
    assert status(DEC, kv_inplace=True, past_k=None, past_v=None,
                  present_k=None) == olk.OLK_E_NULL


def test_overlapping_outputs_rejected():
    io = fake_io(GQA)
    d = olk.make_desc(GQA)
    io.y = io.q
    assert olk.olk_validate(d, io) == olk.OLK_E_SHAPE
    io = fake_io(GQA)
    io.present_v = io.present_k + 64
    assert olk.olk_validate(d, io) == olk.OLK_E_SHAPE


def test_workspace_size_depends_on_sizes_only():
    d = olk.make_desc(DEC)
    n = olk.olk_workspace_bytes(d)
    assert n > 0 and n % 256 == 0
    assert olk.olk_workspace_bytes(olk.make_desc(DEC.with_(B=0))) == 0


def test_status_strings():
    for s in range(7):
        assert olk.olk_status_str(s)
    assert olk.olk_last_kernel_name() == ""


def test_rotary_rules():
    rope = GQA.with_(rotary=1)
    assert status(rope) == olk.OLK_OK
    assert status(rope.with_(rotary_dim=64, rotary_interleaved=1)) == olk.OLK_OK
    assert status(rope.with_(rotary_dim=63)) == olk.OLK_E_ATTR     # odd R
    assert status(rope.with_(rotary_dim=130)) == olk.OLK_E_ATTR    # R > D
    assert status(rope, cos_cache=None) == olk.OLK_E_NULL
    # the rotated keys live in present: present outputs are required
    assert status(rope, present_k=None, present_v=None) == olk.OLK_E_UNSUPPORTED
    # GroupQueryAttention only
    mha = MHA.with_(rotary=1)
    assert status(mha) == olk.OLK_E_ATTR
    d = olk.make_desc(rope)
    d.do_rotary = 2
    assert olk.olk_validate(d, fake_io(rope)) == olk.OLK_E_ATTR
    d = olk.make_desc(rope)
    d.rotary_max_pos = 0
    assert olk.olk_validate(d, fake_io(rope)) == olk.OLK_E_SHAPE
    # caches are inputs: they must not overlap the outputs
    io = fake_io(rope)
    io.cos_cache = io.y
    assert olk.olk_validate(olk.make_desc(rope), io) == olk.OLK_E_SHAPE


def test_mask_rules():
    att = Problem(op="attention", dtype="bf16", B=2, S=8, L=8, Hq=4, Hkv=2, D=64, Dv=64,
                  has_lens=False)
    mha = MHA.with_(has_lens=False)

    def st(p, **io):
        d = olk.make_desc(p)
        f = fake_io(p, **io)
        if p.mask_kind:
            f.attn_mask = _BASE + 40 * (1 << 36)
        return olk.olk_validate(d, f)

    assert st(att.with_(mask_kind="bool", mask_bhs=(1, 1, 8))) == olk.OLK_OK
    assert st(att.with_(mask_kind="bool", mask_bhs=(2, 4, 1), mask_cols=5)) == olk.OLK_OK
    assert st(att.with_(mask_kind="bool", mask_bhs=(3, 1, 1))) == olk.OLK_E_SHAPE
    assert st(att.with_(mask_kind="bool", mask_bhs=(1, 1, 8), mask_cols=9)) == olk.OLK_E_SHAPE
    assert st(GQA.with_(mask_kind="bool", mask_bhs=(1, 1, 1))) == olk.OLK_E_ATTR  # GQA: none
    assert st(mha.with_(mask_kind="int32", mask_bhs=(8, 1, 1))) == olk.OLK_OK
    assert st(mha.with_(mask_kind="bool", mask_bhs=(8, 1, 1))) == olk.OLK_E_ATTR
    # one key-padding input: lengths or a binary mask
    assert st(MHA.with_(mask_kind="int32", mask_bhs=(8, 1, 1))) == olk.OLK_E_ATTR
    assert st(mha.with_(mask_kind="int32", mask_bhs=(8, 1, 1), mask_cols=7)) == olk.OLK_E_SHAPE
    d = olk.make_desc(att.with_(mask_kind="bool", mask_bhs=(1, 1, 8)))
    assert olk.olk_validate(d, fake_io(att)) == olk.OLK_E_NULL          # mask pointer missing
    # short FLOAT masks and query-broadcast bias rows
    assert status(att.with_(bias_bh=(1, 1), bias_s_bcast=True, bias_cols=3)) == olk.OLK_OK
    assert status(MHA.with_(bias_bh=(1, 20), bias_cols=10)) == olk.OLK_E_SHAPE
    # int64 nonpad lengths and the qk output are ai.onnx Attention features
    assert status(att.with_(has_lens=True, lens_i64=True)) == olk.OLK_OK
    assert status(GQA.with_(lens_i64=True)) == olk.OLK_E_ATTR
    qk = _BASE + 41 * (1 << 36)
    assert status(att.with_(qk_mode=3), qk_out=qk) == olk.OLK_OK
    assert status(att.with_(qk_mode=4), qk_out=qk) == olk.OLK_E_ATTR
    assert status(GQA.with_(qk_mode=0), qk_out=qk) == olk.OLK_E_ATTR
    io = fake_io(att)
    io.qk_out = io.q
    assert olk.olk_validate(olk.make_desc(att.with_(qk_mode=0)), io) == olk.OLK_E_SHAPE


def test_backward_rules():
    p = Problem(op="gqa", dtype="bf16", B=2, S=64, L=64, Hq=8, Hkv=2, D=128, Dv=128, causal=1)
    names = ["q", "k", "v", "seqlens", "dy", "dq", "dk", "dv"]

    def st(p, ws=1 << 20, **over):
        ptr = {n: _BASE + (i + 1) * (1 << 36) for i, n in enumerate(names)}
        ptr.update(over)
        io = olk.olk_attn_bwd_io(**ptr)
        return olk.olk_attention_bwd(olk.make_desc(p), io, _BASE + 60 * (1 << 36), ws, 0)

    # invalid inputs are rejected before anything is launched
    assert st(p, dy=None) == olk.OLK_E_NULL
    assert st(p, seqlens=None) == olk.OLK_E_NULL
    assert st(p.with_(P=4)) == olk.OLK_E_UNSUPPORTED          # no past
    assert st(p.with_(softcap=5.0)) == olk.OLK_E_UNSUPPORTED
    assert st(p.with_(rotary=1)) == olk.OLK_E_UNSUPPORTED
    assert st(p.with_(op="mha", Hkv=8, kv_rank=3)) == olk.OLK_E_UNSUPPORTED
    assert st(p, ws=16) == olk.OLK_E_WORKSPACE
    assert st(p, dk=_BASE + 1 * (1 << 36)) == olk.OLK_E_SHAPE  # dk overlaps q
    n = olk.olk_bwd_workspace_bytes(olk.make_desc(p))
    assert n >= 2 * 4 * 2 * 64 * 8 and n % 256 == 0
