"""olk_attention_decode_noalloc (split partials in the library's built-in
scratch instead of a caller workspace) against olk_attention_decode on the
same inputs: two calls in a row, the second smaller, so the scratch still holds
the first call's partials when the second runs; and a call whose partials would
not fit the scratch, which must be rejected with nothing launched."""
import sys

import numpy as np
import pytest
import torch

from oracle import olk_ref
from tests.parity import assert_close, assert_present_exact, to_dev, y_logical
from transformer_attention_fwd_amd.workloads import Problem, make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from transformer_attention_fwd_amd import olk

# the first is an in-place KV cache (as the decode benchmark), the second a
# smaller out-of-place call on another kernel (head size 64, window + sink)
CASES = [
    ("inplace_f16_d128", True,
     Problem(op="gqa", dtype="f16", B=16, S=1, L=1, P=6000, Hq=32, Hkv=8, D=128, Dv=128,
             causal=1, lens_range=(500, 6000))),
    ("outofplace_bf16_d64", False,
     Problem(op="gqa", dtype="bf16", B=3, S=2, L=2, P=700, Hq=8, Hkv=2, D=64, Dv=64,
             causal=1, window=300, has_sink=True, lens_range=(10, 700))),
]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _call(p, dev, inplace):
    # present starts as zeros, so the rows beyond each batch's length (left
    # untouched by the kernels) are the same in every call
    d = dict(dev)
    pk = d["past_k"].new_zeros((p.B, p.Hkv, p.T, p.D))
    pv = d["past_v"].new_zeros((p.B, p.Hkv, p.T, p.Dv))
    if not inplace:
        return olk.Call(p, d, mode="decode", present_k=pk, present_v=pv)
    pk[:, :, : p.P] = d.pop("past_k")
    pv[:, :, : p.P] = d.pop("past_v")
    return olk.Call(p, d, mode="decode", kv_inplace=True, present_k=pk, present_v=pv)


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    stream = torch.cuda.current_stream().cuda_stream
    sizes = []
    for k, (name, inplace, p) in enumerate(CASES):
        inp = make_inputs(p, 900 + k)
        dev = to_dev(inp)
        ref = _call(p, dev, inplace)
        sizes.append(ref.ws_bytes)
        assert 0 < ref.ws_bytes <= olk.NOALLOC_SCRATCH_BYTES
        _say(f"[noalloc] {name}: decode with workspace ({ref.ws_bytes} B)")
        ref.launch()
        c = _call(p, dev, inplace)
        c.y.fill_(float("nan"))
        _say(f"[noalloc] {name}: decode with the built-in scratch")
        st = olk.olk_attention_decode_noalloc(c.desc, c.io, stream)
        assert st == olk.OLK_OK, olk.olk_status_str(st)
        torch.cuda.synchronize()
        # the same kernels and plan: bit-identical to the workspace call
        assert torch.equal(c.y, ref.y)
        for a, b in ((c.present_k, ref.present_k), (c.present_v, ref.present_v)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert_close(p, y_logical(p, c.y), olk_ref.attention(p, inp))
        assert_present_exact(p, inp, c.present_k, c.present_v)
        if not inplace:
            tot = inp["lens"].numpy().astype(np.int64) + 1
            for bi in range(p.B):
                assert (c.present_k[bi, :, tot[bi]:] == 0).all()
                assert (c.present_v[bi, :, tot[bi]:] == 0).all()
    assert sizes[1] < sizes[0]


def test_noalloc_decode_rejects_partials_beyond_the_scratch():
    # 4096 query rows x 256 key chunks of partials: far beyond the scratch
    p = Problem(op="gqa", dtype="f16", B=1, S=16, L=16, P=131056, Hq=256, Hkv=1, D=128,
                Dv=128, causal=1)
    inp = make_inputs(p, 950)
    c = olk.Call(p, to_dev(inp), mode="fwd")
    assert olk.olk_workspace_bytes(c.desc) > olk.NOALLOC_SCRATCH_BYTES
    c.y.fill_(float("nan"))
    torch.cuda.synchronize()
    _say("[noalloc] oversized call (rejected before any launch)")
    st = olk.olk_attention_decode_noalloc(c.desc, c.io, torch.cuda.current_stream().cuda_stream)
    assert st == olk.OLK_E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(c.y.float()).all()
