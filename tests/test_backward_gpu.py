"""GPU parity of the GroupQueryAttention backward (olk_attention_bwd through
the C ABI) against the oracle's float64 gradients."""
import sys

import numpy as np
import pytest
import torch

from oracle import olk_ref
from tests.parity import to_dev
from transformer_attention_fwd_amd.workloads import Problem, make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from transformer_attention_fwd_amd import olk

MFMA = "olk_bwd_dq_mfma+dkv_mfma"
VALU = "olk_bwd_stats+dq+dkv"
# name -> (problem, kernel path the library must take)
CASES = {
    "bf16_d128_causal": (Problem(op="gqa", dtype="bf16", B=2, S=130, L=130, Hq=8, Hkv=2, D=128,
                                 Dv=128, causal=1), MFMA),
    "f16_d64_window": (Problem(op="gqa", dtype="f16", B=2, S=97, L=97, Hq=4, Hkv=4, D=64, Dv=64,
                               causal=1, window=20), MFMA),
    "f32_noncausal_dv": (Problem(op="gqa", dtype="f32", B=1, S=45, L=45, Hq=6, Hkv=2, D=48,
                                 Dv=32, causal=0), VALU),
    "bf16_medium": (Problem(op="gqa", dtype="bf16", B=1, S=512, L=512, Hq=8, Hkv=2, D=128,
                            Dv=128, causal=1), MFMA),
    # non-causal, 8 heads per KV head, ragged tails of both tile sizes
    "f16_d128_noncausal_g8": (Problem(op="gqa", dtype="f16", B=1, S=201, L=201, Hq=16, Hkv=2,
                                      D=128, Dv=128, causal=0), MFMA),
    # window shorter than a key tile, head size 64, two heads per KV head
    "bf16_d64_window5": (Problem(op="gqa", dtype="bf16", B=2, S=300, L=300, Hq=4, Hkv=2, D=64,
                                 Dv=64, causal=1, window=5), MFMA),
    # a sequence shorter than one tile
    "bf16_d128_tiny": (Problem(op="gqa", dtype="bf16", B=3, S=7, L=7, Hq=4, Hkv=1, D=128,
                               Dv=128, causal=1), MFMA),
    # three heads per KV head (not a power of two) takes the VALU kernels
    "bf16_g3_valu": (Problem(op="gqa", dtype="bf16", B=1, S=70, L=70, Hq=6, Hkv=2, D=64, Dv=64,
                             causal=1), VALU),
    "bf16_long": (Problem(op="gqa", dtype="bf16", B=1, S=1100, L=1100, Hq=8, Hkv=2, D=128,
                          Dv=128, causal=1), MFMA),
}
TOL = {"f32": 2e-4, "f16": 1e-2, "bf16": 2e-2}


def _dy(p, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(p.B, p.S, p.Hq * p.Dv, generator=g).to(p.torch_dtype)


def _check(name, got, want, tol):
    got = got.detach().cpu().double().numpy().reshape(want.shape)
    assert np.isfinite(got).all(), name
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got - want).max())
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol} * {scale:.2f}"


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    p, path = CASES[name]
    inp = make_inputs(p, 900 + list(CASES).index(name))
    dy = _dy(p, 5)
    print(f"[bwd] {name}", file=sys.stderr, flush=True)
    dev = to_dev(inp)
    c = olk.BwdCall(p, dev, dy.cuda())
    c.launch()
    torch.cuda.synchronize()
    assert olk.olk_last_kernel_name() == path
    dq, dk, dv = olk_ref.attention_bwd(p, inp, dy)
    tol = TOL[p.dtype]
    _check("dq", c.dq, dq, tol)
    _check("dk", c.dk, dk, tol)
    _check("dv", c.dv, dv, tol)
    # deterministic: a second call gives the same bits
    ref = (c.dq.clone(), c.dk.clone(), c.dv.clone())
    c.launch()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ref, (c.dq, c.dk, c.dv)))


def test_backward_full_size_slices():
    """The bf16 causal prefill shape (B=4, S=2048, Hq=32, Hkv=8, D=128) through
    the library as the backward benchmark launches it.  The gradients of one
    (batch, KV head) depend only on that slice of Q, K, V and dY, so the slice
    of the last batch and the first KV head is checked element by element
    against the oracle run on that slice alone (about 20 s of CPU)."""
    import dataclasses

    from transformer_attention_fwd_amd.workloads import workload
    p, inp = workload("gqa_prefill_causal_bf16")
    dy = _dy(p, 5)
    print("[bwd] full-size slices", file=sys.stderr, flush=True)
    dev = to_dev(inp)
    c = olk.BwdCall(p, dev, dy.cuda())
    c.launch()
    torch.cuda.synchronize()
    assert olk.olk_last_kernel_name() == MFMA
    G = p.Hq // p.Hkv
    got = {n: t.detach().cpu() for n, t in (("dq", c.dq), ("dk", c.dk), ("dv", c.dv))}
    del c, dev
    torch.cuda.empty_cache()
    sub = dataclasses.replace(p, B=1, Hq=G, Hkv=1)
    for b, g in ((p.B - 1, 0),):
        qs = slice(g * G * p.D, (g + 1) * G * p.D)
        ks = slice(g * p.D, (g + 1) * p.D)
        s_inp = {"q": inp["q"][b:b + 1, :, qs].contiguous(),
                 "k": inp["k"][b:b + 1, :, ks].contiguous(),
                 "v": inp["v"][b:b + 1, :, ks].contiguous(),
                 "lens": inp["lens"][b:b + 1].contiguous()}
        s_dy = dy[b:b + 1, :, g * G * p.Dv:(g + 1) * G * p.Dv].contiguous()
        dq, dk, dv = olk_ref.attention_bwd(sub, s_inp, s_dy)
        gq = got["dq"].view(p.B, p.S, p.Hq, p.D)[b:b + 1, :, g * G:(g + 1) * G]
        gk = got["dk"].view(p.B, p.S, p.Hkv, p.D)[b:b + 1, :, g:g + 1]
        gv = got["dv"].view(p.B, p.S, p.Hkv, p.Dv)[b:b + 1, :, g:g + 1]
        _check(f"dq[b={b},g={g}]", gq, dq, TOL["bf16"])
        _check(f"dk[b={b},g={g}]", gk, dk, TOL["bf16"])
        _check(f"dv[b={b},g={g}]", gv, dv, TOL["bf16"])
