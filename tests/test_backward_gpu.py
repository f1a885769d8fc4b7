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

CASES = {
    "bf16_d128_causal": Problem(op="gqa", dtype="bf16", B=2, S=130, L=130, Hq=8, Hkv=2, D=128,
                                Dv=128, causal=1),
    "f16_d64_window": Problem(op="gqa", dtype="f16", B=2, S=97, L=97, Hq=4, Hkv=4, D=64, Dv=64,
                              causal=1, window=20),
    "f32_noncausal_dv": Problem(op="gqa", dtype="f32", B=1, S=45, L=45, Hq=6, Hkv=2, D=48,
                                Dv=32, causal=0),
    "bf16_medium": Problem(op="gqa", dtype="bf16", B=1, S=512, L=512, Hq=8, Hkv=2, D=128,
                           Dv=128, causal=1),
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
    p = CASES[name]
    inp = make_inputs(p, 900 + list(CASES).index(name))
    dy = _dy(p, 5)
    print(f"[bwd] {name}", file=sys.stderr, flush=True)
    dev = to_dev(inp)
    c = olk.BwdCall(p, dev, dy.cuda())
    c.launch()
    torch.cuda.synchronize()
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
