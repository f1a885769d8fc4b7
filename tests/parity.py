"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare with the oracle element by element."""
from __future__ import annotations

import numpy as np
import torch

from oracle import olk_ref
from transformer_attention_fwd_amd.workloads import Problem, valid_lengths

# Max-abs tolerance of Y against the float64 oracle.
TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


def to_dev(inputs):
    return {k: v.to("cuda", non_blocking=False) for k, v in inputs.items()}


def y_logical(p: Problem, y: torch.Tensor) -> np.ndarray:
    """Y as float64 (B, S, Hq, Dv) whatever its rank."""
    y = y.detach().to("cpu").to(torch.float64)
    if p.q_rank == 3:
        return y.view(p.B, p.S, p.Hq, p.Dv).numpy()
    return y.permute(0, 2, 1, 3).contiguous().numpy()


def assert_close(p: Problem, got: np.ndarray, want: np.ndarray, what: str = "Y"):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    tol = TOL[p.dtype]
    if err.size:
        worst = np.unravel_index(np.argmax(err), err.shape)
        assert err.max() <= tol, (f"{what}: max abs err {err.max():.3e} > {tol} at {worst}: "
                                  f"got {got[worst]} want {want[worst]}")


def assert_present_exact(p: Problem, inputs, pk: torch.Tensor, pv: torch.Tensor):
    """Valid prefix [0, total_b) of present_key/value equals the oracle's bits."""
    ek, ev = olk_ref.present(p, inputs)
    tot = valid_lengths(p, inputs) if p.op == "gqa" else np.full(p.B, p.T)
    gk, gv = pk.detach().to("cpu"), pv.detach().to("cpu")
    iview = torch.int16 if ek.element_size() == 2 else torch.int32
    for b in range(p.B):
        n = int(tot[b])
        assert torch.equal(gk[b, :, :n].view(iview), ek[b, :, :n].view(iview)), f"present_k b={b}"
        assert torch.equal(gv[b, :, :n].view(iview), ev[b, :, :n].view(iview)), f"present_v b={b}"
