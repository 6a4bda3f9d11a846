"""Helpers for the GPU tests: run the HIP forward through the C ABI on a layer
dict from synth (or a hand-built one) and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import bit_rank_post_amd as tq
from bit_rank_post_amd import io as tqio

Y_DT = {"f16": tq.TQ_F16, "bf16": tq.TQ_BF16, "f32": tq.TQ_F32}
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()    # raises if the library is missing


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_forward(L, x, ids, gates, act, y_dtype="f32", ws=None):
    """Returns y as float64 numpy [T][d_out] and the dropped-slot count."""
    T, k = ids.shape
    xd, idd, gd = tqio.tokens_to_device(x, ids, gates, act)
    d_out = L.d_ff if L.kind == tq.TQ_SINGLE else L.d_model
    y = torch.empty((T, d_out), dtype=TORCH_DT[y_dtype], device="cuda")
    if ws is None:
        ws = tqio.workspace(L, T, k)
    L.forward(xd, T, idd, gd, k, y, Y_DT[y_dtype], ws)
    torch.cuda.synchronize()
    dropped = int(ws[:4].view(torch.int32).item())
    return y.to(torch.float64).cpu().numpy(), dropped


def bf16_half_ulp(v):
    """Half a unit in the last place of bf16 at |v| (v fp64)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def assert_parity(y, y_ref, y_dtype="f32", tol=2e-3, what=""):
    """max|dy| <= tol * ||y_ref||_inf (plus half a bf16 ulp for bf16 outputs)."""
    scale = float(np.max(np.abs(y_ref)))
    err = np.abs(y - y_ref)
    bound = tol * scale + (bf16_half_ulp(y_ref) if y_dtype == "bf16" else 0.0)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  parity {what}: max|dy| = {float(err.max()):.3e}, ||y||inf = {scale:.3e}, "
        f"worst err/bound = {worst:.3f}")
    assert np.all(err <= bound), f"{what}: max|dy| {err.max()} > bound"
    return worst
