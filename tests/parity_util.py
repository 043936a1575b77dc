"""Helpers for GPU-vs-oracle parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle under the stated tolerances.

Tolerances (max absolute error): O 2e-3 for fp16 outputs, 1e-2 for bf16
outputs; lse 1e-3.  Besides the strict check, the floor-aware check allows
each element tol + |round_dtype(o_exact) - o_exact|, the error that even a
perfectly rounded 16-bit output has; the number of elements whose rounding
floor alone exceeds tol is reported with it."""
from __future__ import annotations

import sys

import numpy as np
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits

TOL_O = {"f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
_TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def note(msg: str) -> None:
    """Name the case on stderr before a GPU step (survives a lost box)."""
    print(msg, file=sys.stderr, flush=True)


def dtype_name(t: torch.Tensor) -> str:
    return "f16" if t.dtype == torch.float16 else "bf16"


def gpu_forward(q, k, v, causal: bool, scale: float, stream=None):
    """Copy CPU q, k, v to cuda:0, run fa_fwd with NaN-filled outputs, and
    return (o, lse) as CPU tensors."""
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


def oracle_forward(q, k, v, causal: bool, scale: float):
    return oracle.attn_fwd(bits(q), bits(k), bits(v), dtype_name(q), causal,
                           float(np.float32(scale)))


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str) -> dict:
    """Error report of the GPU outputs against the fp64 oracle."""
    og = o_gpu.double().numpy()
    lg = lse_gpu.double().numpy()
    err = np.abs(og - o_ref)
    lerr = np.abs(lg - lse_ref)
    tol = TOL_O[dtype]
    floor = np.abs(torch.from_numpy(o_ref).to(_TD[dtype]).double().numpy() - o_ref)
    return {
        "finite": bool(np.isfinite(og).all() and np.isfinite(lg).all()),
        "max_err_o": float(err.max(initial=0.0)),
        "max_err_lse": float(lerr.max(initial=0.0)),
        "strict_ok": bool(err.max(initial=0.0) <= tol and lerr.max(initial=0.0) <= TOL_LSE),
        "floor_ok": bool(np.all(err <= tol + floor) and lerr.max(initial=0.0) <= TOL_LSE),
        "floor_max": float(floor.max(initial=0.0)),
        "n_floor_over_tol": int(np.count_nonzero(floor > tol)),
        "n_over_tol": int(np.count_nonzero(err > tol)),
        "tol": tol,
    }


def assert_parity(rep: dict) -> None:
    """Strict pass, or -- only where the exact result rounded to the output
    type already misses the tolerance somewhere -- the floor-aware pass."""
    assert rep["finite"], rep
    if rep["strict_ok"]:
        return
    assert rep["n_floor_over_tol"] > 0 and rep["floor_ok"], rep
