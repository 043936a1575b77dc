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
        # the kernel's own error beyond the rounding floor: how much of the
        # tolerance the floor-aware check leaves unused (tol minus this)
        "max_err_beyond_floor": float((err - floor).max(initial=0.0)),
        "tol": tol,
    }


def assert_parity(rep: dict) -> None:
    """Strict pass, or -- only where the exact result rounded to the output
    type already misses the tolerance somewhere -- the floor-aware pass."""
    assert rep["finite"], rep
    if rep["strict_ok"]:
        return
    assert rep["n_floor_over_tol"] > 0 and rep["floor_ok"], rep


# ---------------------------------------------------------------- backward

# Backward tolerance: max |g - g_ref| over a gradient tensor, divided by
# max(max |g_ref|, G_FLOOR) of that tensor.  The same numbers as the
# forward's O tolerance, applied to gradients normalised by their own scale
# (gradient magnitudes depend on N and on the softmax spread, O's do not).
# The floor covers tensors whose exact value is zero or nearly so (one key:
# dS = 0, so dq = dk = 0 exactly, while the 16-bit O in D = dO . O leaves
# rounding noise); with standard-normal inputs real gradients are >= 1e-2.
TOL_G = {"f16": 2e-3, "bf16": 1e-2}
G_FLOOR = 1e-3


def gpu_backward(q, k, v, do, causal: bool, scale: float, stream=None):
    """fa_fwd for (o, lse), then fa_bwd, on cuda:0 with NaN-filled outputs.
    Returns CPU (dq, dk, dv)."""
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = (t.to(dev).contiguous() for t in (q, k, v, do))
    B, H, N, d = q.shape
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    st = fa.fa_fwd(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    st = fa.fa_bwd(qd, kd, vd, o, dod, lse, ws, dq, dk, dv, B, H, N, d, int(causal), scale,
                   dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def oracle_backward(q, k, v, do, causal: bool, scale: float, o=None):
    return oracle.attn_bwd(bits(q), bits(k), bits(v), bits(do), dtype_name(q), causal,
                           float(np.float32(scale)), o=None if o is None else bits(o))


def oracle_fwd_inputs(q, k, v, causal: bool, scale: float):
    """The forward results a backward pass is handed, made by the oracle: the
    exact O rounded to the 16-bit type and lse rounded to fp32."""
    o, lse = oracle_forward(q, k, v, causal, scale)
    return (torch.from_numpy(o).to(q.dtype), torch.from_numpy(lse).to(torch.float32))


def gpu_backward_given(q, k, v, o, lse, do, causal: bool, scale: float, stream=None):
    """fa_bwd alone on cuda:0 with the given (o, lse); NaN-filled outputs and
    workspace.  Returns CPU (dq, dk, dv)."""
    dev = torch.device("cuda", 0)
    qd, kd, vd, od, dod = (t.to(dev).contiguous() for t in (q, k, v, o, do))
    ld = lse.to(dev).contiguous()
    B, H, N, d = q.shape
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    st = fa.fa_bwd(qd, kd, vd, od, dod, ld, ws, dq, dk, dv, B, H, N, d, int(causal), scale,
                   dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def ulp16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the 16-bit type at |x| (0 at 0)."""
    if dtype == "f16":
        return np.spacing(np.abs(x).astype(np.float16)).astype(np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 7), 0.0)


def _o_error_bound(o_exact: np.ndarray, do: np.ndarray, dtype: str) -> np.ndarray:
    """b_i >= |D_i(o used) - D_i(exact)|: O rounded to the 16-bit type plus one
    more ulp for the forward pass's own deviation, summed against |dO_i|."""
    r16 = torch.from_numpy(o_exact).to(_TD[dtype]).double().numpy()
    e = np.abs(o_exact - r16) + ulp16(o_exact, dtype)
    return (np.abs(do) * e).sum(-1)


def bwd_floor_full(q, k, v, do, causal: bool, scale: float):
    """First-order bounds on dq and dk errors from the 16-bit O in D = dO . O
    (full tensors, small N): dS_ij changes by -P_ij dD_i, so
    |d dq_ic| <= |scale| b_i sum_j P_ij |k_jc| and
    |d dk_jc| <= |scale| sum_i P_ij b_i |q_ic|.  dv does not depend on D."""
    dt = dtype_name(q)
    sc = float(np.float32(scale))
    o, _ = oracle.attn_fwd(bits(q), bits(k), bits(v), dt, causal, sc)
    P = oracle.attn_probs(bits(q), bits(k), bits(v), dt, causal, sc)
    b = _o_error_bound(o, do.double().numpy(), dt)
    aq, ak = np.abs(q.double().numpy()), np.abs(k.double().numpy())
    fdq = abs(sc) * b[..., None] * (P @ ak)
    fdk = abs(sc) * (np.swapaxes(P, -1, -2) @ (b[..., None] * aq))
    return fdq, fdk, np.zeros_like(fdq)


def bwd_floor_rows(q, k, v, do, causal: bool, scale: float, qrows, krows):
    """The same bounds on sampled flat query rows (dq) and key rows (dk, dv);
    the heads of the key rows are evaluated in full by the oracle."""
    dt = dtype_name(q)
    sc = float(np.float32(scale))
    B, H, N, d = q.shape
    q64 = q.double().numpy().reshape(B * H, N, d)
    k64 = k.double().numpy().reshape(B * H, N, d)
    do64 = do.double().numpy().reshape(B * H, N, d)
    heads = sorted(set((np.asarray(qrows) // N).tolist()) | set((np.asarray(krows) // N).tolist()))
    info = {}
    for h in heads:
        sl = lambda t: t.reshape(B * H, N, d)[h:h + 1].reshape(1, 1, N, d).contiguous()
        o, lse = oracle.attn_fwd(bits(sl(q)), bits(sl(k)), bits(sl(v)), dt, causal, sc)
        info[h] = (lse[0, 0], _o_error_bound(o[0, 0], do64[h], dt))
    def prow(h, i):   # P_i. for query i of head h
        s = sc * (k64[h] @ q64[h, i])
        if causal:
            s[i + 1:] = -np.inf
        return np.exp(s - info[h][0][i])
    fdq = np.stack([abs(sc) * info[r // N][1][r % N] * (prow(r // N, r % N) @ np.abs(k64[r // N]))
                    for r in qrows])
    fdk = []
    for r in krows:
        h, j = r // N, r % N
        s = sc * (q64[h] @ k64[h, j])
        pcol = np.exp(s - info[h][0])
        if causal:
            pcol[:j] = 0.0
        fdk.append(abs(sc) * ((pcol * info[h][1]) @ np.abs(q64[h])))
    fdk = np.stack(fdk)
    return fdq, fdk, np.zeros_like(fdk)


def compare_grads(got, ref, dtype: str, floor=None) -> dict:
    """Normalised max errors of (dq, dk, dv) against fp64 references (any
    matching shapes: full tensors or sampled rows).  ok: every element within
    tol * max(max |ref|, G_FLOOR), plus, when floor is given, that element's
    first-order bound of the error the 16-bit O in D brings (floor-aware)."""
    rep = {"finite": True, "tol": TOL_G[dtype], "strict_ok": True, "ok": True}
    floors = floor if floor is not None else (None, None, None)
    for name, g, r, f in zip(("dq", "dk", "dv"), got, ref, floors):
        g = g.double().numpy() if isinstance(g, torch.Tensor) else np.asarray(g, np.float64)
        r = np.asarray(r, np.float64)
        rep["finite"] &= bool(np.isfinite(g).all())
        scale_r = max(float(np.abs(r).max(initial=0.0)), G_FLOOR)
        err = np.abs(g - r)
        rep[f"err_{name}"] = float(err.max(initial=0.0)) / scale_r
        rep[f"max_{name}"] = scale_r
        strict = bool(np.all(err <= rep["tol"] * scale_r))
        rep["strict_ok"] &= strict
        if f is not None:
            rep[f"floor_max_{name}"] = float(np.max(f, initial=0.0)) / scale_r
            rep["ok"] &= bool(np.all(err <= rep["tol"] * scale_r + f))
        else:
            rep["ok"] &= strict
    rep["ok"] = bool(rep["ok"] and rep["finite"])
    return rep
