"""GPU parity of the backward pass (fa_bwd, called through the C ABI)
against the fp64 oracle's gradients.

Kernel parity: fa_bwd is handed the forward results the boundary specifies
(o rounded to the 16-bit type, lse in fp32), made here by the oracle, and is
compared with the oracle's gradients for the same definition (row term
D_i = dO_i . o_i with that o).  Small shapes compare every element, the
forward-pass workloads compare sampled query rows (dq) and key rows (dk,
dv).  Tolerance: max |g - g_ref| / max(max |g_ref|, 1e-3) per gradient.

End to end: fa_fwd then fa_bwd against the plain gradients, where the
16-bit o in D adds an error the test bounds (floor-aware comparison)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import WORKLOADS, bits, make_qkv, make_workload
from tests.parity_util import (bwd_floor_full, compare_grads, gpu_backward, gpu_backward_given,
                               note, oracle_backward, oracle_fwd_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def grad_inputs(B, H, N, d, dtype, seed, gain=1.0):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed, qk_gain=gain)
    do = make_qkv(B, H, N, d, dtype, seed=seed + 7919)[0]
    return q, k, v, do


def kernel_parity(q, k, v, do, causal, scale):
    o, lse = oracle_fwd_inputs(q, k, v, causal, scale)
    got = gpu_backward_given(q, k, v, o, lse, do, causal, scale)
    ref = oracle_backward(q, k, v, do, causal, scale, o=o)
    return compare_grads(got, ref, "f16" if q.dtype == torch.float16 else "bf16")


EDGE_N = [1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 300, 513]


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_edge_sweep(N, d, dtype, causal):
    note(f"[bwd parity] edge N={N} d={d} {dtype} causal={causal}")
    q, k, v, do = grad_inputs(1, 2, N, d, dtype, seed=N + d)
    rep = kernel_parity(q, k, v, do, causal, float(np.float32(1 / math.sqrt(d))))
    assert rep["ok"], rep


@pytest.mark.parametrize("B,H", [(3, 5), (2, 1)])
def test_bwd_batch_head_layout(B, H):
    note(f"[bwd parity] layout B={B} H={H}")
    q, k, v, do = grad_inputs(B, H, 200, 128, "bf16", seed=B * 10 + H)
    for causal in (False, True):
        rep = kernel_parity(q, k, v, do, causal, 0.08)
        assert rep["ok"], rep


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_scale_values(scale, dtype):
    note(f"[bwd parity] scale={scale} {dtype}")
    q, k, v, do = grad_inputs(1, 2, 150, 64, dtype, seed=31)
    for causal in (False, True):
        o, lse = oracle_fwd_inputs(q, k, v, causal, scale)
        got = gpu_backward_given(q, k, v, o, lse, do, causal, scale)
        if scale == 0.0:
            # dq = scale * (...) and dk likewise: exactly zero
            assert torch.count_nonzero(got[0].float()) == 0
            assert torch.count_nonzero(got[1].float()) == 0
        rep = compare_grads(got, oracle_backward(q, k, v, do, causal, scale, o=o), dtype)
        assert rep["ok"], rep


def test_bwd_peaky():
    note("[bwd parity] peaky x3")
    q, k, v, do = grad_inputs(1, 2, 384, 128, "bf16", seed=41, gain=3.0)
    for causal in (False, True):
        rep = kernel_parity(q, k, v, do, causal, float(np.float32(1 / math.sqrt(128))))
        assert rep["ok"], rep


WORKLOAD_NAMES = ["tiny", "n1k", "n1000", "n4k_causal", "n8k_causal_peaky", "n16k_d64"]


@pytest.mark.parametrize("name", WORKLOAD_NAMES)
def test_bwd_workload_sampled(name):
    """Full-size workloads: every dq/dk/dv element of a sample of rows.  Key
    rows are drawn from at most four heads (each needs a full pass over its
    head in the oracle)."""
    w = WORKLOADS[name]
    note(f"[bwd parity] workload {name}: {w.note}")
    q, k, v = make_workload(w, seed=0)
    do = make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=12345)[0]
    o, lse = oracle_fwd_inputs(q, k, v, w.causal, w.scale)
    got = gpu_backward_given(q, k, v, o, lse, do, w.causal, w.scale)
    BH, N = w.B * w.H, w.N
    rng = np.random.default_rng(7)
    qrows = np.unique(np.concatenate([rng.integers(0, BH * N, 48), [0, N - 1, BH * N - 1]]))
    heads = rng.choice(BH, size=min(4, BH), replace=False)
    krows = np.unique(np.concatenate([h * N + rng.integers(0, N, 12) for h in heads] +
                                     [[heads[0] * N, heads[0] * N + N - 1]]))
    rq, rk, rv = oracle.attn_bwd_rows(bits(q), bits(k), bits(v), bits(do), w.dtype, w.causal,
                                      w.scale, qrows, krows, o=bits(o))
    gq = got[0].reshape(-1, w.d)[torch.from_numpy(qrows)]
    gk = got[1].reshape(-1, w.d)[torch.from_numpy(krows)]
    gv = got[2].reshape(-1, w.d)[torch.from_numpy(krows)]
    rep = compare_grads((gq, gk, gv), (rq, rk, rv), w.dtype)
    print(name, rep)
    assert rep["ok"], rep


# ---------------------------------------------------------------- end to end

@pytest.mark.parametrize("N,d,dtype,causal", [(2, 64, "bf16", True), (77, 128, "bf16", False),
                                              (257, 64, "f16", True), (520, 128, "bf16", True)])
def test_bwd_end_to_end(N, d, dtype, causal):
    """fa_fwd -> fa_bwd against the plain gradients; each element may also
    carry the first-order error of the 16-bit o in D (bound computed from the
    oracle's P and O)."""
    note(f"[bwd parity] end to end N={N} d={d} {dtype} causal={causal}")
    q, k, v, do = grad_inputs(1, 2, N, d, dtype, seed=N * 3 + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    got = gpu_backward(q, k, v, do, causal, scale)
    rep = compare_grads(got, oracle_backward(q, k, v, do, causal, scale), dtype,
                        floor=bwd_floor_full(q, k, v, do, causal, scale))
    print(rep)
    assert rep["ok"], rep


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dk_sums_to_zero_and_dv_sums_to_do(causal):
    note(f"[bwd parity] column sums causal={causal}")
    q, k, v, do = grad_inputs(1, 2, 333, 128, "f16", seed=51)
    o, lse = oracle_fwd_inputs(q, k, v, causal, 0.1)
    dq, dk, dv = gpu_backward_given(q, k, v, o, lse, do, causal, 0.1)
    dk64, dv64 = dk.double().numpy(), dv.double().numpy()
    # each row of dS sums to zero (up to the rounding of o in D), so
    # sum_j dK_j ~ 0; each row of P sums to one, so sum_j dV_j = sum_i dO_i
    ref = oracle_backward(q, k, v, do, causal, 0.1, o=o)
    assert np.abs(dk64.sum(2) - ref[1].sum(2)).max() <= 333 * 2e-3 * np.abs(ref[1]).max()
    assert np.abs(ref[2].sum(2) - do.double().numpy().sum(2)).max() < 1e-9
    assert np.abs(dv64.sum(2) - do.double().numpy().sum(2)).max() <= 333 * 2e-3 * np.abs(dv64).max()


def test_bwd_zero_upstream_gives_zero():
    note("[bwd parity] dO = 0")
    q, k, v, _ = grad_inputs(2, 2, 190, 64, "bf16", seed=53)
    do = torch.zeros_like(q)
    for causal in (False, True):
        dq, dk, dv = gpu_backward(q, k, v, do, causal, 0.2)
        for g in (dq, dk, dv):
            assert torch.count_nonzero(g.float()) == 0


def test_bwd_constant_v():
    note("[bwd parity] constant V")
    q, k, _, do = grad_inputs(1, 2, 257, 128, "bf16", seed=54)
    u = torch.randn(128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    v = u.reshape(1, 1, 1, 128).expand(1, 2, 257, 128).contiguous()
    for causal in (False, True):
        # o = u exactly (a convex combination of equal rows), so D_i = dO_i . u
        # = dP_ij for every j: dS = 0, dq = dk = 0 exactly in the oracle
        o, lse = oracle_fwd_inputs(q, k, v, causal, 0.1)
        assert torch.equal(o, v)
        dq, dk, dv = gpu_backward_given(q, k, v, o, lse, do, causal, 0.1)
        ref = oracle_backward(q, k, v, do, causal, 0.1, o=o)
        assert np.abs(ref[0]).max() < 1e-12 and np.abs(ref[1]).max() < 1e-12
        dvs = np.abs(ref[2]).max()
        assert dq.double().abs().max().item() <= 1e-3 * dvs
        assert dk.double().abs().max().item() <= 1e-3 * dvs
        assert compare_grads((dq, dk, dv), ref, "bf16")["err_dv"] <= 1e-2


def test_bwd_deterministic():
    note("[bwd parity] determinism")
    q, k, v, do = grad_inputs(1, 4, 700, 128, "bf16", seed=61)
    a = gpu_backward(q, k, v, do, True, 0.09)
    b = gpu_backward(q, k, v, do, True, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_attention_backward_helper():
    note("[bwd parity] attention_backward() helper")
    q, k, v, do = (t.cuda() for t in grad_inputs(1, 2, 96, 64, "f16", seed=63))
    o, lse = fa.attention(q, k, v, causal=True)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    ref = oracle_backward(q.cpu(), k.cpu(), v.cpu(), do.cpu(), True, 64 ** -0.5)
    rep = compare_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, "f16",
                        floor=bwd_floor_full(q.cpu(), k.cpu(), v.cpu(), do.cpu(), True, 64 ** -0.5))
    assert rep["ok"], rep
