"""GPU parity of the dropout forward and backward passes (fa_fwd_dropout,
fa_bwd_dropout, called through the C ABI) against the fp64 oracle's
dropout attention, which draws the same Philox4x32-10 pattern from its own
implementation.

Forward: lse to 1e-3 (it is the undropped one).  o to the forward
tolerance (2e-3 fp16 / 1e-2 bf16), or else, per element, to tol plus two
first-order floors: pf = u * sum_j P_ij Z_ij |v_jc| (the 16-bit P operand,
u = 2^-11 fp16 / 2^-8 bf16) and half a 16-bit ulp at |o| + pf (the output
rounding of a value already off by up to pf).  Without dropout the kernel
divides by the sum of the rounded weights, so the rounding of a dominant
weight cancels; with dropout the kept weights are not a convex combination
and that error stays, and the kept weights are scaled by 256 / T (x256 at
T = 1), so |o| and its ulp grow with them.

Backward (kernel parity): fa_bwd_dropout handed o (the oracle's dropout
output rounded to 16 bits) and lse, against the oracle's gradients for the
same o, max |g - g_ref| / max(max |g_ref|, 1e-3) within 2e-3 / 1e-2.

Dropped and kept elements are decided by integer comparisons on both sides,
so the pattern itself is exact: a single wrong byte moves a weight by its
whole size and fails the tolerance."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import TOL_LSE, TOL_O, compare_grads, note, ulp16

pytestmark = pytest.mark.gpu

_TD = {"f16": torch.float16, "bf16": torch.bfloat16}
_U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def _dt(t):
    return "f16" if t.dtype == torch.float16 else "bf16"


def thr(p):
    return oracle.dropout_threshold(float(np.float32(p)))


def gpu_fwd_dropout(q, k, v, causal, scale, p, seed, offset):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd_dropout(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale, p, seed, offset,
                           dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


def gpu_bwd_dropout(q, k, v, o, lse, do, causal, scale, p, seed, offset):
    dev = torch.device("cuda", 0)
    qd, kd, vd, od, dod = (t.to(dev).contiguous() for t in (q, k, v, o, do))
    ld = lse.to(dev).contiguous()
    B, H, N, d = q.shape
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    st = fa.fa_bwd_dropout(qd, kd, vd, od, dod, ld, ws, dq, dk, dv, B, H, N, d, int(causal),
                           scale, p, seed, offset, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def oracle_fwd_dropout(q, k, v, causal, scale, p, seed, offset):
    return oracle.attn_fwd_dropout(bits(q), bits(k), bits(v), _dt(q), causal,
                                   float(np.float32(scale)), thr(p), seed, offset)


def p_round_floor(q, k, v, causal, scale, p, seed, offset):
    """u * sum_j P_ij Z_ij |v_jc|: first-order effect of rounding the kept
    weights to the 16-bit MFMA operand."""
    dt = _dt(q)
    B, H, N, d = q.shape
    P = oracle.attn_probs(bits(q), bits(k), bits(v), dt, causal, float(np.float32(scale)))
    Z = oracle.dropout_factors(B * H, N, seed, offset, thr(p)).reshape(B, H, N, N)
    return _U[dt] * ((P * Z) @ np.abs(v.double().numpy()))


def check_fwd(q, k, v, causal, scale, p, seed, offset):
    dt = _dt(q)
    o, lse = gpu_fwd_dropout(q, k, v, causal, scale, p, seed, offset)
    ro, rl = oracle_fwd_dropout(q, k, v, causal, scale, p, seed, offset)
    og, lg = o.double().numpy(), lse.double().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    err = np.abs(og - ro)
    lerr = float(np.abs(lg - rl).max())
    assert lerr <= TOL_LSE, lerr
    tol = TOL_O[dt]
    if err.max() <= tol:
        return float(err.max())
    pf = p_round_floor(q, k, v, causal, scale, p, seed, offset)
    floor = pf + 0.5 * ulp16(np.abs(ro) + pf, dt)
    bad = err > tol + floor
    assert not bad.any(), (float(err.max()), int(bad.sum()), float((err - tol - floor).max()))
    return float(err.max())


SEED = 0x5EED0000ABCD1234   # both key words non-zero

EDGE_N = [1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 255, 256, 257, 300, 513]


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_edge_sweep(N, d, dtype, causal):
    note(f"[dropout fwd] N={N} d={d} {dtype} causal={causal}")
    q, k, v = make_qkv(1, 2, N, d, dtype, seed=N * 3 + d)
    check_fwd(q, k, v, causal, float(np.float32(1 / math.sqrt(d))), 0.2, SEED, 7)


@pytest.mark.parametrize("p", [0.0, 0.05, 0.5, 0.9, 0.998, 0.999])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fwd_probabilities(p, dtype):
    """p = 0 keeps everything (T = 256); p = 0.998 keeps only byte 0
    (T = 1, kept weights x256); p = 0.999 drops everything (T = 0: o = 0)."""
    note(f"[dropout fwd] p={p} {dtype}")
    q, k, v = make_qkv(1, 2, 300, 64, dtype, seed=17)
    for causal in (False, True):
        if thr(p) == 0:
            o, lse = gpu_fwd_dropout(q, k, v, causal, 0.125, p, SEED, 1)
            _, rl = oracle_fwd_dropout(q, k, v, causal, 0.125, p, SEED, 1)
            assert torch.all(o == 0)
            assert float(np.abs(lse.double().numpy() - rl).max()) <= TOL_LSE
        else:
            check_fwd(q, k, v, causal, 0.125, p, SEED, 1)


@pytest.mark.parametrize("B,H", [(3, 5), (2, 1)])
def test_fwd_batch_head_layout(B, H):
    """The head index b*H+h is a counter word: a wrong one fails."""
    note(f"[dropout fwd] layout B={B} H={H}")
    q, k, v = make_qkv(B, H, 200, 128, "bf16", seed=B * 7 + H)
    for causal in (False, True):
        check_fwd(q, k, v, causal, 0.09, 0.3, SEED, 2)


@pytest.mark.parametrize("seed,offset", [(0, 0), (1, 0), (0xFFFFFFFF, 5), (1 << 32, 5),
                                         (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF)])
def test_fwd_seed_and_offset_words(seed, offset):
    note(f"[dropout fwd] seed={seed:#x} offset={offset:#x}")
    q, k, v = make_qkv(1, 1, 130, 64, "f16", seed=3)
    check_fwd(q, k, v, True, 0.125, 0.25, seed, offset)


def test_fwd_reproducible_and_offset_changes_pattern():
    note("[dropout fwd] reproducibility")
    q, k, v = make_qkv(2, 2, 500, 128, "bf16", seed=11)
    a = gpu_fwd_dropout(q, k, v, False, 0.088, 0.1, SEED, 9)
    b = gpu_fwd_dropout(q, k, v, False, 0.088, 0.1, SEED, 9)
    c = gpu_fwd_dropout(q, k, v, False, 0.088, 0.1, SEED, 10)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[1], c[1])
    assert not torch.equal(a[0], c[0])


def test_fwd_workload_shape():
    """Several 256-row Q blocks and 128-key tiles, a ragged tail, causal."""
    note("[dropout fwd] B1 H2 N1100 d128 bf16 causal")
    q, k, v = make_qkv(1, 2, 1100, 128, "bf16", seed=5)
    check_fwd(q, k, v, True, float(np.float32(1 / math.sqrt(128))), 0.1, SEED, 0)


# ---------------------------------------------------------------- backward

def grad_inputs(B, H, N, d, dtype, seed):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed)
    do = make_qkv(B, H, N, d, dtype, seed=seed + 7919)[0]
    return q, k, v, do


def oracle_given(q, k, v, causal, scale, p, seed, offset):
    """The (o, lse) a dropout backward is handed, made by the oracle."""
    o, lse = oracle_fwd_dropout(q, k, v, causal, scale, p, seed, offset)
    return torch.from_numpy(o).to(q.dtype), torch.from_numpy(lse).to(torch.float32)


def bwd_kernel_parity(q, k, v, do, causal, scale, p, seed, offset):
    o, lse = oracle_given(q, k, v, causal, scale, p, seed, offset)
    got = gpu_bwd_dropout(q, k, v, o, lse, do, causal, scale, p, seed, offset)
    ref = oracle.attn_bwd_dropout(bits(q), bits(k), bits(v), bits(do), bits(o), _dt(q), causal,
                                  float(np.float32(scale)), thr(p), seed, offset)
    return compare_grads(got, ref, _dt(q))


@pytest.mark.parametrize("N", EDGE_N)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_edge_sweep(N, d, dtype, causal):
    note(f"[dropout bwd] N={N} d={d} {dtype} causal={causal}")
    q, k, v, do = grad_inputs(1, 2, N, d, dtype, seed=N + 5 * d)
    rep = bwd_kernel_parity(q, k, v, do, causal, float(np.float32(1 / math.sqrt(d))), 0.2,
                            SEED, 7)
    assert rep["ok"], rep


@pytest.mark.parametrize("p", [0.0, 0.5, 0.998, 0.999])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bwd_probabilities(p, dtype):
    """p = 0.999 (T = 0): dv = 0 exactly and dS = -P D."""
    note(f"[dropout bwd] p={p} {dtype}")
    q, k, v, do = grad_inputs(1, 2, 200, 64, dtype, seed=23)
    for causal in (False, True):
        rep = bwd_kernel_parity(q, k, v, do, causal, 0.125, p, SEED, 3)
        assert rep["ok"], rep


@pytest.mark.parametrize("B,H", [(3, 5), (2, 1)])
def test_bwd_batch_head_layout(B, H):
    note(f"[dropout bwd] layout B={B} H={H}")
    q, k, v, do = grad_inputs(B, H, 170, 128, "bf16", seed=B * 3 + H)
    for causal in (False, True):
        rep = bwd_kernel_parity(q, k, v, do, causal, 0.09, 0.3, SEED, 4)
        assert rep["ok"], rep


@pytest.mark.parametrize("seed,offset", [(0, 0), (1 << 32, 1), (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF)])
def test_bwd_seed_and_offset_words(seed, offset):
    note(f"[dropout bwd] seed={seed:#x} offset={offset:#x}")
    q, k, v, do = grad_inputs(1, 1, 100, 64, "f16", seed=8)
    rep = bwd_kernel_parity(q, k, v, do, True, 0.125, 0.25, seed, offset)
    assert rep["ok"], rep


def test_bwd_workload_shape():
    note("[dropout bwd] B1 H2 N700 d128 bf16 causal")
    q, k, v, do = grad_inputs(1, 2, 700, 128, "bf16", seed=6)
    rep = bwd_kernel_parity(q, k, v, do, True, float(np.float32(1 / math.sqrt(128))), 0.1,
                            SEED, 0)
    assert rep["ok"], rep


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_end_to_end_same_pattern(dtype, causal):
    """fa_fwd_dropout then fa_bwd_dropout on the GPU's own o and lse: the
    backward must redraw the forward's pattern.  Checked against the oracle
    (given its own rounded o) with the first-order floor of the o
    difference in D = dO . o: |dD_i| <= sum_c |dO_ic| e_ic, e the forward's
    own bound (tol + floors) plus the rounding of the oracle's o, carried
    into dq and dk through P."""
    note(f"[dropout e2e] {dtype} causal={causal}")
    q, k, v, do = grad_inputs(1, 2, 257, 64, dtype, seed=40)
    scale, p, seed, off = 0.125, 0.15, SEED, 12
    o, lse = gpu_fwd_dropout(q, k, v, causal, scale, p, seed, off)
    got = gpu_bwd_dropout(q, k, v, o, lse, do, causal, scale, p, seed, off)
    ro, _ = oracle_fwd_dropout(q, k, v, causal, scale, p, seed, off)
    o16 = torch.from_numpy(ro).to(q.dtype)
    ref = oracle.attn_bwd_dropout(bits(q), bits(k), bits(v), bits(do), bits(o16), dtype, causal,
                                  scale, thr(p), seed, off)
    # |o_gpu - o16| <= |o_gpu - o| + |o - o16|: the forward bound plus one
    # more output rounding
    pf = p_round_floor(q, k, v, causal, scale, p, seed, off)
    e = TOL_O[dtype] + pf + ulp16(np.abs(ro) + pf, dtype)
    b = (np.abs(do.double().numpy()) * e).sum(-1)
    P = oracle.attn_probs(bits(q), bits(k), bits(v), dtype, causal, scale)
    fdq = scale * b[..., None] * (P @ np.abs(k.double().numpy()))
    fdk = scale * (np.swapaxes(P, -1, -2) @ (b[..., None] * np.abs(q.double().numpy())))
    rep = compare_grads(got, ref, dtype, floor=(fdq, fdk, np.zeros_like(fdq)))
    assert rep["ok"], rep


# ---------------------------------------------------------------- full size

# The dropout launch bench.py times: the B1 H32 N8192 d128 bf16 causal
# workload with Q, K x3, p = 0.1, this seed and offset 0.
BENCH_DROPOUT = ("n8k_causal_peaky", 0.1, 0x243F6A8885A308D3, 0)


def _sample_rows(BH, N, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, BH * N, n),
                                     [0, 1, N - 1, N, BH * N - 2, BH * N - 1]]))


def test_fwd_full_size_sampled():
    """fa_fwd_dropout on the whole benchmarked workload; sampled rows against
    the oracle's row variant.  The P-operand floor uses Z <= 256/T:
    pf <= u (256/T) sum_j P_ij |v_jc|, P from the row's fp64 softmax."""
    from io_aware_transformer_amd.inputs import WORKLOADS, make_workload
    name, p, seed, off = BENCH_DROPOUT
    w = WORKLOADS[name]
    note(f"[dropout fwd] full size {name}: {w.note}, p={p}")
    q, k, v = make_workload(w, seed=0)
    o, lse = gpu_fwd_dropout(q, k, v, w.causal, w.scale, p, seed, off)
    rows = _sample_rows(w.B * w.H, w.N, 300, 11)
    ro, rl = oracle.attn_fwd_dropout_rows(bits(q), bits(k), bits(v), w.dtype, w.causal,
                                          w.scale, thr(p), seed, off, rows)
    og = o.reshape(-1, w.d)[torch.from_numpy(rows)].double().numpy()
    lg = lse.reshape(-1)[torch.from_numpy(rows)].double().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert float(np.abs(lg - rl).max()) <= TOL_LSE
    err = np.abs(og - ro)
    tol = TOL_O[w.dtype]
    if err.max() > tol:
        q64 = q.double().numpy().reshape(-1, w.N, w.d)
        k64 = k.double().numpy().reshape(-1, w.N, w.d)
        v64 = np.abs(v.double().numpy().reshape(-1, w.N, w.d))
        pf = np.empty_like(ro)
        for t, r in enumerate(rows):
            h, i = divmod(int(r), w.N)
            s = w.scale * (k64[h] @ q64[h, i])
            if w.causal:
                s[i + 1:] = -np.inf
            pr = np.exp(s - s.max())
            pf[t] = (pr / pr.sum()) @ v64[h]
        pf *= _U[w.dtype] * 256.0 / thr(p)
        bad = err > tol + pf + 0.5 * ulp16(np.abs(ro) + pf, w.dtype)
        assert not bad.any(), (float(err.max()), int(bad.sum()))


def test_bwd_full_size_sampled():
    """fa_bwd_dropout on the whole benchmarked workload, handed the oracle's
    full dropout forward (o rounded to bf16, lse in fp32); sampled query rows
    (dq) and key rows of four heads (dk, dv) against the oracle's row
    variant, R16's normalised tolerance."""
    from io_aware_transformer_amd.inputs import WORKLOADS, make_workload
    name, p, seed, off = BENCH_DROPOUT
    w = WORKLOADS[name]
    note(f"[dropout bwd] full size {name}: {w.note}, p={p}")
    q, k, v = make_workload(w, seed=0)
    do = make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=12345)[0]
    o, lse = oracle_given(q, k, v, w.causal, w.scale, p, seed, off)
    got = gpu_bwd_dropout(q, k, v, o, lse, do, w.causal, w.scale, p, seed, off)
    BH, N = w.B * w.H, w.N
    rng = np.random.default_rng(5)
    qrows = _sample_rows(BH, N, 48, 6)
    heads = rng.choice(BH, size=min(4, BH), replace=False)
    krows = np.unique(np.concatenate([h * N + rng.integers(0, N, 12) for h in heads] +
                                     [[heads[0] * N, heads[0] * N + N - 1]]))
    ref = oracle.attn_bwd_dropout_rows(bits(q), bits(k), bits(v), bits(do), bits(o), w.dtype,
                                       w.causal, w.scale, thr(p), seed, off, qrows, krows)
    gq = got[0].reshape(-1, w.d)[torch.from_numpy(qrows)]
    gk = got[1].reshape(-1, w.d)[torch.from_numpy(krows)]
    gv = got[2].reshape(-1, w.d)[torch.from_numpy(krows)]
    rep = compare_grads((gq, gk, gv), ref, w.dtype)
    print(name, rep)
    assert rep["ok"], rep
