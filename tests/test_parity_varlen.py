"""GPU parity of the packed variable-length forward and backward passes
(fa_fwd_varlen, fa_bwd_varlen, called through the C ABI) against the oracle
(plain attention, and its gradients, on every sequence slice).

Forward: the forward tolerances, max abs 2e-3 (fp16 o) / 1e-2 (bf16 o),
1e-3 (lse), strict or floor-aware as for the other forward tests.

Backward: fa_bwd_varlen is handed the forward results the boundary
specifies, made by the oracle (o rounded to the 16-bit type, lse to fp32),
and compared with the oracle's gradients for that o.  Every sequence is its
own problem, so the normalised tolerance of the batched backward test
applies per sequence: max |g - g_ref| / max(max |g_ref| over the sequence,
1e-3).

Both: rows of tokens outside every sequence stay untouched (NaN sentinels),
and a batch of equal lengths reproduces fa_fwd / fa_bwd bit for bit."""
from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv, varlen_offsets
from tests.parity_util import (assert_parity, compare, compare_grads, gpu_backward_given, note,
                               oracle_fwd_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def packed(H, total, d, dtype, seed):
    """q, k, v as [H, total, d] CPU tensors (one draw of the seeded generator)."""
    return tuple(t[0] for t in make_qkv(1, H, total, d, dtype, seed=seed))


def gpu_varlen(q, k, v, cu, max_seqlen, causal, scale):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    H, total, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((H, total), float("nan"), dtype=torch.float32, device=dev)
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd_varlen(qd, kd, vd, o, lse, cud, len(cu) - 1, H, total, max_seqlen, d,
                          int(causal), scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


def check(q, k, v, cu, causal, scale, max_seqlen=None):
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    lens = np.diff(cu)
    ms = int(max(lens.max(initial=0), 1)) if max_seqlen is None else max_seqlen
    o, lse = gpu_varlen(q, k, v, cu, ms, causal, scale)
    ro, rl = oracle.attn_fwd_varlen(bits(q), bits(k), bits(v), dt, cu, causal,
                                    float(np.float32(scale)))
    end = cu[-1]
    # tokens outside every sequence: not written
    assert torch.isnan(o[:, end:]).all() and torch.isnan(lse[:, end:]).all()
    if end > 0:
        rep = compare(o[:, :end], lse[:, :end], ro[:, :end], rl[:, :end], dt)
        assert_parity(rep)
        return rep
    return None


CASES = [
    [0, 300, 300, 1000, 1001, 1300],     # an empty and a one-token sequence
    [0, 1, 2, 3],                        # one-token sequences only
    [0, 256, 512, 513],                  # exact Q-block multiples and a tail
    [0, 700],                            # one sequence
    [0, 37, 600, 1000, 1290],            # ragged, trailing tokens unused
]


@pytest.mark.parametrize("cu", CASES, ids=[str(len(c) - 1) + "seq-" + str(c[-1]) for c in CASES])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_cases(cu, d, dtype, causal):
    note(f"[varlen parity] cu={cu} d={d} {dtype} causal={causal}")
    total = cu[-1] + 7
    q, k, v = packed(3, total, d, dtype, seed=cu[-1] + d)
    check(q, k, v, cu, causal, float(np.float32(1 / math.sqrt(d))))


def test_varlen_long_mixed_lengths():
    """Long and short sequences together: several 256-row Q blocks, 128-key
    tiles, causal tile skipping per sequence."""
    cu = [0, 4096, 4113, 5113, 7613]
    note(f"[varlen parity] long mixed cu={cu}")
    q, k, v = packed(4, cu[-1], 128, "bf16", seed=9)
    check(q, k, v, cu, True, float(np.float32(1 / math.sqrt(128))))


def test_varlen_grid_larger_than_needed():
    """max_seqlen above the longest sequence only adds work-groups that exit."""
    cu = [0, 100, 350]
    q, k, v = packed(2, 350, 64, "f16", seed=12)
    a = gpu_varlen(q, k, v, cu, 250, True, 0.125)
    b = gpu_varlen(q, k, v, cu, 350, True, 0.125)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_fa_fwd(causal):
    """B sequences of length N packed into [H, B*N, d] give fa_fwd's bits."""
    note(f"[varlen parity] equal lengths causal={causal}")
    B, H, N, d = 3, 2, 333, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=21)
    dev = torch.device("cuda", 0)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    st = fa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, B, H, N, d, int(causal), 0.09,
                   fa.FA_DTYPE_BF16, torch.cuda.current_stream(dev))
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous()
    ov, lv = gpu_varlen(pack(q), pack(k), pack(v), [0, N, 2 * N, 3 * N], N, causal, 0.09)
    assert torch.equal(ov.view(torch.int16), pack(o.cpu()).view(torch.int16))
    assert torch.equal(lv, lse.cpu().permute(1, 0, 2).reshape(H, B * N))


def test_varlen_malformed_offsets_stay_in_bounds():
    """Offsets out of order and past total (the caller's contract broken):
    the kernel clamps them, so the call completes without touching memory
    outside the tensors, and the well-formed first sequence is written."""
    q, k, v = packed(1, 200, 64, "f16", seed=4)
    o, lse = gpu_varlen(q, k, v, [0, 150, 90, 5000], 200, False, 0.125)
    torch.cuda.synchronize()
    assert torch.isfinite(o[:, :150]).all()


@functools.lru_cache(maxsize=1)
def benchmarked_launch():
    """The launch bench.py times: 8 sequences of seeded lengths in [512, 8192]
    (24 900 tokens), 32 heads, d128 bf16 causal; inputs and the oracle's
    forward (computed once for both passes)."""
    cu = varlen_offsets(8, 512, 8192, seed=0)
    q, k, v = packed(32, cu[-1], 128, "bf16", seed=0)
    scale = float(np.float32(128 ** -0.5))
    ro, rl = oracle.attn_fwd_varlen(bits(q), bits(k), bits(v), "bf16", cu, True, scale)
    return cu, q, k, v, scale, ro, rl


def test_varlen_benchmarked_launch():
    """Every row of the benchmarked forward launch."""
    cu, q, k, v, scale, ro, rl = benchmarked_launch()
    note(f"[varlen parity] benchmarked launch cu={cu}")
    o, lse = gpu_varlen(q, k, v, cu, max(np.diff(cu)), True, scale)
    assert_parity(compare(o, lse, ro, rl, "bf16"))


# ---------------------------------------------------------------- backward

def oracle_fwd_given(q, k, v, cu, causal, scale):
    """The forward results handed to the backward pass, made by the oracle:
    o rounded to the 16-bit type, lse to fp32; rows outside every sequence
    NaN (the backward must not read them)."""
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    ro, rl = oracle.attn_fwd_varlen(bits(q), bits(k), bits(v), dt, cu, causal,
                                    float(np.float32(scale)))
    return rounded_given(ro, rl, q.dtype, cu)


def rounded_given(ro, rl, dtype, cu):
    o = torch.from_numpy(ro).to(dtype)
    lse = torch.from_numpy(rl).to(torch.float32)
    o[:, cu[-1]:] = float("nan")
    lse[:, cu[-1]:] = float("nan")
    return o, lse


def gpu_varlen_bwd(q, k, v, o, lse, do, cu, max_seqlen, causal, scale):
    """fa_bwd_varlen on cuda:0 with NaN-filled outputs and workspace; CPU
    (dq, dk, dv)."""
    dev = torch.device("cuda", 0)
    qd, kd, vd, od, dod = (t.to(dev).contiguous() for t in (q, k, v, o, do))
    ld = lse.to(dev).contiguous()
    H, total, d = q.shape
    B = len(cu) - 1
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    ws = torch.full((fa.fa_bwd_varlen_workspace_size(B, H, total) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_bwd_varlen(qd, kd, vd, od, dod, ld, cud, ws, dq, dk, dv, B, H, total, max_seqlen,
                          d, int(causal), scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def upstream(q, seed):
    H, total, d = q.shape
    return make_qkv(1, H, total, d, "f16" if q.dtype == torch.float16 else "bf16",
                    seed=seed)[0][0]


def check_bwd(q, k, v, do, cu, causal, scale, max_seqlen=None):
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    lens = np.diff(cu)
    ms = int(max(lens.max(initial=0), 1)) if max_seqlen is None else max_seqlen
    o, lse = oracle_fwd_given(q, k, v, cu, causal, scale)
    got = gpu_varlen_bwd(q, k, v, o, lse, do, cu, ms, causal, scale)
    ref = oracle.attn_bwd_varlen(bits(q), bits(k), bits(v), bits(do), bits(o), dt, cu, causal,
                                 float(np.float32(scale)))
    end = cu[-1]
    for g in got:   # tokens outside every sequence: not written
        assert torch.isnan(g[:, end:]).all()
    reps = []
    for lo, hi in zip(cu[:-1], cu[1:]):
        if hi == lo:
            continue
        rep = compare_grads(tuple(g[:, lo:hi] for g in got), tuple(r[:, lo:hi] for r in ref),
                            dt)
        assert rep["ok"], (lo, hi, rep)
        reps.append(rep)
    return reps


@pytest.mark.parametrize("cu", CASES, ids=[str(len(c) - 1) + "seq-" + str(c[-1]) for c in CASES])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_cases(cu, d, dtype, causal):
    note(f"[varlen bwd parity] cu={cu} d={d} {dtype} causal={causal}")
    total = cu[-1] + 7
    q, k, v = packed(3, total, d, dtype, seed=cu[-1] + d)
    do = upstream(q, seed=cu[-1] + d + 7919)
    check_bwd(q, k, v, do, cu, causal, float(np.float32(1 / math.sqrt(d))))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_long_mixed_lengths(causal):
    """A 4096-token sequence beside short ones: many 256-key and 256-query
    blocks per sequence, 32-row workspace blocks straddling no sequence."""
    cu = [0, 4096, 4113, 5113, 6000]
    note(f"[varlen bwd parity] long mixed cu={cu} causal={causal}")
    q, k, v = packed(2, cu[-1], 128, "bf16", seed=19)
    do = upstream(q, seed=20)
    check_bwd(q, k, v, do, cu, causal, float(np.float32(1 / math.sqrt(128))))


def test_varlen_bwd_grid_larger_than_needed():
    """max_seqlen above the longest sequence only adds work-groups that exit."""
    cu = [0, 100, 350]
    q, k, v = packed(2, 350, 64, "f16", seed=12)
    do = upstream(q, seed=13)
    o, lse = oracle_fwd_given(q, k, v, cu, True, 0.125)
    a = gpu_varlen_bwd(q, k, v, o, lse, do, cu, 250, True, 0.125)
    b = gpu_varlen_bwd(q, k, v, o, lse, do, cu, 350, True, 0.125)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_equal_lengths_is_fa_bwd(causal):
    """B sequences of length N packed into [H, B*N, d] give fa_bwd's bits."""
    note(f"[varlen bwd parity] equal lengths causal={causal}")
    B, H, N, d = 3, 2, 333, 128
    q, k, v = make_qkv(B, H, N, d, "bf16", seed=22)
    do = make_qkv(B, H, N, d, "bf16", seed=23)[0]
    o, lse = oracle_fwd_inputs(q, k, v, causal, 0.09)
    want = gpu_backward_given(q, k, v, o, lse, do, causal, 0.09)
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(H, B * N, d).contiguous()
    got = gpu_varlen_bwd(pack(q), pack(k), pack(v), pack(o), lse.permute(1, 0, 2).reshape(
        H, B * N).contiguous(), pack(do), [0, N, 2 * N, 3 * N], N, causal, 0.09)
    for g, w in zip(got, want):
        assert torch.equal(g.view(torch.int16), pack(w).view(torch.int16))


def test_varlen_bwd_malformed_offsets_stay_in_bounds():
    """Offsets out of order and past total (the caller's contract broken):
    bounds are clamped, so the call completes inside the tensors and the
    workspace, and the rows only the first sequence covers are finite."""
    q, k, v = packed(1, 200, 64, "f16", seed=4)
    do = upstream(q, seed=5)
    o, lse = oracle_fwd_given(q, k, v, [0, 150], False, 0.125)
    o[:, 150:] = 0.0
    lse[:, 150:] = 0.0
    got = gpu_varlen_bwd(q, k, v, o, lse, do, [0, 150, 90, 5000], 200, False, 0.125)
    for g in got:
        assert torch.isfinite(g[:, :90]).all()


def test_varlen_bwd_benchmarked_launch():
    """The benchmarked launch (32 heads, 8 seeded lengths in [512, 8192], d128
    bf16 causal): every dq/dk/dv element of sampled rows of every sequence,
    key rows from two heads per sequence."""
    cu, q, k, v, scale, ro, rl = benchmarked_launch()
    note(f"[varlen bwd parity] benchmarked launch cu={cu}")
    do = upstream(q, seed=12345)
    o, lse = rounded_given(ro, rl, q.dtype, cu)
    got = gpu_varlen_bwd(q, k, v, o, lse, do, cu, max(np.diff(cu)), True, scale)
    H, _, d = q.shape
    rng = np.random.default_rng(3)
    for lo, hi in zip(cu[:-1], cu[1:]):
        L = hi - lo
        qrows = np.unique(np.concatenate([rng.integers(0, H * L, 12), [0, L - 1, H * L - 1]]))
        heads = rng.choice(H, size=2, replace=False)
        krows = np.unique(np.concatenate([h * L + rng.integers(0, L, 4) for h in heads] +
                                         [[heads[0] * L, heads[0] * L + L - 1]]))
        sl = lambda t: np.ascontiguousarray(bits(t)[:, lo:hi, :][None])
        rq, rk, rv = oracle.attn_bwd_rows(sl(q), sl(k), sl(v), sl(do), "bf16", True, scale,
                                          qrows, krows, o=sl(o))
        flat = lambda t: t[:, lo:hi, :].reshape(-1, d)
        rep = compare_grads((flat(got[0])[torch.from_numpy(qrows)],
                             flat(got[1])[torch.from_numpy(krows)],
                             flat(got[2])[torch.from_numpy(krows)]), (rq, rk, rv), "bf16")
        assert rep["ok"], (lo, hi, rep)
