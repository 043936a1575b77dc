"""GPU parity of the windowed / length-masked backward pass (fa_bwd_window,
called through the C ABI) against the oracle's masked gradients
(oracle.attn_bwd_masked).

fa_bwd_window is handed the forward results the boundary specifies, made by
the oracle's masked forward: o rounded to the 16-bit type and lse to fp32
(rows without keys: o = 0, lse = -inf).  The reference takes its row term
from the same o.  Tolerance: the normalised backward one, max |g - g_ref| /
max(max |g_ref|, 1e-3) per gradient.  Padded rows and keys must get exactly
zero.  Windows (-1,-1) and (-1,0) without lengths must reproduce fa_bwd bit
for bit, and a window side of N or more must equal an open side bit for
bit."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import compare_grads, gpu_backward_given, note

pytestmark = pytest.mark.gpu

INT_MAX = 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def dname(t):
    return "f16" if t.dtype == torch.float16 else "bf16"


def oracle_given(q, k, v, wl, wr, lens, scale):
    ro, rl = oracle.attn_fwd_masked(bits(q), bits(k), bits(v), dname(q), wl, wr, lens,
                                    float(np.float32(scale)))
    return torch.from_numpy(ro).to(q.dtype), torch.from_numpy(rl).to(torch.float32)


def gpu_bwd_window(q, k, v, o, lse, do, wl, wr, lens, scale):
    """fa_bwd_window on cuda:0 with NaN-filled outputs and workspace."""
    dev = torch.device("cuda", 0)
    qd, kd, vd, od, dod = (t.to(dev).contiguous() for t in (q, k, v, o, do))
    ld = lse.to(dev).contiguous()
    B, H, N, d = q.shape
    lens_d = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.full((fa.fa_bwd_workspace_size(B, H, N) // 4,), float("nan"),
                    dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.full_like(qd, float("nan")) for _ in range(3))
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_bwd_window(qd, kd, vd, od, dod, ld, ws, dq, dk, dv, B, H, N, d, wl, wr, lens_d,
                          scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(q, k, v, do, wl, wr, lens, scale):
    o, lse = oracle_given(q, k, v, wl, wr, lens, scale)
    got = gpu_bwd_window(q, k, v, o, lse, do, wl, wr, lens, scale)
    ref = oracle.attn_bwd_masked(bits(q), bits(k), bits(v), bits(do), dname(q), wl, wr, lens,
                                 float(np.float32(scale)), o=bits(o))
    if lens is not None:
        for b, L in enumerate(lens):
            for g in got:
                assert torch.count_nonzero(g[b, :, L:]) == 0
    rep = compare_grads(got, ref, dname(q))
    assert rep["ok"], rep
    return rep


def inputs(B, H, N, d, dtype, seed, gain=1.0):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed, qk_gain=gain)
    do = make_qkv(B, H, N, d, dtype, seed=seed + 7919)[0]
    return q, k, v, do


WINDOWS = [(0, 0), (1, 0), (31, 0), (64, 0), (100, 0), (255, 0), (17, 23), (-1, 5), (5, -1),
           (128, 128)]


@pytest.mark.parametrize("wl,wr", WINDOWS)
@pytest.mark.parametrize("N", [1, 65, 300, 700])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
def test_window_bwd_sweep(wl, wr, N, d, dtype):
    note(f"[window bwd parity] ({wl},{wr}) N={N} d={d} {dtype}")
    q, k, v, do = inputs(1, 2, N, d, dtype, seed=N + 3 * wl + wr + 5)
    check(q, k, v, do, wl, wr, None, float(np.float32(1 / math.sqrt(d))))


LENGTHS = [[300, 150, 0], [1, 299, 37], [300, 300, 300], [0, 0, 0], [256, 257, 255]]


@pytest.mark.parametrize("lens", LENGTHS)
@pytest.mark.parametrize("wl,wr", [(-1, -1), (-1, 0), (40, 0), (9, 70)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_window_bwd_lengths(lens, wl, wr, d, dtype):
    note(f"[window bwd parity] lengths {lens} ({wl},{wr}) d={d} {dtype}")
    q, k, v, do = inputs(3, 2, 300, d, dtype, seed=sum(lens) + d + 1)
    check(q, k, v, do, wl, wr, lens, 0.1)


@pytest.mark.parametrize("causal", [False, True])
def test_no_window_matches_fa_bwd_bitwise(causal):
    note(f"[window bwd parity] (-1,{0 if causal else -1}) equals fa_bwd causal={causal}")
    q, k, v, do = inputs(2, 3, 333, 128, "bf16", seed=73)
    wr = 0 if causal else -1
    o, lse = oracle_given(q, k, v, -1, wr, None, 0.09)
    a = gpu_bwd_window(q, k, v, o, lse, do, -1, wr, None, 0.09)
    b = gpu_backward_given(q, k, v, o, lse, do, causal, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_huge_sides_equal_open_sides():
    """Sides of N or more allow every key on that side: INT_MAX must give the
    bits of -1, in the backward and the forward (both with lengths, so the
    forward takes its general kernel either way)."""
    note("[window bwd parity] sides INT_MAX vs -1")
    q, k, v, do = inputs(2, 2, 200, 64, "f16", seed=74)
    lens = [200, 131]
    o, lse = oracle_given(q, k, v, -1, 0, lens, 0.125)
    a = gpu_bwd_window(q, k, v, o, lse, do, INT_MAX, 0, lens, 0.125)
    b = gpu_bwd_window(q, k, v, o, lse, do, -1, 0, lens, 0.125)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    dev = torch.device("cuda", 0)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    outs = []
    for wl, wr in ((INT_MAX, INT_MAX), (-1, -1)):
        of = torch.empty_like(q.to(dev))
        lf = torch.empty((2, 2, 200), dtype=torch.float32, device=dev)
        st = fa.fa_fwd_window(q.to(dev), k.to(dev), v.to(dev), of, lf, 2, 2, 200, 64, wl, wr, ld,
                              0.125, fa.FA_DTYPE_F16, torch.cuda.current_stream(dev))
        assert st == fa.FA_OK
        torch.cuda.synchronize()
        outs.append((of.cpu(), lf.cpu()))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


def test_window_bwd_benchmarked_launch():
    """The window launch bench.py times: B1 H32 N8192 d128 bf16, Q,K x3, each
    query sees the 1024 keys ending at itself.  Every gradient element of
    two heads against the oracle on those heads (heads are independent)."""
    note("[window bwd parity] N=8192 H=32 window (1023, 0)")
    q, k, v, do = inputs(1, 32, 8192, 128, "bf16", seed=0, gain=3.0)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, lse = oracle_given(q, k, v, 1023, 0, None, scale)
    got = gpu_bwd_window(q, k, v, o, lse, do, 1023, 0, None, scale)
    for h in (0, 17):
        sl = lambda t: t[:, h:h + 1].contiguous()
        ref = oracle.attn_bwd_masked(bits(sl(q)), bits(sl(k)), bits(sl(v)), bits(sl(do)), "bf16",
                                     1023, 0, None, scale, o=bits(sl(o)))
        rep = compare_grads(tuple(sl(g) for g in got), ref, "bf16")
        print(h, rep)
        assert rep["ok"], (h, rep)
