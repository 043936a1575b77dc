"""GPU parity of the windowed / length-masked forward pass (fa_fwd_window,
called through the C ABI) against the fp64 oracle's masked attention.

Rows with keys: the forward tolerances (max abs 2e-3 fp16 / 1e-2 bf16 on o,
1e-3 on lse), strict first.  Each o element is also allowed its own rounding
floor |rnd(o) - o| in two cases only: where the exact result rounded to the
output type already misses the tolerance somewhere (as in the unmasked
tests), and where every row sees at most two keys, whose two comparable
weights' 16-bit rounding does not average out, so the error approaches two
roundings.  Rows without keys (i >= L_b): o exactly 0 and lse exactly -inf."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import compare, gpu_forward, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def gpu_forward_window(q, k, v, wl, wr, lens, scale):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd_window(qd, kd, vd, o, lse, B, H, N, d, wl, wr, ld, scale, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


def check(q, k, v, wl, wr, lens, scale):
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    o, lse = gpu_forward_window(q, k, v, wl, wr, lens, scale)
    ro, rl = oracle.attn_fwd_masked(bits(q), bits(k), bits(v), dt, wl, wr, lens,
                                    float(np.float32(scale)))
    empty = np.isneginf(rl)
    og, lg = o.double().numpy(), lse.double().numpy()
    # rows without keys: exact zeros and -inf
    assert np.all(og[empty] == 0.0) and np.all(np.isneginf(lg[empty]))
    full = ~empty
    if full.any():
        rep = compare(o[torch.from_numpy(full)], lse[torch.from_numpy(full)], ro[full], rl[full], dt)
        assert rep["finite"], rep
        if not rep["strict_ok"]:
            two_keys = wl >= 0 and wr >= 0 and wl + wr + 1 <= 2
            assert rep["floor_ok"] and (rep["n_floor_over_tol"] > 0 or two_keys), rep
        return rep
    return None


WINDOWS = [(0, 0), (1, 0), (31, 0), (64, 0), (100, 0), (255, 0), (17, 23), (-1, 5), (5, -1),
           (128, 128)]


@pytest.mark.parametrize("wl,wr", WINDOWS)
@pytest.mark.parametrize("N", [1, 65, 300, 1000])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
def test_window_sweep(wl, wr, N, d, dtype):
    note(f"[mask parity] window ({wl},{wr}) N={N} d={d} {dtype}")
    q, k, v = make_qkv(1, 2, N, d, dtype, seed=N + wl * 3 + wr)
    check(q, k, v, wl, wr, None, float(np.float32(1 / math.sqrt(d))))


LENGTHS = [[300, 150, 0], [1, 299, 37], [300, 300, 300], [0, 0, 0], [256, 257, 255]]


@pytest.mark.parametrize("lens", LENGTHS)
@pytest.mark.parametrize("wl,wr", [(-1, -1), (-1, 0), (40, 0), (9, 70)])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "f16")])
def test_lengths(lens, wl, wr, d, dtype):
    note(f"[mask parity] lengths {lens} window ({wl},{wr}) d={d} {dtype}")
    q, k, v = make_qkv(3, 2, 300, d, dtype, seed=sum(lens) + d)
    check(q, k, v, wl, wr, lens, 0.1)


@pytest.mark.parametrize("causal", [False, True])
def test_no_window_matches_fa_fwd_bitwise(causal):
    note(f"[mask parity] (-1,{0 if causal else -1}) equals fa_fwd causal={causal}")
    q, k, v = make_qkv(2, 3, 333, 128, "bf16", seed=71)
    o1, l1 = gpu_forward_window(q, k, v, -1, 0 if causal else -1, None, 0.09)
    o2, l2 = gpu_forward(q, k, v, causal, 0.09)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_full_lengths_match_no_lengths():
    """seqlens all N takes the general kernel; it must agree with the tuned
    causal kernel to the tolerance (different instruction order, same math)."""
    note("[mask parity] lengths = N vs none")
    q, k, v = make_qkv(2, 2, 400, 64, "f16", seed=72)
    o1, l1 = gpu_forward_window(q, k, v, -1, 0, [400, 400], 0.125)
    o2, l2 = gpu_forward(q, k, v, True, 0.125)
    assert (o1.double() - o2.double()).abs().max().item() <= 2e-3
    assert (l1.double() - l2.double()).abs().max().item() <= 1e-3


def test_large_sliding_window():
    """N = 8192, 32 heads, causal window of 1024 keys (bf16, Q,K x3)."""
    note("[mask parity] N=8192 window (1023, 0)")
    q, k, v = make_qkv(1, 32, 8192, 128, "bf16", seed=0, qk_gain=3.0)
    rep = check(q, k, v, 1023, 0, None, float(np.float32(1 / math.sqrt(128))))
    print(rep)
