"""GPU parity of the packed variable-length forward pass (fa_fwd_varlen,
called through the C ABI) against the oracle (plain attention on every
sequence slice), with the forward tolerances: max abs 2e-3 (fp16 o) /
1e-2 (bf16 o), 1e-3 (lse), strict or floor-aware as for the other forward
tests.  Rows of tokens outside every sequence must stay untouched (NaN
sentinels), and a batch of equal lengths must reproduce fa_fwd bit for bit."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import assert_parity, compare, note

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


def test_varlen_benchmarked_launch():
    """The launch bench.py times: 8 sequences of seeded lengths in [512, 8192]
    (24 900 tokens), 32 heads, d128 bf16 causal, every row compared."""
    from io_aware_transformer_amd.inputs import varlen_offsets
    cu = varlen_offsets(8, 512, 8192, seed=0)
    note(f"[varlen parity] benchmarked launch cu={cu}")
    q, k, v = packed(32, cu[-1], 128, "bf16", seed=0)
    check(q, k, v, cu, True, float(np.float32(128 ** -0.5)))
