"""fa_fwd_split_noalloc (the split forward pass with its partials in a static
per-device scratch array instead of a caller workspace) against
fa_fwd_split on the same inputs: two calls in a row, the second smaller, each
bit-identical to the workspace entry point, plus the oracle check of the
forward tolerances and the refusal of a problem larger than the scratch."""
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


def _dt(q):
    return fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16


def _both(q, k, v, causal, scale, splits, stream):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = q.shape
    outs = []
    for noalloc in (False, True):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
        if noalloc:
            st = fa.fa_fwd_split_noalloc(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale,
                                         splits, _dt(q), stream)
        else:
            ws = torch.full((fa.fa_fwd_split_workspace_size(B, H, N, d, splits) // 4,),
                            float("nan"), dtype=torch.float32, device=dev)
            st = fa.fa_fwd_split(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale, splits,
                                 ws, _dt(q), stream)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        stream.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    return outs


def test_noalloc_matches_split_twice_second_smaller():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()
    dev = torch.device("cuda", 0)
    cases = [  # B, H, N, d, dtype, causal, splits, stream
        (2, 4, 2000, 128, "bf16", True, 5, torch.cuda.current_stream(dev)),
        (1, 2, 300, 64, "f16", False, 3, torch.cuda.Stream(dev)),
    ]
    for B, H, N, d, dtype, causal, splits, stream in cases:
        need = fa.fa_fwd_split_workspace_size(B, H, N, d, splits)
        assert 0 < need <= fa.FA_NOALLOC_SCRATCH_BYTES
        note(f"[noalloc] B={B} H={H} N={N} d={d} {dtype} causal={causal} splits={splits} "
             f"partials={need} bytes")
        q, k, v = make_qkv(B, H, N, d, dtype, seed=N + splits)
        scale = float(np.float32(1 / math.sqrt(d)))
        (o1, l1), (o2, l2) = _both(q, k, v, causal, scale, splits, stream)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
        ro, rl = oracle.attn_fwd(bits(q), bits(k), bits(v), dtype, causal, scale)
        assert_parity(compare(o2, l2, ro, rl, dtype))


def test_noalloc_refuses_more_than_the_scratch():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda", 0)
    B, H, N, d, splits = 1, 8, 8192, 128, 2
    assert fa.fa_fwd_split_workspace_size(B, H, N, d, splits) > fa.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=dev)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    st = fa.fa_fwd_split_noalloc(q, q, q, o, lse, B, H, N, d, 0, 0.125, splits,
                                 fa.FA_DTYPE_BF16, torch.cuda.current_stream(dev))
    assert st == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(lse).all()
