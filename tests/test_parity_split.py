"""GPU parity of the split-key forward pass (fa_fwd_split: key segments in
separate work-groups, merged per row) against the fp64 oracle's plain
attention -- the same function fa_fwd computes -- under the forward
tolerances."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import assert_parity, compare, gpu_forward, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def gpu_forward_split(q, k, v, causal, scale, num_splits):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.full((fa.fa_fwd_split_workspace_size(B, H, N, d, num_splits) // 4,),
                    float("nan"), dtype=torch.float32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd_split(qd, kd, vd, o, lse, B, H, N, d, int(causal), scale, num_splits, ws,
                         dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("N", [1, 100, 128, 129, 300, 1000])
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_split_sweep(N, splits, d, dtype, causal):
    note(f"[split parity] N={N} splits={splits} d={d} {dtype} causal={causal}")
    q, k, v = make_qkv(1, 2, N, d, dtype, seed=N + splits)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = gpu_forward_split(q, k, v, causal, scale, splits)
    ro, rl = oracle.attn_fwd(bits(q), bits(k), bits(v), dtype, causal, scale)
    assert_parity(compare(o, lse, ro, rl, dtype))


@pytest.mark.parametrize("causal", [False, True])
def test_split_few_heads_long(causal):
    """B=1, H=4, N=4096, d=128 bf16: 64 work-groups without splitting."""
    note(f"[split parity] few heads causal={causal}")
    q, k, v = make_qkv(1, 4, 4096, 128, "bf16", seed=81)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, lse = gpu_forward_split(q, k, v, causal, scale, 8)
    ro, rl = oracle.attn_fwd(bits(q), bits(k), bits(v), "bf16", causal, scale)
    rep = compare(o, lse, ro, rl, "bf16")
    print(rep)
    assert_parity(rep)
    o2, l2 = gpu_forward(q, k, v, causal, scale)
    assert (o.double() - o2.double()).abs().max().item() <= 2e-2
    assert (lse.double() - l2.double()).abs().max().item() <= 1e-3


def test_split_peaky_and_scales():
    note("[split parity] peaky / scale values")
    q, k, v = make_qkv(2, 2, 700, 64, "bf16", seed=82, qk_gain=3.0)
    for scale in (0.0, -0.125, 0.125):
        for causal in (False, True):
            o, lse = gpu_forward_split(q, k, v, causal, scale, 3)
            ro, rl = oracle.attn_fwd(bits(q), bits(k), bits(v), "bf16", causal, scale)
            assert_parity(compare(o, lse, ro, rl, "bf16"))
