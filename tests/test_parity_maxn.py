"""GPU parity at the largest sequence length the boundary accepts,
FA_MAX_N = 2^22 rows per head, where one head of K or V at d = 128 fills
2^30 bytes of a buffer descriptor's 32-bit range.

Forward: every element of sampled query rows (the first, the last and
seeded others) against the oracle's attention on those rows, with the
forward tolerances.

Backward: with q = 0 every score is 0, so under the causal mask the weights
are uniform, P_ij = 1/(i+1).  Then o_i is the mean of v_0..v_i and
lse_i = ln(i+1) (computed here in fp64, o rounded to the 16-bit type once,
lse to fp32), and the gradients of the definition have closed forms that
cost O(N d^2):
    dV_j = sum_{i >= j} dO_i / (i+1)
    dK_j = scale * sum_i dS_ij q_i = 0                        (exactly)
    dQ_i = scale / (i+1) * [ (sum_{j<=i} k_j v_j^T) dO_i - D_i sum_{j<=i} k_j ],
           D_i = dO_i . o_i
dV and dQ are compared on sampled rows with the normalised backward
tolerance; dK must be exactly zero everywhere."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
import oracle
from io_aware_transformer_amd.inputs import bits, make_qkv
from tests.parity_util import (assert_parity, compare, compare_grads, gpu_backward_given,
                               gpu_forward, note)

pytestmark = pytest.mark.gpu

MAX_N = 1 << 22


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n - 1], rng.integers(0, n, count)]))


@pytest.mark.parametrize("d,dtype,causal", [(128, "bf16", True), (64, "f16", False)])
def test_forward_at_max_n(d, dtype, causal):
    note(f"[max-N parity] forward N={MAX_N} d={d} {dtype} causal={causal}")
    q, k, v = make_qkv(1, 1, MAX_N, d, dtype, seed=5)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = gpu_forward(q, k, v, causal, scale)
    rows = sample_rows(MAX_N, 6, seed=d)
    ro, rl = oracle.attn_fwd_rows(bits(q), bits(k), bits(v), dtype, causal, scale, rows)
    idx = torch.from_numpy(rows)
    rep = compare(o.reshape(-1, d)[idx], lse.reshape(-1)[idx], ro, rl, dtype)
    print(rep)
    assert_parity(rep)


def test_backward_at_max_n_uniform_weights():
    N, d, dtype = MAX_N, 64, "f16"
    note(f"[max-N parity] backward N={N} d={d} {dtype} causal, q = 0")
    _, k, v = make_qkv(1, 1, N, d, dtype, seed=6)
    do = make_qkv(1, 1, N, d, dtype, seed=7)[0]
    q = torch.zeros_like(k)
    scale = 0.125
    cnt = torch.arange(1, N + 1, dtype=torch.float64)
    # o_i = mean of v_0..v_i, lse_i = ln(i+1)
    o64 = torch.cumsum(v[0, 0].double(), dim=0) / cnt[:, None]
    o = o64.to(torch.float16)[None, None]
    lse = torch.log(cnt).to(torch.float32)[None, None]
    del o64
    got = gpu_backward_given(q, k, v, o, lse, do, True, scale)
    assert torch.count_nonzero(got[1]) == 0          # dK = 0 exactly

    k64, v64, do64 = (t[0, 0].double() for t in (k, v, do))
    o16 = o[0, 0].double()
    # dV on sampled key rows: suffix sums of dO_i / (i+1)
    w = do64 / cnt[:, None]
    suffix = torch.flip(torch.cumsum(torch.flip(w, [0]), dim=0), [0])
    del w
    krows = sample_rows(N, 6, seed=11)
    ref_dv = suffix[torch.from_numpy(krows)].numpy()
    del suffix
    # dQ on sampled query rows: prefix sums of k_j v_j^T and of k_j
    qrows = sample_rows(N, 6, seed=12)
    ref_dq = np.empty((qrows.size, d))
    kv = torch.zeros((d, d), dtype=torch.float64)
    ks = torch.zeros(d, dtype=torch.float64)
    start = 0
    for t, i in enumerate(qrows):
        kv += k64[start:i + 1].T @ v64[start:i + 1]
        ks += k64[start:i + 1].sum(0)
        start = i + 1
        D = float(do64[i] @ o16[i])
        ref_dq[t] = (scale / (i + 1) * (kv @ do64[i] - D * ks)).numpy()
    gq = got[0].reshape(-1, d)[torch.from_numpy(qrows)]
    gv = got[2].reshape(-1, d)[torch.from_numpy(krows)]
    gk = got[1].reshape(-1, d)[torch.from_numpy(krows)]
    rep = compare_grads((gq, gk, gv), (ref_dq, np.zeros_like(ref_dv), ref_dv), dtype)
    print(rep)
    assert rep["ok"], rep
