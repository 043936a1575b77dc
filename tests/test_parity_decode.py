"""GPU parity of fa_fwd_decode (Nq query rows against Nk keys, causal aligned
bottom-right, split over key segments and merged per row) against the fp64
oracle's attn_fwd_decode under the forward tolerances, through the C ABI."""
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


def decode_inputs(B, H, Nq, Nk, d, dtype, seed, gain=1.0):
    q = make_qkv(B, H, Nq, d, dtype, seed=seed, qk_gain=gain)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed=seed + 1, qk_gain=gain)
    return q, k, v


def gpu_decode(q, k, v, causal, scale, num_splits, stream=None):
    dev = torch.device("cuda", 0)
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    wsb = fa.fa_fwd_decode_workspace_size(B, H, Nq, Nk, d, num_splits)
    assert wsb > 0
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device=dev)
    dt = fa.FA_DTYPE_F16 if q.dtype == torch.float16 else fa.FA_DTYPE_BF16
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = fa.fa_fwd_decode(qd, kd, vd, o, lse, B, H, Nq, Nk, d, int(causal), scale, num_splits,
                          ws, dt, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    stream.synchronize()
    return o.cpu(), lse.cpu()


def check(q, k, v, causal, scale, num_splits, dtype):
    o, lse = gpu_decode(q, k, v, causal, scale, num_splits)
    ro, rl = oracle.attn_fwd_decode(bits(q), bits(k), bits(v), dtype, causal, scale)
    rep = compare(o, lse, ro, rl, dtype)
    assert_parity(rep)
    return o, lse, rep


# Nq <= 32 runs two waves per key segment (each half of every key tile is a
# segment of its own), Nq = 33 the one-wave-per-row-slab path
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 129), (3, 1000), (16, 4097), (32, 1100),
                                   (33, 1100), (64, 300), (100, 100), (257, 700), (300, 5000)])
@pytest.mark.parametrize("splits", [0, 1, 3, 64])
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_sweep(Nq, Nk, splits, d, dtype, causal):
    note(f"[decode parity] Nq={Nq} Nk={Nk} splits={splits} d={d} {dtype} causal={causal}")
    q, k, v = decode_inputs(2, 3, Nq, Nk, d, dtype, seed=Nq * 31 + Nk + splits)
    scale = float(np.float32(1 / math.sqrt(d)))
    check(q, k, v, causal, scale, splits, dtype)


@pytest.mark.parametrize("Nk", [32768, 131072])
@pytest.mark.parametrize("Nq", [1, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_decode_long_keys(Nk, Nq, causal):
    """Few query rows against 32K and 128K keys, d128 bf16, 32 heads, the
    library's split count."""
    note(f"[decode parity] long Nk={Nk} Nq={Nq} causal={causal}")
    q, k, v = decode_inputs(1, 32, Nq, Nk, 128, "bf16", seed=Nk + Nq)
    scale = float(np.float32(1 / math.sqrt(128)))
    _, _, rep = check(q, k, v, causal, scale, 0, "bf16")
    print(rep)


def test_decode_long_keys_d64_peaky():
    note("[decode parity] Nk=65536 d64 f16 peaky")
    q, k, v = decode_inputs(2, 4, 8, 65536, 64, "f16", seed=77, gain=3.0)
    _, _, rep = check(q, k, v, True, 0.125, 0, "f16")
    print(rep)


def test_decode_largest_key_count():
    """Nk = FA_MAX_N keys (one head of K fills 2^29 bytes at d = 64)."""
    Nk = 1 << 22
    note(f"[decode parity] Nk={Nk} (largest) d64 f16")
    q, k, v = decode_inputs(1, 1, 2, Nk, 64, "f16", seed=5)
    for splits in (0, 64):
        _, _, rep = check(q, k, v, True, 0.125, splits, "f16")
        print(rep)


def test_decode_square_matches_fa_fwd_definition():
    """Nq = Nk: the square causal mask of fa_fwd (checked against the plain
    oracle, which the decoding oracle reduces to there)."""
    note("[decode parity] square")
    q, k, v = decode_inputs(1, 4, 777, 777, 128, "bf16", seed=9)
    o, lse = gpu_decode(q, k, v, True, 0.09, 0)
    ro, rl = oracle.attn_fwd(bits(q), bits(k), bits(v), "bf16", True, 0.09)
    assert_parity(compare(o, lse, ro, rl, "bf16"))


@pytest.mark.parametrize("causal", [False, True])
def test_decode_closed_forms_long(causal):
    """Q = 0 at Nk = 40000: lse = ln |A_i| and o = mean of the allowed V rows;
    constant V rows give that constant."""
    Nq, Nk = 5, 40000
    note(f"[decode parity] closed forms causal={causal}")
    q, k, v = decode_inputs(1, 2, Nq, Nk, 128, "bf16", seed=13)
    o, lse = gpu_decode(torch.zeros_like(q), k, v, causal, 0.3, 0)
    vv = v.double().numpy()
    for i in range(Nq):
        n = (i + Nk - Nq + 1) if causal else Nk
        assert np.abs(lse[:, :, i].double().numpy() - math.log(n)).max() <= 1e-3
        mean = vv[:, :, :n].mean(axis=2)
        assert np.abs(o[:, :, i].double().numpy() - mean).max() <= 1e-2
    cv = torch.full_like(v, -2.75)
    o, _ = gpu_decode(q, k, cv, causal, 0.3, 0)
    assert torch.all(o.double() == -2.75)


def test_decode_hygiene():
    """Bitwise-identical reruns (and on another stream), every output written."""
    note("[decode parity] hygiene")
    q, k, v = decode_inputs(2, 8, 7, 9000, 128, "bf16", seed=21)
    a = gpu_decode(q, k, v, True, 0.1, 0)
    b = gpu_decode(q, k, v, True, 0.1, 0)
    c = gpu_decode(q, k, v, True, 0.1, 0, stream=torch.cuda.Stream(torch.device("cuda", 0)))
    for x in (b, c):
        assert torch.equal(a[0].view(torch.int16), x[0].view(torch.int16))
        assert torch.equal(a[1].view(torch.int32), x[1].view(torch.int32))
    assert torch.isfinite(a[0].float()).all() and torch.isfinite(a[1]).all()


def test_decode_more_queries_than_keys():
    """Without the causal flag Nq may exceed Nk."""
    note("[decode parity] Nq=300 > Nk=129 non-causal")
    q, k, v = decode_inputs(1, 3, 300, 129, 128, "bf16", seed=31)
    check(q, k, v, False, 0.0884, 0, "bf16")
    check(q, k, v, False, 0.0884, 2, "bf16")
