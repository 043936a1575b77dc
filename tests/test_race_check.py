"""LDS race check: the forward kernels built with every LDS byte poisoned to a
NaN pattern at kernel start, and built with each tile's loads serialised
behind all reads of the previous tile (no load in flight during any read),
must reproduce the product library's outputs bit for bit on every forward
entry point.  A read that overtook its tile load would see the poison (or,
serialised, different data); a tile refilled while still being read would
differ from the serial build.  The debug libraries are built from the same
source by io_aware_transformer_amd.build.build_debug (part of build())."""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import io_aware_transformer_amd as fa
from io_aware_transformer_amd.build import DEBUG_LIBS
from io_aware_transformer_amd.inputs import make_qkv
from tests.parity_util import note

pytestmark = pytest.mark.gpu


def _bind(path):
    assert path.exists(), f"{path.name} missing: run io_aware_transformer_amd.build.build_debug()"
    lib = ctypes.CDLL(str(path))
    p, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    u64, u32 = ctypes.c_ulonglong, ctypes.c_uint
    lib.fa_fwd.argtypes = [p, p, p, p, p, i, i, i, i, i, f, i, p]
    lib.fa_fwd_split.argtypes = [p, p, p, p, p, i, i, i, i, i, f, i, p, i, p]
    lib.fa_fwd_window.argtypes = [p, p, p, p, p, i, i, i, i, i, i, p, f, i, p]
    lib.fa_fwd_varlen.argtypes = [p, p, p, p, p, p, i, i, i, i, i, i, f, i, p]
    lib.fa_fwd_dropout.argtypes = [p, p, p, p, p, i, i, i, i, i, f, f, u64, u32, i, p]
    lib.fa_fwd_decode.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, i, p, i, p]
    for n in ("fa_fwd", "fa_fwd_split", "fa_fwd_window", "fa_fwd_varlen", "fa_fwd_dropout",
              "fa_fwd_decode"):
        getattr(lib, n).restype = ctypes.c_int
    return lib


@pytest.fixture(scope="module")
def libs():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()
    return {"product": fa.load(), **{k: _bind(v[0]) for k, v in DEBUG_LIBS.items()}}


def _run(lib, call, shapes):
    """call(lib, outs) with NaN-filled outputs of the given shapes/dtypes."""
    dev = torch.device("cuda", 0)
    outs = [torch.full(s, float("nan"), dtype=dt, device=dev) for s, dt in shapes]
    st = call(lib, outs)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return [o.cpu() for o in outs]


def _same(results):
    ref = results["product"]
    for name, outs in results.items():
        for a, b in zip(ref, outs):
            assert not torch.isnan(b.float()).any(), name   # -inf lse: rows without keys
            ia = a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32)
            ib = b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int32)
            assert torch.equal(ia, ib), name


def _ptr(t):
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream(torch.device("cuda", 0)).cuda_stream


CASES = [(1, 3, 1000, 128, "bf16", 1), (2, 2, 700, 64, "f16", 0), (1, 2, 129, 128, "f16", 1),
         (1, 4, 4096, 128, "bf16", 1), (1, 1, 1, 64, "bf16", 1), (2, 3, 65, 128, "bf16", 0),
         (1, 2, 3000, 64, "f16", 1)]


@pytest.mark.parametrize("B,H,N,d,dtype,causal", CASES)
def test_forward_matches_race_check_builds(libs, B, H, N, d, dtype, causal):
    note(f"[race check] fa_fwd B{B} H{H} N{N} d{d} {dtype} causal{causal}")
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dtype, seed=N + d, qk_gain=2.0))
    dt = fa.FA_DTYPE_F16 if dtype == "f16" else fa.FA_DTYPE_BF16
    shapes = [((B, H, N, d), q.dtype), ((B, H, N), torch.float32)]
    scale = 1 / math.sqrt(d)

    def call(lib, outs):
        return lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(outs[0]), _ptr(outs[1]), B, H, N, d,
                          causal, scale, dt, _stream())

    _same({n: _run(lib, call, shapes) for n, lib in libs.items()})


def test_other_forward_entry_points_match_race_check_builds(libs):
    dev = torch.device("cuda", 0)
    B, H, N, d = 2, 3, 1500, 128
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, "bf16", seed=3))
    bf = fa.FA_DTYPE_BF16
    shapes = [((B, H, N, d), q.dtype), ((B, H, N), torch.float32)]
    ws = torch.empty(fa.fa_fwd_split_workspace_size(B, H, N, d, 3) // 4, device=dev)
    lens = torch.tensor([1500, 777], dtype=torch.int32, device=dev)

    note("[race check] fa_fwd_split")
    _same({n: _run(lib, lambda L, o: L.fa_fwd_split(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o[0]), _ptr(o[1]), B, H, N, d, 1, 0.09, 3, _ptr(ws), bf,
        _stream()), shapes) for n, lib in libs.items()})
    note("[race check] fa_fwd_window")
    _same({n: _run(lib, lambda L, o: L.fa_fwd_window(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o[0]), _ptr(o[1]), B, H, N, d, 300, 40, _ptr(lens), 0.09,
        bf, _stream()), shapes) for n, lib in libs.items()})
    note("[race check] fa_fwd_dropout")
    _same({n: _run(lib, lambda L, o: L.fa_fwd_dropout(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o[0]), _ptr(o[1]), B, H, N, d, 1, 0.09, 0.1, 1234, 7, bf,
        _stream()), shapes) for n, lib in libs.items()})

    note("[race check] fa_fwd_varlen")
    cu = torch.tensor([0, 700, 701, 2000, 3000], dtype=torch.int32, device=dev)
    Hv, total = 3, 3000
    qv, kv, vv = (t.cuda() for t in make_qkv(1, Hv, total, 64, "f16", seed=4))
    _same({n: _run(lib, lambda L, o: L.fa_fwd_varlen(
        _ptr(qv), _ptr(kv), _ptr(vv), _ptr(o[0]), _ptr(o[1]), _ptr(cu), 4, Hv, total, 1300, 64, 1,
        0.125, fa.FA_DTYPE_F16, _stream()), [((1, Hv, total, 64), qv.dtype),
                                              ((1, Hv, total), torch.float32)])
           for n, lib in libs.items()})

    note("[race check] fa_fwd_decode")
    qd = make_qkv(1, 8, 5, 128, "bf16", seed=5)[0].cuda()
    _, kd, vd = (t.cuda() for t in make_qkv(1, 8, 20000, 128, "bf16", seed=6))
    wsd = torch.empty(fa.fa_fwd_decode_workspace_size(1, 8, 5, 20000, 128, 0) // 4, device=dev)
    _same({n: _run(lib, lambda L, o: L.fa_fwd_decode(
        _ptr(qd), _ptr(kd), _ptr(vd), _ptr(o[0]), _ptr(o[1]), 1, 8, 5, 20000, 128, 1, 0.09, 0,
        _ptr(wsd), bf, _stream()), [((1, 8, 5, 128), qd.dtype), ((1, 8, 5), torch.float32)])
           for n, lib in libs.items()})
