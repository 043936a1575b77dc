"""CPU tests of the C-ABI library: it loads, exports every function that
include/*.h declares, and rejects bad arguments on the host, before any
HIP call (so these run without a GPU).  No compute call is made here."""
from __future__ import annotations

import math
import re
import subprocess

import pytest

import io_aware_transformer_amd as fa
from tests.conftest import ROOT

HEADERS = sorted((ROOT / "include").glob("*.h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", h.read_text(), flags=re.S)
        names |= set(re.findall(r"\b(fa_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    fa.load()
    out = subprocess.run(["nm", "-D", "--defined-only", str(fa.library_path())],
                         check=True, capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings_cover_every_code():
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED,
                 fa.FA_ERR_MISALIGNED, fa.FA_ERR_LAUNCH, fa.FA_ERR_SCRATCH):
        s = fa.fa_status_string(code)
        assert s.startswith(("FA_OK", "FA_ERR_")), s
    assert fa.fa_status_string(7) == "unknown fa_status"


# Fake, well-aligned, non-overlapping device addresses: validation must
# reject the call before anything dereferences them.
Q, K, V, O, L = (0x10000 * (i + 1) for i in range(5))


def call(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=64, d=128, causal=0, scale=0.125,
         dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype, None)


@pytest.mark.parametrize("kw", [dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0)])
def test_null_pointers(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(B=-1), dict(N=-5)])
def test_non_positive_sizes(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("causal", [-1, 2, 7])
def test_causal_flag(causal):
    assert call(causal=causal) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("scale", [math.inf, -math.inf, math.nan])
def test_non_finite_scale(scale):
    assert call(scale=scale) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype", [-1, 2, 99])
def test_unknown_dtype(dtype):
    assert call(dtype=dtype) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [1, 32, 63, 96, 127, 256])
def test_unsupported_head_dim(d):
    assert call(d=d) == fa.FA_ERR_UNSUPPORTED


def test_sequence_too_long():
    assert call(N=(1 << 22) + 1, q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40,
                lse=5 << 40) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(q=Q + 8), dict(k=K + 2), dict(v=V + 4), dict(o=O + 1),
                                dict(lse=L + 2)])
def test_misaligned(kw):
    assert call(**kw) == fa.FA_ERR_MISALIGNED


def test_lse_needs_only_4_byte_alignment():
    # passes validation checks up to the overlap test; with overlapping o it
    # must still be rejected as INVALID, proving alignment was accepted
    assert call(lse=L + 4, o=L) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(o=Q), dict(o=K + 64), dict(lse=V + 128), dict(lse=O)])
def test_overlapping_outputs(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARG


def test_typed_entry_points_validate():
    assert fa.fa_fwd_f16(0, K, V, O, L, 1, 1, 64, 64, 0, 1.0) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fwd_bf16(Q, K, V, O, L, 1, 1, 64, 80, 0, 1.0) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_f16(Q, K, V, O + 2, L, 1, 1, 64, 64, 0, 1.0) == fa.FA_ERR_MISALIGNED


def test_grid_too_large():
    # B*H*ceil(N/128) above INT_MAX is refused on the host
    assert call(B=1 << 16, H=1 << 16, N=1 << 10, q=1 << 44, k=2 << 44, v=3 << 44,
                o=4 << 44, lse=5 << 44) == fa.FA_ERR_INVALID_ARG


# ---------------------------------------------------------------- backward

DO, WS, DQ, DK, DV = (0x10000 * (i + 6) for i in range(5))


def bcall(q=Q, k=K, v=V, o=O, do=DO, lse=L, ws=WS, dq=DQ, dk=DK, dv=DV, B=1, H=1, N=64,
          d=128, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd(q, k, v, o, do, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, dtype,
                     None)


def test_workspace_size():
    # per head: ceil(N/32) blocks of 32 (lse*log2e) + 32 (D) fp32 values
    assert fa.fa_bwd_workspace_size(1, 1, 1) == 256
    assert fa.fa_bwd_workspace_size(2, 3, 33) == 2 * 3 * 2 * 256
    assert fa.fa_bwd_workspace_size(1, 1, 64) == 2 * 256
    assert fa.fa_bwd_workspace_size(0, 1, 64) == 0
    assert fa.fa_bwd_workspace_size(1, 1, -3) == 0


@pytest.mark.parametrize("kw", [dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(do=0),
                                dict(lse=0), dict(ws=0), dict(dq=0), dict(dk=0), dict(dv=0)])
def test_bwd_null_pointers(kw):
    assert bcall(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=-1), dict(causal=2), dict(scale=math.nan),
                                dict(dtype=5)])
def test_bwd_invalid(kw):
    assert bcall(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(d=32), dict(N=(1 << 22) + 1, q=1 << 40,
                                k=2 << 40, v=3 << 40, o=4 << 40, do=5 << 40, lse=6 << 40,
                                ws=7 << 40, dq=8 << 40, dk=9 << 40, dv=10 << 40)])
def test_bwd_unsupported(kw):
    assert bcall(**kw) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(q=Q + 2), dict(do=DO + 8), dict(ws=WS + 4),
                                dict(dq=DQ + 2), dict(dv=DV + 6), dict(lse=L + 1)])
def test_bwd_misaligned(kw):
    assert bcall(**kw) == fa.FA_ERR_MISALIGNED


@pytest.mark.parametrize("kw", [dict(dq=Q), dict(dk=K + 32), dict(dv=DO), dict(ws=L),
                                dict(dq=DK), dict(ws=DV + 16), dict(dk=O + 256)])
def test_bwd_overlaps(kw):
    assert bcall(**kw) == fa.FA_ERR_INVALID_ARG


# ---------------------------------------------------------------- window / lengths

LENS = 0x10000 * 12


def wcall(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=64, d=128, wl=16, wr=0, lens=LENS,
          scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_window(q, k, v, o, lse, B, H, N, d, wl, wr, lens, scale, dtype, None)


@pytest.mark.parametrize("kw", [dict(wl=-2), dict(wr=-5), dict(q=0), dict(B=0),
                                dict(scale=math.inf), dict(dtype=3), dict(o=Q + 256),
                                dict(lse=LENS), dict(o=LENS - 16)])
def test_window_invalid(kw):
    assert wcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_window_unsupported_and_misaligned():
    assert wcall(d=80) == fa.FA_ERR_UNSUPPORTED
    assert wcall(lens=LENS + 2) == fa.FA_ERR_MISALIGNED
    assert wcall(v=V + 8) == fa.FA_ERR_MISALIGNED


# ---------------------------------------------------------------- split keys

SWS = 0x10000 * 13


def scall(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=64, d=128, causal=0, scale=0.125, ns=2,
          ws=SWS, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_split(q, k, v, o, lse, B, H, N, d, causal, scale, ns, ws, dtype, None)


def test_split_workspace_size():
    # segments are whole 128-key tiles: N = 300 in 2 splits -> 256 + 44 keys
    assert fa.fa_fwd_split_workspace_size(1, 2, 300, 64, 2) == 2 * 2 * 300 * 65 * 4
    # more splits than tiles: only non-empty segments are counted
    assert fa.fa_fwd_split_workspace_size(1, 1, 100, 128, 64) == 1 * 100 * 129 * 4
    assert fa.fa_fwd_split_workspace_size(1, 1, 100, 128, 0) == 0
    assert fa.fa_fwd_split_workspace_size(1, 1, 100, 128, fa.FA_MAX_SPLITS + 1) == 0
    assert fa.fa_fwd_split_workspace_size(1, 1, 100, 96, 2) == 0


@pytest.mark.parametrize("kw", [dict(ns=0), dict(ns=65), dict(ws=0), dict(causal=3),
                                dict(q=0), dict(N=0), dict(ws=Q), dict(ws=L - 16)])
def test_split_invalid(kw):
    assert scall(**kw) == fa.FA_ERR_INVALID_ARG


def test_split_unsupported_and_misaligned():
    assert scall(d=32) == fa.FA_ERR_UNSUPPORTED
    assert scall(ws=SWS + 4) == fa.FA_ERR_MISALIGNED
    assert scall(k=K + 2) == fa.FA_ERR_MISALIGNED


def ncall(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=64, d=128, causal=0, scale=0.125, ns=2,
          dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_split_noalloc(q, k, v, o, lse, B, H, N, d, causal, scale, ns, dtype, None)


@pytest.mark.parametrize("kw", [dict(ns=0), dict(ns=65), dict(causal=3), dict(q=0),
                                dict(lse=0), dict(N=0), dict(o=Q), dict(scale=float("nan"))])
def test_split_noalloc_invalid(kw):
    assert ncall(**kw) == fa.FA_ERR_INVALID_ARG


def test_split_noalloc_unsupported_misaligned_and_too_large():
    assert ncall(d=32) == fa.FA_ERR_UNSUPPORTED
    assert ncall(k=K + 2) == fa.FA_ERR_MISALIGNED
    # partials larger than the static scratch: refused before any HIP call
    far = dict(q=1 << 36, k=2 << 36, v=3 << 36, o=4 << 36, lse=5 << 36)
    B, H, N, d, ns = 1, 8, 8192, 128, 2
    assert fa.fa_fwd_split_workspace_size(B, H, N, d, ns) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert ncall(B=B, H=H, N=N, d=d, ns=ns, **far) == fa.FA_ERR_SCRATCH
    # the largest problem of one head and one segment that still fits
    n_fit = fa.FA_NOALLOC_SCRATCH_BYTES // (129 * 4)
    assert fa.fa_fwd_split_workspace_size(1, 1, n_fit, 128, 1) <= fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_fwd_split_workspace_size(1, 1, n_fit + 1, 128, 1) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert ncall(N=n_fit + 1, ns=1, **far) == fa.FA_ERR_SCRATCH


# ---------------------------------------------------------------- decoding

QD, KD, VD, OD, LD, WD = ((1 << 36) * (i + 1) for i in range(6))


def dccall(q=QD, k=KD, v=VD, o=OD, lse=LD, B=1, H=2, Nq=4, Nk=1000, d=128, causal=1,
           scale=0.125, ns=0, ws=WD, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_decode(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, ns, ws, dtype, None)


def test_decode_workspace_size_and_split_rule():
    # segments of whole 128-key tiles: Nk = 1000 in 3 splits -> 384 + 384 + 232;
    # up to 32 query rows each segment holds two halves (two waves' partials)
    assert fa.fa_fwd_decode_workspace_size(1, 2, 4, 1000, 128, 3) == 2 * 3 * 2 * 4 * 129 * 4
    assert fa.fa_fwd_decode_workspace_size(2, 3, 5, 100, 64, 64) == 2 * 1 * 6 * 5 * 65 * 4
    assert fa.fa_fwd_decode_workspace_size(1, 2, 32, 1000, 128, 3) == 2 * 3 * 2 * 32 * 129 * 4
    assert fa.fa_fwd_decode_workspace_size(1, 2, 33, 1000, 128, 3) == 3 * 2 * 33 * 129 * 4
    # num_splits = 0 resolves to the library's rule
    ns = fa.fa_fwd_decode_splits(1, 32, 1, 32768)
    assert ns == 8      # 32 work-groups -> 8 segments of 4096 keys: 256 work-groups
    assert fa.fa_fwd_decode_workspace_size(1, 32, 1, 32768, 128, 0) == 2 * 8 * 32 * 1 * 129 * 4
    assert fa.fa_fwd_decode_splits(1, 1, 1, 1 << 22) == fa.FA_MAX_SPLITS
    assert fa.fa_fwd_decode_splits(1, 1, 1, 300) == 1        # under 4 tiles per segment
    assert fa.fa_fwd_decode_splits(1, 4, 300, 65536) == 32   # 8 work-groups
    assert fa.fa_fwd_decode_splits(64, 32, 1, 65536) == 1
    assert fa.fa_fwd_decode_splits(0, 1, 1, 1) == 0
    for bad in ((0, 1, 1, 1, 64, 1), (1, 1, 0, 1, 64, 1), (1, 1, 1, 0, 64, 1),
                (1, 1, 1, 1, 96, 1), (1, 1, 1, 1, 64, -1), (1, 1, 1, 1, 64, 65)):
        assert fa.fa_fwd_decode_workspace_size(*bad) == 0


@pytest.mark.parametrize("kw", [dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
                                dict(ws=0), dict(B=0), dict(H=0), dict(Nq=0), dict(Nk=0),
                                dict(causal=2), dict(Nq=1001), dict(ns=-1), dict(ns=65),
                                dict(scale=float("inf")), dict(dtype=2), dict(o=QD),
                                dict(lse=KD + 64), dict(ws=OD), dict(o=KD + 1024)])
def test_decode_invalid(kw):
    assert dccall(**kw) == fa.FA_ERR_INVALID_ARG


def test_decode_unsupported_and_misaligned():
    assert dccall(d=32) == fa.FA_ERR_UNSUPPORTED
    assert dccall(Nk=(1 << 22) + 1) == fa.FA_ERR_UNSUPPORTED
    assert dccall(Nq=(1 << 22) + 1, causal=0) == fa.FA_ERR_UNSUPPORTED
    for kw in (dict(q=QD + 8), dict(k=KD + 2), dict(ws=WD + 4), dict(lse=LD + 2)):
        assert dccall(**kw) == fa.FA_ERR_MISALIGNED
    # non-causal decoding allows more queries than keys
    assert fa.fa_fwd_decode_workspace_size(1, 1, 50, 10, 64, 1) > 0


# ---------------------------------------------------------------- dropout

def dcall(q=Q, k=K, v=V, o=O, lse=L, B=1, H=1, N=64, d=128, causal=0, scale=0.125, p=0.1,
          seed=(1 << 40) + 7, offset=3, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, p, seed, offset, dtype,
                             None)


def dbcall(q=Q, k=K, v=V, o=O, do=DO, lse=L, ws=WS, dq=DQ, dk=DK, dv=DV, B=1, H=1, N=64,
           d=128, causal=0, scale=0.125, p=0.1, seed=5, offset=0, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd_dropout(q, k, v, o, do, lse, ws, dq, dk, dv, B, H, N, d, causal, scale, p,
                             seed, offset, dtype, None)


@pytest.mark.parametrize("kw", [dict(p=1.0), dict(p=-0.01), dict(p=math.nan), dict(p=2.0),
                                dict(causal=2), dict(q=0), dict(lse=0), dict(B=0),
                                dict(scale=math.nan), dict(dtype=9), dict(o=K + 64)])
def test_dropout_fwd_invalid(kw):
    assert dcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_dropout_fwd_unsupported_and_misaligned():
    assert dcall(d=96) == fa.FA_ERR_UNSUPPORTED
    assert dcall(q=Q + 4) == fa.FA_ERR_MISALIGNED
    assert dcall(lse=L + 2) == fa.FA_ERR_MISALIGNED


@pytest.mark.parametrize("kw", [dict(p=1.0), dict(p=-0.5), dict(p=math.inf), dict(p=math.nan),
                                dict(causal=-1), dict(ws=0), dict(dv=0), dict(N=0),
                                dict(dq=DK), dict(ws=Q)])
def test_dropout_bwd_invalid(kw):
    assert dbcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_dropout_bwd_unsupported_and_misaligned():
    assert dbcall(d=256) == fa.FA_ERR_UNSUPPORTED
    assert dbcall(dk=DK + 8) == fa.FA_ERR_MISALIGNED
    assert dbcall(ws=WS + 4) == fa.FA_ERR_MISALIGNED


# ---------------------------------------------------------------- packed varlen

CU = 0x10000 * 14


def vcall(q=Q, k=K, v=V, o=O, lse=L, cu=CU, B=2, H=1, total=64, maxlen=40, d=128, causal=0,
          scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_fwd_varlen(q, k, v, o, lse, cu, B, H, total, maxlen, d, causal, scale, dtype,
                            None)


@pytest.mark.parametrize("kw", [dict(cu=0), dict(q=0), dict(lse=0), dict(B=0), dict(H=0),
                                dict(total=0), dict(maxlen=0), dict(maxlen=65), dict(causal=2),
                                dict(scale=math.inf), dict(dtype=2), dict(o=Q + 16),
                                dict(cu=O + 64), dict(lse=CU)])
def test_varlen_invalid(kw):
    assert vcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_varlen_unsupported_and_misaligned():
    assert vcall(d=96) == fa.FA_ERR_UNSUPPORTED
    assert vcall(total=(1 << 22) + 2, maxlen=(1 << 22) + 1, q=1 << 40, k=2 << 40, v=3 << 40,
                 o=4 << 40, lse=5 << 40, cu=6 << 40) == fa.FA_ERR_UNSUPPORTED
    assert vcall(cu=CU + 2) == fa.FA_ERR_MISALIGNED
    assert vcall(v=V + 8) == fa.FA_ERR_MISALIGNED


def vbcall(q=Q, k=K, v=V, o=O, do=DO, lse=L, cu=CU, ws=WS, dq=DQ, dk=DK, dv=DV, B=2, H=1,
           total=64, maxlen=40, d=128, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd_varlen(q, k, v, o, do, lse, cu, ws, dq, dk, dv, B, H, total, maxlen, d,
                            causal, scale, dtype, None)


def test_varlen_bwd_workspace_size():
    # per head: 32 * (ceil(total / 32) + B) rows of two fp32 values
    assert fa.fa_bwd_varlen_workspace_size(1, 1, 1) == 2 * 32 * 2 * 4
    assert fa.fa_bwd_varlen_workspace_size(3, 2, 100) == 2 * 32 * (4 + 3) * 2 * 4
    assert fa.fa_bwd_varlen_workspace_size(2, 1, 64) == 32 * (2 + 2) * 2 * 4
    assert fa.fa_bwd_varlen_workspace_size(0, 1, 64) == 0
    assert fa.fa_bwd_varlen_workspace_size(1, 0, 64) == 0
    assert fa.fa_bwd_varlen_workspace_size(1, 1, 0) == 0


@pytest.mark.parametrize("kw", [dict(cu=0), dict(ws=0), dict(do=0), dict(dk=0), dict(B=0),
                                dict(H=0), dict(total=0), dict(maxlen=0), dict(maxlen=65),
                                dict(causal=2), dict(scale=math.nan), dict(dtype=2),
                                dict(dq=CU), dict(ws=CU - 16), dict(dv=DQ + 16),
                                dict(ws=DO), dict(dk=Q + 32)])
def test_varlen_bwd_invalid(kw):
    assert vbcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_varlen_bwd_unsupported_and_misaligned():
    assert vbcall(d=80) == fa.FA_ERR_UNSUPPORTED
    big = dict(total=(1 << 22) + 2, maxlen=(1 << 22) + 1)
    big.update({n: (i + 1) << 40 for i, n in enumerate(
        ("q", "k", "v", "o", "do", "lse", "cu", "ws", "dq", "dk", "dv"))})
    assert vbcall(**big) == fa.FA_ERR_UNSUPPORTED
    assert vbcall(cu=CU + 2) == fa.FA_ERR_MISALIGNED
    assert vbcall(ws=WS + 4) == fa.FA_ERR_MISALIGNED
    assert vbcall(dk=DK + 8) == fa.FA_ERR_MISALIGNED
    assert vbcall(lse=L + 1) == fa.FA_ERR_MISALIGNED


def wbcall(q=Q, k=K, v=V, o=O, do=DO, lse=L, ws=WS, dq=DQ, dk=DK, dv=DV, B=1, H=1, N=64,
           d=128, wl=16, wr=0, lens=LENS, scale=0.125, dtype=fa.FA_DTYPE_BF16):
    return fa.fa_bwd_window(q, k, v, o, do, lse, ws, dq, dk, dv, B, H, N, d, wl, wr, lens,
                            scale, dtype, None)


@pytest.mark.parametrize("kw", [dict(wl=-2), dict(wr=-3), dict(q=0), dict(ws=0), dict(B=0),
                                dict(N=0), dict(scale=math.inf), dict(dtype=4),
                                dict(dq=LENS), dict(ws=LENS - 16), dict(dk=Q + 64),
                                dict(ws=DO)])
def test_window_bwd_invalid(kw):
    assert wbcall(**kw) == fa.FA_ERR_INVALID_ARG


def test_window_bwd_unsupported_and_misaligned():
    assert wbcall(d=96) == fa.FA_ERR_UNSUPPORTED
    assert wbcall(lens=LENS + 2) == fa.FA_ERR_MISALIGNED
    assert wbcall(dv=DV + 8) == fa.FA_ERR_MISALIGNED
    assert wbcall(ws=WS + 4) == fa.FA_ERR_MISALIGNED
