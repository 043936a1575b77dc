"""Pins for the fp64 oracle, runnable against any build of oracle.c.

Each pin checks the oracle against something other than itself: a library
softmax/logsumexp on decoded inputs (torch fp64, decoding by torch's own
cast), pure-Python loops with math.fsum, closed forms, or invariants of the
definition.  ``run_pins(orc)`` returns the names of the pins that fail, so a
mutated oracle (a planted mistake) can be shown to fail at least one.

Pages: [P-baidu] "FlashAttention 优化原理与实现要点解析" (cloud.baidu.com),
[P-wmrh] "FlashAttention V2 核心原理与架构设计" (wmrh.cn).
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import torch

from io_aware_transformer_amd.inputs import bits, make_qkv

GOLDEN = Path(__file__).resolve().parent / "golden"

_TD = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Values -> 16-bit torch tensor (round to nearest even)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(_TD[dtype])


def torch_reference(q, k, v, causal: bool, scale: float):
    """Softmax(Q K^T * scale) V and logsumexp via torch fp64 library calls,
    on inputs decoded by torch's own cast."""
    q64, k64, v64 = q.double(), k.double(), v.double()
    s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * float(scale)
    N = q.shape[-2]
    if causal:
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p, v64)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy(), p.numpy()


def python_reference(q, k, v, causal: bool, scale: float):
    """Pure-Python loops, math.fsum sums; tiny inputs only."""
    qa, ka, va = q.double().tolist(), k.double().tolist(), v.double().tolist()
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(qa[b][h][i][c] * ka[b][h][j][c] for c in range(d))
                     for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                for c in range(d):
                    o[b, h, i, c] = math.fsum(w[t] * va[b][h][j][c]
                                              for t, j in enumerate(keys)) / den
                lse[b, h, i] = mx + math.log(den)
    return o, lse


def _close(a, b, tol) -> bool:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return False
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        return False
    return bool(np.max(np.abs(a - b), initial=0.0) <= tol)


def _qkv(B, H, N, d, dtype, seed, gain=1.0):
    q, k, v = make_qkv(B, H, N, d, dtype, seed=seed, qk_gain=gain)
    return q, k, v


def pin_brute_force(orc) -> bool:
    ok = True
    for dtype in ("f16", "bf16"):
        for causal in (False, True):
            q, k, v = _qkv(1, 2, 17, 8, dtype, seed=3)
            scale = float(np.float32(1 / math.sqrt(8)))
            o, lse = orc.attn_fwd(bits(q), bits(k), bits(v), dtype, causal, scale)
            ro, rl, _ = torch_reference(q, k, v, causal, scale)
            ok &= _close(o, ro, 1e-12) and _close(lse, rl, 1e-12)
    return ok


def pin_python_loops(orc) -> bool:
    q, k, v = _qkv(1, 1, 5, 3, "f16", seed=11)
    ok = True
    for causal in (False, True):
        o, lse = orc.attn_fwd(bits(q), bits(k), bits(v), "f16", causal, 0.7)
        po, pl = python_reference(q, k, v, causal, 0.7)
        ok &= _close(o, po, 1e-13) and _close(lse, pl, 1e-13)
    return ok


def pin_tiled(orc) -> bool:
    q, k, v = _qkv(1, 2, 23, 4, "bf16", seed=5)
    ok = True
    for causal in (False, True):
        ro, rl, _ = torch_reference(q, k, v, causal, 0.5)
        for br, bc in ((1, 1), (7, 5), (23, 23)):
            o, lse = orc.attn_fwd_tiled(bits(q), bits(k), bits(v), "bf16", causal, 0.5, br, bc)
            ok &= _close(o, ro, 1e-12) and _close(lse, rl, 1e-12)
    return ok


def pin_decode_golden(orc) -> bool:
    g = json.loads((GOLDEN / "decode_values.json").read_text())
    ok = True
    for dtype in ("f16", "bf16"):
        hx = np.array([int(h, 16) for h, _, _ in g[dtype]], dtype=np.uint16)
        want = [float(v) for _, v, _ in g[dtype]]
        got = orc.decode(hx, dtype)
        for a, b in zip(got, want):
            if math.isnan(b):
                ok &= math.isnan(a)
            else:
                ok &= (a == b) and (math.copysign(1, a) == math.copysign(1, b))
    return ok


def pin_softmax_1d(orc) -> bool:
    x = np.array([0.3, -2.0, 5.5, 5.5, -40.0, 1e-3, 700.0, 699.0])
    ref = torch.softmax(torch.from_numpy(x), 0).numpy()
    return (_close(orc.softmax_1d(x), ref, 1e-15)
            and _close(orc.softmax_online_1d(x), ref, 1e-15))


def pin_peaky_finite(orc) -> bool:
    q, k, v = _qkv(1, 1, 64, 64, "f16", seed=2, gain=30.0)
    o, lse = orc.attn_fwd(bits(q), bits(k), bits(v), "f16", False, 0.125)
    return bool(np.isfinite(o).all() and np.isfinite(lse).all())


def pin_causal_row0(orc) -> bool:
    q, k, v = _qkv(2, 2, 9, 16, "bf16", seed=4)
    o, lse = orc.attn_fwd(bits(q), bits(k), bits(v), "bf16", True, 0.25)
    ok = np.array_equal(o[:, :, 0, :], v[:, :, 0, :].double().numpy())
    s00 = 0.25 * (q[:, :, 0, :].double() * k[:, :, 0, :].double()).sum(-1).numpy()
    return bool(ok and _close(lse[:, :, 0], s00, 1e-14))


def pin_probs(orc) -> bool:
    q, k, v = _qkv(1, 2, 12, 8, "f16", seed=6)
    ok = True
    for causal in (False, True):
        p = orc.attn_probs(bits(q), bits(k), bits(v), "f16", causal, 0.4)
        _, _, rp = torch_reference(q, k, v, causal, 0.4)
        ok &= _close(p.sum(-1), np.ones(p.shape[:-1]), 1e-14) and _close(p, rp, 1e-14)
    return ok


def pin_rows(orc) -> bool:
    q, k, v = _qkv(2, 3, 19, 8, "bf16", seed=8)
    rows = np.array([0, 5, 18, 19, 57, 113], dtype=np.int64)
    ok = True
    for causal in (False, True):
        o, lse = orc.attn_fwd_rows(bits(q), bits(k), bits(v), "bf16", causal, 0.3, rows)
        ro, rl, _ = torch_reference(q, k, v, causal, 0.3)
        ok &= _close(o, ro.reshape(-1, 8)[rows], 1e-12)
        ok &= _close(lse, rl.reshape(-1)[rows], 1e-12)
    return ok


# ---------------------------------------------------------------- gradients

def torch_grad_reference(q, k, v, do, causal: bool, scale: float):
    """dQ, dK, dV by torch fp64 autograd through the library attention of
    torch_reference (inputs decoded by torch's own cast)."""
    qq, kk, vv = (t.double().clone().requires_grad_() for t in (q, k, v))
    s = torch.matmul(qq, kk.transpose(-1, -2)) * float(scale)
    N = q.shape[-2]
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    o.backward(do.double())
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


def _loss_python(q64, k64, v64, do64, causal, scale) -> float:
    """sum(dO * O) with O from the pure-Python forward (fp64 inputs)."""
    o, _ = python_reference(q64, k64, v64, causal, scale)
    return math.fsum((o * do64.numpy()).ravel().tolist())


def pin_bwd_autograd(orc) -> bool:
    ok = True
    for dtype in ("f16", "bf16"):
        for causal in (False, True):
            for (B, H, N, d) in ((1, 2, 13, 8), (2, 1, 5, 3)):
                q, k, v = _qkv(B, H, N, d, dtype, seed=N + d)
                do = _qkv(B, H, N, d, dtype, seed=N + d + 100)[0]
                dq, dk, dv = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), dtype, causal, 0.4)
                rq, rk, rv = torch_grad_reference(q, k, v, do, causal, 0.4)
                ok &= _close(dq, rq, 1e-12) and _close(dk, rk, 1e-12) and _close(dv, rv, 1e-12)
    return ok


def pin_bwd_finite_difference(orc) -> bool:
    """Central differences of sum(dO * O), O from the pure-Python loops:
    d/dx_e = (L(x + h e) - L(x - h e)) / 2h, for every element of q, k, v."""
    q, k, v = _qkv(1, 1, 4, 3, "f16", seed=12)
    do = _qkv(1, 1, 4, 3, "f16", seed=13)[0]
    h = 1e-6
    ok = True
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "f16", causal, 0.6)
        base = [q.double(), k.double(), v.double()]
        for which, got in enumerate((dq, dk, dv)):
            fd = np.zeros(got.shape)
            for idx in np.ndindex(*got.shape):
                plus = [t.clone() for t in base]
                minus = [t.clone() for t in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                fd[idx] = (_loss_python(*plus, do.double(), causal, 0.6)
                           - _loss_python(*minus, do.double(), causal, 0.6)) / (2 * h)
            ok &= _close(got, fd, 1e-7)
    return ok


def pin_bwd_invariants(orc) -> bool:
    """sum_j dK_j = 0 (every row of dS sums to zero), sum_j dV_j = sum_i dO_i
    (every row of P sums to one), constant V gives dQ = dK = 0, and causal
    row 0 (one key, weight 1) gets dQ_0 = 0."""
    ok = True
    for causal in (False, True):
        q, k, v = _qkv(2, 2, 21, 16, "bf16", seed=14)
        do = _qkv(2, 2, 21, 16, "bf16", seed=15)[0]
        dq, dk, dv = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.3)
        ok &= _close(dk.sum(2), np.zeros((2, 2, 16)), 1e-12)
        ok &= _close(dv.sum(2), do.double().numpy().sum(2), 1e-12)
        if causal:
            ok &= _close(dq[:, :, 0, :], np.zeros((2, 2, 16)), 1e-15)
        vc = v[:, :, :1, :].expand(2, 2, 21, 16).contiguous()
        dq2, dk2, _ = orc.attn_bwd(bits(q), bits(k), bits(vc), bits(do), "bf16", causal, 0.3)
        ok &= _close(dq2, np.zeros_like(dq2), 1e-13) and _close(dk2, np.zeros_like(dk2), 1e-13)
    return ok


def pin_bwd_rows(orc) -> bool:
    q, k, v = _qkv(2, 2, 19, 8, "f16", seed=16)
    do = _qkv(2, 2, 19, 8, "f16", seed=17)[0]
    qr = np.array([0, 4, 18, 19, 40, 75], dtype=np.int64)
    kr = np.array([0, 1, 18, 20, 37, 75], dtype=np.int64)
    ok = True
    for causal in (False, True):
        dq, dk, dv = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "f16", causal, 0.35)
        a, b, c = orc.attn_bwd_rows(bits(q), bits(k), bits(v), bits(do), "f16", causal, 0.35,
                                    qr, kr)
        ok &= _close(a, dq.reshape(-1, 8)[qr], 1e-12)
        ok &= _close(b, dk.reshape(-1, 8)[kr], 1e-12)
        ok &= _close(c, dv.reshape(-1, 8)[kr], 1e-12)
    return ok


def pin_bwd_given_o(orc) -> bool:
    """With a given 16-bit o the row term becomes dO_i . o_i, so the result
    moves from the plain gradients by exactly dD_i = dO_i . (o_i - O_i):
    dq by -scale dD_i (P K)_i, dk by -scale (P^T (dD q))_j, dv not at all."""
    ok = True
    for causal in (False, True):
        q, k, v = _qkv(1, 2, 19, 8, "bf16", seed=18)
        do = _qkv(1, 2, 19, 8, "bf16", seed=19)[0]
        ro, _, rp = torch_reference(q, k, v, causal, 0.45)
        o16 = to_tensor(ro, "bf16")
        dD = (do.double().numpy() * (o16.double().numpy() - ro)).sum(-1)
        g0 = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.45)
        g1 = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.45, o=bits(o16))
        q64, k64 = q.double().numpy(), k.double().numpy()
        want_dq = g0[0] - 0.45 * dD[..., None] * (rp @ k64)
        want_dk = g0[1] - 0.45 * (np.swapaxes(rp, -1, -2) @ (dD[..., None] * q64))
        ok &= _close(g1[0], want_dq, 1e-12) and _close(g1[1], want_dk, 1e-12)
        ok &= _close(g1[2], g0[2], 0.0)
        ok &= float(np.abs(dD).max()) > 1e-6          # the case really moves D
        r = np.array([0, 7, 18, 20, 37], dtype=np.int64)
        a, b, c = orc.attn_bwd_rows(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.45,
                                    r, r, o=bits(o16))
        ok &= _close(a, g1[0].reshape(-1, 8)[r], 1e-12) and _close(b, g1[1].reshape(-1, 8)[r], 1e-12)
        ok &= _close(c, g1[2].reshape(-1, 8)[r], 1e-12)
    return ok


# ---------------------------------------------------------------- masks

def masked_reference(q, k, v, wl, wr, seqlens, scale):
    """torch fp64 softmax with an explicit boolean mask matrix; rows without
    keys give o = 0 and lse = -inf."""
    B, H, N, d = q.shape
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    for b in range(B):
        L = N if seqlens is None else int(seqlens[b])
        allow = (j < L) & (i < L)
        if wl >= 0:
            allow &= j >= i - wl
        if wr >= 0:
            allow &= j <= i + wr
        s = torch.matmul(q[b].double(), k[b].double().transpose(-1, -2).contiguous()) * scale
        s = s.masked_fill(~allow, float("-inf"))
        has = allow.any(-1)
        p = torch.softmax(s[:, has], dim=-1)
        o[b][:, has.numpy()] = torch.matmul(p, v[b].double()).numpy()
        lse[b][:, has.numpy()] = torch.logsumexp(s[:, has], dim=-1).numpy()
    return o, lse


def pin_masked(orc) -> bool:
    ok = True
    q, k, v = _qkv(3, 2, 23, 8, "f16", seed=20)
    # no window, no padding = the plain definition; (-1, 0) = causal
    for causal, (wl, wr) in ((False, (-1, -1)), (True, (-1, 0))):
        o, lse = orc.attn_fwd_masked(bits(q), bits(k), bits(v), "f16", wl, wr, None, 0.3)
        ro, rl = orc.attn_fwd(bits(q), bits(k), bits(v), "f16", causal, 0.3)
        ok &= _close(o, ro, 0.0) and _close(lse, rl, 0.0)
    # a padded element equals its unpadded slice, on the valid rows
    lens = [23, 9, 1]
    o, lse = orc.attn_fwd_masked(bits(q), bits(k), bits(v), "f16", -1, -1, lens, 0.3)
    for b, L in enumerate(lens):
        sl = lambda t: t[b:b + 1, :, :L, :].contiguous()
        ro, rl = orc.attn_fwd(bits(sl(q)), bits(sl(k)), bits(sl(v)), "f16", False, 0.3)
        ok &= _close(o[b:b + 1, :, :L], ro, 1e-15) and _close(lse[b:b + 1, :, :L], rl, 1e-15)
        ok &= bool(np.all(o[b, :, L:] == 0.0) and np.all(np.isneginf(lse[b, :, L:])))
    # sliding windows against a library softmax with an explicit mask
    for (wl, wr), lens in (((4, 0), None), ((3, 2), [23, 17, 0]), ((0, 0), None),
                           ((-1, 5), [5, 23, 12])):
        o, lse = orc.attn_fwd_masked(bits(q), bits(k), bits(v), "f16", wl, wr, lens, 0.3)
        ro, rl = masked_reference(q, k, v, wl, wr, lens, 0.3)
        fin = np.isfinite(rl)
        ok &= _close(o, ro, 1e-12) and bool(np.array_equal(fin, np.isfinite(lse)))
        ok &= _close(lse[fin], rl[fin], 1e-12)
    return ok


def masked_grad_reference(q, k, v, do, wl, wr, seqlens, scale):
    """dQ, dK, dV by torch fp64 autograd through masked_reference's
    definition: a library softmax over each row's allowed keys (explicit
    boolean mask), rows without keys giving o = 0."""
    B, H, N, d = q.shape
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    grads = [np.zeros((B, H, N, d)) for _ in range(3)]
    for b in range(B):
        L = N if seqlens is None else int(seqlens[b])
        allow = (j < L) & (i < L)
        if wl >= 0:
            allow &= j >= i - wl
        if wr >= 0:
            allow &= j <= i + wr
        has = allow.any(-1)
        if not bool(has.any()):
            continue
        qq, kk, vv = (t[b].double().clone().requires_grad_() for t in (q, k, v))
        s = torch.matmul(qq, kk.transpose(-1, -2)) * float(scale)
        s = s.masked_fill(~allow, float("-inf"))
        o = torch.matmul(torch.softmax(s[:, has], dim=-1), vv)
        (o * do[b].double()[:, has]).sum().backward()
        for g, t in zip(grads, (qq, kk, vv)):
            g[b] = t.grad.numpy()
    return tuple(grads)


def pin_bwd_masked(orc) -> bool:
    ok = True
    q, k, v = _qkv(3, 2, 21, 8, "bf16", seed=30)
    do = _qkv(3, 2, 21, 8, "bf16", seed=31)[0]
    # no window, no padding = the plain gradients; (-1, 0) = causal; also
    # with the row term from a given o
    o16 = _qkv(3, 2, 21, 8, "bf16", seed=32)[0]
    for causal, (wl, wr) in ((False, (-1, -1)), (True, (-1, 0))):
        for given in (None, bits(o16)):
            g = orc.attn_bwd_masked(bits(q), bits(k), bits(v), bits(do), "bf16", wl, wr, None,
                                    0.35, o=given)
            r = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.35,
                             o=given)
            ok &= all(_close(a, c, 1e-14) for a, c in zip(g, r))
    # windows and lengths against autograd through a library softmax
    for (wl, wr), lens in (((4, 0), None), ((3, 2), [21, 15, 0]), ((0, 0), None),
                           ((-1, 5), [5, 21, 1]), ((6, -1), [20, 2, 21])):
        g = orc.attn_bwd_masked(bits(q), bits(k), bits(v), bits(do), "bf16", wl, wr, lens, 0.35)
        r = masked_grad_reference(q, k, v, do, wl, wr, lens, 0.35)
        ok &= all(_close(a, c, 1e-12) for a, c in zip(g, r))
        # padded rows and keys get no gradient
        if lens is not None:
            for b, L in enumerate(lens):
                ok &= all(bool(np.all(x[b, :, L:] == 0.0)) for x in g)
    return ok


# ---------------------------------------------------------------- dropout

def pin_philox_kat(orc) -> bool:
    g = json.loads((GOLDEN / "philox4x32_10_kat.json").read_text())
    ok = True
    for vec in g["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        kk = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["out"]]
        ok &= [int(x) for x in orc.philox4x32_10(c, kk)] == want
    return ok


def pin_dropout(orc) -> bool:
    import oracle as _o
    ok = True
    seed, off = 0x0123456789ABCDEF, 7
    # the mapping: element (bh, i, j) takes byte 4 (j%32 // 8) + j%4 of the call
    # with counter (i, 2 (j // 32) + (j // 4) % 2, bh, offset)
    T = _o.dropout_threshold(0.3)
    z = orc.dropout_factors(3, 70, seed, off, T)
    key = [seed & 0xffffffff, seed >> 32]
    want = np.zeros_like(z)
    for bh in range(3):
        for i in range(70):
            for jb in range(3):
                for hh in range(2):
                    out = orc.philox4x32_10([i, 2 * jb + hh, bh, off], key)
                    for g in range(4):
                        for e in range(4):
                            j = 32 * jb + 8 * g + 4 * hh + e
                            if j < 70:
                                byte = (int(out[g]) >> (8 * e)) & 0xff
                                want[bh, i, j] = 256.0 / T if byte < T else 0.0
    ok &= bool(np.array_equal(z, want))
    # keep rate within 5 sigma of T/256
    kept = float((z > 0).mean())
    ok &= abs(kept - T / 256) <= 5 * math.sqrt(T / 256 * (1 - T / 256) / z.size)
    # p = 0: plain attention; o_i = sum_j P_ij Z_ij v_j against torch fp64
    q, k, v = _qkv(2, 2, 29, 8, "bf16", seed=22)
    do = _qkv(2, 2, 29, 8, "bf16", seed=23)[0]
    for causal in (False, True):
        o0, l0 = orc.attn_fwd_dropout(bits(q), bits(k), bits(v), "bf16", causal, 0.4, 256, seed, off)
        ro, rl = orc.attn_fwd(bits(q), bits(k), bits(v), "bf16", causal, 0.4)
        ok &= _close(o0, ro, 1e-14) and _close(l0, rl, 0.0)
        o1, l1 = orc.attn_fwd_dropout(bits(q), bits(k), bits(v), "bf16", causal, 0.4, T, seed, off)
        _, tl, tp = torch_reference(q, k, v, causal, 0.4)
        Z = orc.dropout_factors(4, 29, seed, off, T).reshape(2, 2, 29, 29)
        ok &= _close(o1, (tp * Z) @ v.double().numpy(), 1e-12) and _close(l1, tl, 1e-12)
        # backward: autograd of sum(dO * (softmax(S) o Z) V), shifted by the
        # given-o row term dD_i = dO_i . (o_i - O_i) exactly as without dropout
        ro16 = to_tensor(o1, "bf16")
        g = orc.attn_bwd_dropout(bits(q), bits(k), bits(v), bits(do), bits(ro16), "bf16", causal,
                                 0.4, T, seed, off)
        qq, kk2, vv = (t.double().clone().requires_grad_() for t in (q, k, v))
        sc = torch.matmul(qq, kk2.transpose(-1, -2)) * 0.4
        if causal:
            sc = sc.masked_fill(torch.ones(29, 29, dtype=torch.bool).triu(1), float("-inf"))
        P = torch.softmax(sc, dim=-1)
        torch.matmul(P * torch.from_numpy(Z), vv).backward(do.double())
        dD = (do.double().numpy() * (ro16.double().numpy() - o1)).sum(-1)
        Pn = P.detach().numpy()
        want_dq = qq.grad.numpy() - 0.4 * dD[..., None] * (Pn @ k.double().numpy())
        want_dk = kk2.grad.numpy() - 0.4 * (np.swapaxes(Pn, -1, -2) @ (dD[..., None] * q.double().numpy()))
        ok &= _close(g[0], want_dq, 1e-12) and _close(g[1], want_dk, 1e-12)
        ok &= _close(g[2], vv.grad.numpy(), 1e-12)
        g0 = orc.attn_bwd_dropout(bits(q), bits(k), bits(v), bits(do), bits(ro16), "bf16", causal,
                                  0.4, 256, seed, off)
        g1 = orc.attn_bwd(bits(q), bits(k), bits(v), bits(do), "bf16", causal, 0.4, o=bits(ro16))
        ok &= all(_close(a, b, 1e-14) for a, b in zip(g0, g1))
    return ok


def pin_dropout_rows(orc) -> bool:
    """The sampled-row dropout functions against the full ones."""
    import oracle as _o
    seed, off = 0xFEEDFACE12345678, 3
    T = _o.dropout_threshold(0.25)
    q, k, v = _qkv(2, 2, 45, 8, "f16", seed=31)
    do = _qkv(2, 2, 45, 8, "f16", seed=32)[0]
    qr = np.array([0, 7, 44, 45, 90, 179], dtype=np.int64)
    kr = np.array([0, 1, 44, 46, 100, 179], dtype=np.int64)
    ok = True
    for causal in (False, True):
        o, lse = orc.attn_fwd_dropout(bits(q), bits(k), bits(v), "f16", causal, 0.35, T, seed, off)
        a, b = orc.attn_fwd_dropout_rows(bits(q), bits(k), bits(v), "f16", causal, 0.35, T, seed,
                                         off, qr)
        ok &= bool(np.array_equal(a, o.reshape(-1, 8)[qr]) and np.array_equal(b, lse.reshape(-1)[qr]))
        o16 = to_tensor(o, "f16")
        dq, dk, dv = orc.attn_bwd_dropout(bits(q), bits(k), bits(v), bits(do), bits(o16), "f16",
                                          causal, 0.35, T, seed, off)
        a, b, c = orc.attn_bwd_dropout_rows(bits(q), bits(k), bits(v), bits(do), bits(o16), "f16",
                                            causal, 0.35, T, seed, off, qr, kr)
        ok &= _close(a, dq.reshape(-1, 8)[qr], 1e-12)
        ok &= _close(b, dk.reshape(-1, 8)[kr], 1e-12)
        ok &= _close(c, dv.reshape(-1, 8)[kr], 1e-12)
    return ok


# ---------------------------------------------------------------- decoding

def decode_reference(q, k, v, causal: bool, scale: float):
    """torch fp64 softmax over an explicit mask for Nq queries against Nk
    keys: query i may use key j when j <= i + Nk - Nq if causal (every key
    otherwise); rows without keys give o = 0 and lse = -inf."""
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    allow = (j <= i + (Nk - Nq)) if causal else torch.ones(Nq, Nk, dtype=torch.bool)
    s = torch.matmul(q.double(), k.double().transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~allow, float("-inf"))
    has = allow.any(-1)
    o = np.zeros((B, H, Nq, d))
    lse = np.full((B, H, Nq), -np.inf)
    if bool(has.any()):
        sh = s[:, :, has, :]
        o[:, :, has.numpy()] = torch.matmul(torch.softmax(sh, dim=-1), v.double()).numpy()
        lse[:, :, has.numpy()] = torch.logsumexp(sh, dim=-1).numpy()
    return o, lse


def _decode_qkv(B, H, Nq, Nk, d, dtype, seed):
    q = make_qkv(B, H, Nq, d, dtype, seed=seed)[0]
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed=seed + 1)
    return q, k, v


def pin_decode(orc) -> bool:
    ok = True
    # a library softmax with the explicit bottom-right mask; B*H > 1 so the
    # per-head strides of Q (Nq rows) and K/V (Nk rows) both matter
    for dtype in ("f16", "bf16"):
        for Nq, Nk in ((1, 37), (5, 37), (37, 37), (6, 4)):
            q, k, v = _decode_qkv(2, 3, Nq, Nk, 8, dtype, seed=40 + Nq)
            for causal in (False, True):
                o, lse = orc.attn_fwd_decode(bits(q), bits(k), bits(v), dtype, causal, 0.35)
                ro, rl = decode_reference(q, k, v, causal, 0.35)
                fin = np.isfinite(rl)
                ok &= bool(np.array_equal(fin, np.isfinite(lse)))
                ok &= _close(o, ro, 1e-12) and _close(lse[fin], rl[fin], 1e-12)
    # the last Nq rows of a square causal problem over the same keys
    qf, k, v = _qkv(2, 2, 29, 8, "bf16", seed=47)
    fo, fl = orc.attn_fwd(bits(qf), bits(k), bits(v), "bf16", True, 0.4)
    for Nq in (1, 3, 29):
        qs = qf[:, :, 29 - Nq:, :].contiguous()
        o, lse = orc.attn_fwd_decode(bits(qs), bits(k), bits(v), "bf16", True, 0.4)
        ok &= _close(o, fo[:, :, 29 - Nq:], 1e-15) and _close(lse, fl[:, :, 29 - Nq:], 1e-15)
    # Q = 0: every allowed key weighs the same, so lse = ln |A_i| and o is
    # the mean of the allowed V rows; constant V rows give that constant
    Nq, Nk = 4, 11
    q, k, v = _decode_qkv(1, 2, Nq, Nk, 8, "f16", seed=48)
    z = torch.zeros_like(q)
    vv = v.double().numpy()
    for causal in (False, True):
        o, lse = orc.attn_fwd_decode(bits(z), bits(k), bits(v), "f16", causal, 0.7)
        for i in range(Nq):
            n = (i + Nk - Nq + 1) if causal else Nk
            ok &= _close(lse[:, :, i], np.full((1, 2), math.log(n)), 1e-15)
            ok &= _close(o[:, :, i], vv[:, :, :n].mean(axis=2), 1e-14)
        cv = torch.full_like(v, 1.625)
        o, _ = orc.attn_fwd_decode(bits(q), bits(k), bits(cv), "f16", causal, 0.7)
        ok &= _close(o, np.full(o.shape, 1.625), 1e-14)
    return ok


PINS = {
    "brute_force": pin_brute_force,
    "python_loops": pin_python_loops,
    "tiled": pin_tiled,
    "decode_golden": pin_decode_golden,
    "softmax_1d": pin_softmax_1d,
    "peaky_finite": pin_peaky_finite,
    "causal_row0": pin_causal_row0,
    "probs": pin_probs,
    "rows": pin_rows,
    "bwd_autograd": pin_bwd_autograd,
    "bwd_finite_difference": pin_bwd_finite_difference,
    "bwd_invariants": pin_bwd_invariants,
    "bwd_rows": pin_bwd_rows,
    "bwd_given_o": pin_bwd_given_o,
    "masked": pin_masked,
    "decode": pin_decode,
    "bwd_masked": pin_bwd_masked,
    "philox_kat": pin_philox_kat,
    "dropout": pin_dropout,
    "dropout_rows": pin_dropout_rows,
}


def run_pins(orc) -> list:
    """Names of the pins that fail (an exception counts as a failure)."""
    failed = []
    for name, fn in PINS.items():
        try:
            ok = fn(orc)
        except Exception:  # a mutant may crash a pin; that is a failure
            ok = False
        if not ok:
            failed.append(name)
    return failed
