"""HIP graph capture of the library's entry points.

The calls allocate nothing, never synchronise and only enqueue kernels on
the stream they are given, so a whole forward + backward step can be
captured once and replayed.  The test captures fa_fwd, fa_bwd,
fa_fwd_dropout, fa_bwd_dropout, fa_fwd_split, fa_fwd_window, fa_fwd_varlen
and fa_bwd_varlen into one graph.  It replays the graph three times with new inputs copied into the
captured buffers (eager work and synchronisations in between) and checks
every replay bit for bit against the same calls run eagerly."""
from __future__ import annotations

import pytest
import torch

import io_aware_transformer_amd as fa
from io_aware_transformer_amd.inputs import make_qkv
from tests.parity_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.load()


def _ok(st):
    assert st == fa.FA_OK, fa.fa_status_string(st)


def test_graph_replay_matches_eager():
    note("[graph] capture of forward, backward, dropout, split, window and varlen calls")
    dev = torch.device("cuda", 0)
    B, H, N, d, causal, scale = 1, 3, 700, 128, 1, 0.088
    dt = fa.FA_DTYPE_BF16
    q, k, v, do = (torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev) for _ in range(4))
    o, o2, o3, o4 = (torch.empty_like(q) for _ in range(4))
    lse, lse2, lse3, lse4 = (torch.empty((B, H, N), dtype=torch.float32, device=dev)
                             for _ in range(4))
    g1, g2 = ([torch.empty_like(q) for _ in range(3)] for _ in range(2))
    ws1, ws2 = (torch.empty(fa.fa_bwd_workspace_size(B, H, N) // 4, dtype=torch.float32,
                            device=dev) for _ in range(2))
    sws = torch.empty(fa.fa_fwd_split_workspace_size(B, H, N, d, 3) // 4, dtype=torch.float32,
                      device=dev)
    # packed layout: q[0] is [H, N, d], three sequences of the N tokens
    cu = torch.tensor([0, 200, 450, N], dtype=torch.int32, device=dev)
    o5 = torch.empty_like(q[0])
    lse5 = torch.empty((H, N), dtype=torch.float32, device=dev)
    g3 = [torch.empty_like(q[0]) for _ in range(3)]
    ws3 = torch.empty(fa.fa_bwd_varlen_workspace_size(3, H, N) // 4, dtype=torch.float32,
                      device=dev)
    outs = (o, lse, *g1, o2, lse2, *g2, o3, lse3, o4, lse4, o5, lse5, *g3)

    def step(stream):
        _ok(fa.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dt, stream))
        _ok(fa.fa_bwd(q, k, v, o, do, lse, ws1, *g1, B, H, N, d, causal, scale, dt, stream))
        _ok(fa.fa_fwd_dropout(q, k, v, o2, lse2, B, H, N, d, causal, scale, 0.1, 77, 5, dt,
                              stream))
        _ok(fa.fa_bwd_dropout(q, k, v, o2, do, lse2, ws2, *g2, B, H, N, d, causal, scale, 0.1,
                              77, 5, dt, stream))
        _ok(fa.fa_fwd_split(q, k, v, o3, lse3, B, H, N, d, causal, scale, 3, sws, dt, stream))
        _ok(fa.fa_fwd_window(q, k, v, o4, lse4, B, H, N, d, 200, 0, None, scale, dt, stream))
        _ok(fa.fa_fwd_varlen(q[0], k[0], v[0], o5, lse5, cu, 3, H, N, 250, d, causal, scale, dt,
                             stream))
        _ok(fa.fa_bwd_varlen(q[0], k[0], v[0], o5, do[0], lse5, cu, ws3, *g3, 3, H, N, 250, d,
                             causal, scale, dt, stream))

    def load_inputs(seed):
        a, b, c = make_qkv(B, H, N, d, "bf16", seed=seed)
        e = make_qkv(B, H, N, d, "bf16", seed=seed + 1)[0]
        for dst, src in zip((q, k, v, do), (a, b, c, e)):
            dst.copy_(src.to(dev))

    # warm-up on a side stream, then capture
    load_inputs(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for trial in range(3):
        load_inputs(200 + trial)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = [t.clone() for t in outs]
        for t in outs:
            t.fill_(float("nan"))
        step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for a, b in zip(replayed, outs):
            assert torch.isfinite(a).all()
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
