"""HIP-graph capture of the library's calls, as a serving loop would use them.

A decode step (one new token per sequence appended to a contiguous cache and to a
ring, then a full-layer and a window-layer decode) and prefills (BSHD full and
window, and packed THD whose lengths change between replays) are captured once
with torch.cuda.graph and replayed several times. Between replays the inputs
change eagerly (new tokens and queries, lengths advanced, new cu_seqlens), and
the same calls also run eagerly on a copy of the state. Every replay must equal
the eager result bit for bit: the kernels are deterministic, and the library
makes no allocation, memset or synchronising call, and reads every length and
work list on the device, so a captured step needs nothing from the host.
Correctness against the oracle is the other test files' job.
"""

import pytest
import torch

import attention_yarn_rope_amd as gx
from helpers import say

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def _randn(shape, g):
    return torch.randn(shape, generator=g).to(BF).cuda()


def test_decode_step_graph():
    N, cap, Hkv, Hq = 6, 512, 8, 64
    g = torch.Generator().manual_seed(90)
    table = gx.rope_table(cap)
    kc, vc = _randn((N, cap, Hkv, 64), g), _randn((N, cap, Hkv, 64), g)
    rk, rv = _randn((N, 128, Hkv, 64), g), _randn((N, 128, Hkv, 64), g)
    sinks = torch.randn(Hq, generator=g).cuda()
    lens = torch.randint(1, 300, (N,), generator=g, dtype=torch.int32).cuda()
    q = torch.empty((N, Hq, 64), dtype=BF, device="cuda")
    kn = torch.empty((N, Hkv, 64), dtype=BF, device="cuda")
    vn = torch.empty_like(kn)
    ws_full = torch.empty(gx.decode_kv_workspace_size(q, kc, window=0, table=table), dtype=torch.uint8,
                          device="cuda")
    ws_ring = torch.empty(gx.decode_kv_workspace_size(q, rk, kind="ring", window=128, table=table),
                          dtype=torch.uint8, device="cuda")

    def step(kc, vc, rk, rv, o_full, o_ring):
        gx.kv_append(kc, vc, kn, vn, lens, table=table)
        gx.kv_append(rk, rv, kn, vn, lens, kind="ring", table=table)
        gx.attn_decode_kv(q, kc, vc, lens, sinks, window=0, table=table, out=o_full, workspace=ws_full)
        gx.attn_decode_kv(q, rk, rv, lens, sinks, kind="ring", window=128, table=table, out=o_ring,
                          workspace=ws_ring)

    state_e = [t.clone() for t in (kc, vc, rk, rv)]
    o_graph = [torch.empty_like(q), torch.empty_like(q)]
    o_eager = [torch.empty_like(q), torch.empty_like(q)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(kc, vc, rk, rv, *o_graph)
    for it in range(5):
        q.copy_(_randn((N, Hq, 64), g))
        kn.copy_(_randn((N, Hkv, 64), g))
        vn.copy_(_randn((N, Hkv, 64), g))
        lens.add_(1)
        graph.replay()
        step(*state_e, *o_eager)
        torch.cuda.synchronize()
        say(f"[gpu] decode step graph replay {it}: lengths {lens.tolist()}")
        assert torch.equal(o_graph[0], o_eager[0]), f"replay {it}: full-layer decode differs from eager"
        assert torch.equal(o_graph[1], o_eager[1]), f"replay {it}: ring decode differs from eager"
        for a, b, nm in zip((kc, vc, rk, rv), state_e, ("k cache", "v cache", "k ring", "v ring")):
            assert torch.equal(a, b), f"replay {it}: {nm} differs from eager"


def test_prefill_graph_bshd():
    B, S = 2, 700
    g = torch.Generator().manual_seed(91)
    table = gx.rope_table(S)
    q, k, v = _randn((B, S, 64, 64), g), _randn((B, S, 8, 64), g), _randn((B, S, 8, 64), g)
    sinks = torch.randn(64, generator=g).cuda()
    ws = torch.empty(gx.prefill_workspace_size(q, k), dtype=torch.uint8, device="cuda")
    o_graph = [torch.empty_like(q), torch.empty_like(q)]
    o_eager = [torch.empty_like(q), torch.empty_like(q)]

    def step(outs):
        gx.attn_prefill(q, k, v, sinks, window=0, table=table, out=outs[0], workspace=ws)
        gx.attn_prefill(q, k, v, sinks, window=128, table=table, out=outs[1], workspace=ws)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o_graph)
    for it in range(3):
        for t in (q, k, v):
            t.copy_(_randn(t.shape, g))
        graph.replay()
        step(o_eager)
        torch.cuda.synchronize()
        say(f"[gpu] BSHD prefill graph replay {it}")
        assert torch.equal(o_graph[0], o_eager[0]) and torch.equal(o_graph[1], o_eager[1]), f"replay {it}"


def test_prefill_graph_thd_lengths_change_between_replays():
    """The THD work list is built on the device from cu_seqlens, so one captured graph serves
    any packing of the same token count (max_seqlen, a host bound, is fixed at capture)."""
    T, bound = 900, 700
    g = torch.Generator().manual_seed(92)
    table = gx.rope_table(bound)
    q, k, v = _randn((T, 64, 64), g), _randn((T, 8, 64), g), _randn((T, 8, 64), g)
    sinks = torch.randn(64, generator=g).cuda()
    cu = torch.tensor([0, 300, 700, 900], dtype=torch.int32, device="cuda")
    ws = torch.empty(gx.prefill_workspace_size(q, k, cu_seqlens=cu, max_seqlen=bound), dtype=torch.uint8,
                     device="cuda")
    o_graph = [torch.empty_like(q), torch.empty_like(q)]
    o_eager = [torch.empty_like(q), torch.empty_like(q)]

    def step(outs):
        for i, w in enumerate((0, 128)):
            gx.attn_prefill(q, k, v, sinks, window=w, table=table, cu_seqlens=cu, max_seqlen=bound, out=outs[i],
                            workspace=ws)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o_graph)
    for it, lengths in enumerate(([300, 400, 200], [100, 700, 100], [450, 0, 450], [1, 699, 200])):
        cu.copy_(torch.tensor([0] + torch.tensor(lengths).cumsum(0).tolist(), dtype=torch.int32))
        q.copy_(_randn(q.shape, g))
        graph.replay()
        step(o_eager)
        torch.cuda.synchronize()
        say(f"[gpu] THD prefill graph replay {it}: lengths {lengths}")
        assert torch.equal(o_graph[0], o_eager[0]) and torch.equal(o_graph[1], o_eager[1]), f"replay {it}"
