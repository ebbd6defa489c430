"""GPU parity of partial rotary inside the attention calls (rotary_dim 16, 32, 48 with a table).

The rope_utils page's apply_rotary_emb rotates the first rotary_dim dims of each
head in half-split pairs (i, i + rotary_dim / 2) and passes the rest through
(RotaryEmbedding's partial_rotary_factor). With such a table the prefill and
decode kernels rotate q themselves (k by the K pass, or by the KV-cache append)
and must equal the oracle with the same RopeConfig, and bit for bit the path that
rotates q and k with gptoss_rope_qk first and passes table = NULL.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say
from oracle import context_parallel as cp
from oracle import kvcache as kv

pytestmark = pytest.mark.gpu
TAU = 0.125


def _table(rd, rows):
    return gx.rope_table(rows, gx.rope_config(rotary_dim=rd)), oracle.RopeConfig(rotary_dim=rd)


@pytest.mark.parametrize("rd", [16, 32, 48])
@pytest.mark.parametrize("window", [0, 128])
def test_prefill_bshd(rd, window):
    table, cfg = _table(rd, 400)
    inp = wl.prefill_bshd(2, 333, seed=700 + rd + window)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    say(f"[gpu] prefill with rotary_dim {rd} W={window}")
    out = gx.attn_prefill(q, k, v, s, window=window, table=table)
    ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), TAU, window, cfg)
    assert_close(out, ref, f"rd={rd} W={window}")
    qr, kr = gx.rope_qk(q, k, table)
    assert torch.equal(out, gx.attn_prefill(qr, kr, v, s, window=window, table=None)), "fused != pre-rotated"


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_thd_and_lse(window):
    table, cfg = _table(32, 600)
    inp = wl.prefill_thd(0, 0, 0, seed=710 + window, lengths=[37, 0, 300, 129, 500])
    q, k, v, s, cu = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), inp.cu_seqlens.cuda()
    say(f"[gpu] THD prefill with rotary_dim 32 W={window}")
    out, lse = gx.attn_prefill_lse(q, k, v, s, window=window, table=table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    ref = oracle.prefill_thd(np64(inp.q), np64(inp.k), np64(inp.v), inp.cu_seqlens.numpy(), np64(inp.sinks), TAU,
                             window, cfg)
    assert_close(out, ref, f"thd rd=32 W={window}")
    qr, kr = gx.rope_qk(q, k, table, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    o2, l2 = gx.attn_prefill_lse(qr, kr, v, s, window=window, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_shard():
    table, cfg = _table(48, 2000)
    g = torch.Generator().manual_seed(720)
    q = torch.randn((1, 96, 64, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, 160, 8, 64), generator=g).to(torch.bfloat16)
    v = torch.randn((1, 160, 8, 64), generator=g).to(torch.bfloat16)
    say("[gpu] context-parallel shard with rotary_dim 48")
    out, lse = gx.attn_prefill_shard(q.cuda(), k.cuda(), v.cuda(), 1000, 900, window=0, table=table)
    ro, rl = cp.shard_attention(np64(q), np64(k), np64(v), TAU, 0, 1000, 900, cfg)
    assert_close(out, ro, "shard rd=48")
    assert float(np.abs(np64(lse).reshape(rl.shape) - rl).max()) <= 2.0 ** -8 + 1e-4


@pytest.mark.parametrize("rd", [16, 32])
@pytest.mark.parametrize("window", [0, 128])
def test_decode(rd, window):
    table, cfg = _table(rd, 2100)
    d = wl.decode(0, 0, 0, seed=730 + rd + window, max_len=2048, lengths=[1, 100, 2048, 777])
    say(f"[gpu] decode with rotary_dim {rd} W={window}")
    q, kc, vc, lens, s = d.q.cuda(), d.k_cache.cuda(), d.v_cache.cuda(), d.cache_seqlens.cuda(), d.sinks.cuda()
    out = gx.attn_decode(q, kc, vc, lens, s, window=window, table=table)
    ref = oracle.decode(np64(d.q), np64(d.k_cache), np64(d.v_cache), d.lengths, np64(d.sinks), TAU, window, cfg)
    assert_close(out, ref, f"decode rd={rd} W={window}")
    # the same over the cache-layout entry point and the allocation-free one
    assert torch.equal(out, gx.attn_decode_kv(q, kc, vc, lens, s, window=window, table=table))
    assert torch.equal(out, gx.attn_decode_kv_noalloc(q, kc, vc, lens, s, window=window, table=table))


def test_generation_step_paged():
    """A prompt appended with a rotary_dim-32 table, then one decode step from the paged cache."""
    table, cfg = _table(32, 600)
    lengths = [50, 300, 17]
    w = wl.paged_decode(lengths, 32, seed=740)
    say("[gpu] paged decode with rotary_dim 32")
    out = gx.attn_decode_kv(w.q.cuda(), w.k_pool.cuda(), w.v_pool.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda(),
                            kind="paged", block_table=w.block_table.cuda(), table=table, max_seqlen=300)
    lay = kv.KVLayout(kv.PAGED, w.k_pool.shape[1], w.block_table.numpy())
    ref = kv.decode(lay, np64(w.q), w.k_pool.float().numpy(), w.v_pool.float().numpy(), w.lengths, np64(w.sinks),
                    TAU, 0, cfg)
    assert_close(out, ref, "paged rd=32")
