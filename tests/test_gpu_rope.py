"""GPU parity of the YaRN table and the standalone q/k rotation (through the C ABI).

Bar: the table and the rotated q/k are compared BIT-FOR-BIT with the oracle
(both round the exact value once to bf16). The table allows a handful of
1-ulp entries, which can only come from the device and host libm cos/sin
differing in the last fp64 bit right at a bf16 midpoint; the count is printed.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import bits16, np64, say

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()


@pytest.fixture(scope="module")
def table128k():
    say("[gpu] rope table 131072 rows")
    t = gx.rope_table(131072)
    torch.cuda.synchronize()
    return t


def test_table_matches_oracle_bits(table128k):
    ref = oracle.bf16_bits(oracle.freqs_cis(CFG, 131072))
    got = bits16(table128k)
    diff = got != ref
    n = int(diff.sum())
    say(f"  table entries differing: {n} of {ref.size}")
    if n:
        d = np.abs(got[diff].astype(np.int32) - ref[diff].astype(np.int32))
        assert d.max() == 1, "differences larger than one bf16 ulp"
    assert n <= 8


@pytest.mark.parametrize("cfg", [oracle.RopeConfig(scaling_factor=1.0), oracle.RopeConfig(base=10000.0,
                                 scaling_factor=8.0, initial_context_length=2048)])
def test_table_other_configs(cfg):
    c = gx.rope_config(base=cfg.base, scaling_factor=cfg.scaling_factor,
                       initial_context_length=cfg.initial_context_length)
    om, conc = gx.yarn_params(c)
    om_ref, conc_ref, _ = oracle.yarn_params(cfg)
    assert np.array_equal(np.array(om), om_ref) and conc == conc_ref
    got = bits16(gx.rope_table(5000, c))
    ref = oracle.bf16_bits(oracle.freqs_cis(cfg, 5000))
    assert int((got != ref).sum()) <= 2


def _rope_ref(q, k, cu=None):
    if cu is None:
        return oracle.rope_qk_bshd(np64(q), np64(k), CFG)
    return oracle.rope_qk_thd(np64(q), np64(k), cu, CFG)


@pytest.mark.parametrize("B,S", [(1, 1), (2, 300), (3, 1031)])
def test_rope_qk_bshd_bit_exact(table128k, B, S):
    inp = wl.prefill_bshd(B, S, seed=100 + S)
    say(f"[gpu] rope_qk bshd B={B} S={S}")
    q, k = inp.q.cuda(), inp.k.cuda()
    qo, ko = gx.rope_qk(q, k, table128k)
    rq, rk = _rope_ref(inp.q, inp.k)
    assert np.array_equal(np64(qo), rq)
    assert np.array_equal(np64(ko), rk)


def test_rope_qk_thd_bit_exact(table128k):
    inp = wl.prefill_thd(0, 0, 0, seed=7, lengths=[5, 0, 130, 1, 777, 64])
    say("[gpu] rope_qk thd")
    cu = inp.cu_seqlens.cuda()
    qo, ko = gx.rope_qk(inp.q.cuda(), inp.k.cuda(), table128k, cu_seqlens=cu, max_seqlen=inp.max_seqlen)
    rq, rk = _rope_ref(inp.q, inp.k, inp.cu_seqlens.numpy())
    assert np.array_equal(np64(qo), rq)
    assert np.array_equal(np64(ko), rk)


def test_rope_qk_strided_views(table128k):
    """q and k as views into one fused qkv buffer [B, S, Hq + 2 Hkv, D] (arbitrary strides)."""
    g = torch.Generator().manual_seed(9)
    B, S = 2, 257
    qkv = torch.randn((B, S, 64 + 16, 64), generator=g).to(torch.bfloat16)
    q, k = qkv[:, :, :64], qkv[:, :, 64:72]
    say("[gpu] rope_qk strided")
    qd = qkv.cuda()
    qo, ko = gx.rope_qk(qd[:, :, :64], qd[:, :, 64:72], table128k)
    rq, rk = _rope_ref(q, k)
    assert qo.is_contiguous() and np.array_equal(np64(qo), rq)
    assert np.array_equal(np64(ko), rk)


def test_rope_qk_far_positions(table128k):
    """Positions near 128K: one sequence of 131072 tokens, spot-checked over the last rows."""
    g = torch.Generator().manual_seed(10)
    S = 131072
    q = torch.randn((1, S, 8, 64), generator=g).to(torch.bfloat16)
    k = torch.randn((1, S, 1, 64), generator=g).to(torch.bfloat16)
    say("[gpu] rope_qk S=131072")
    qo, ko = gx.rope_qk(q.cuda(), k.cuda(), table128k)
    rows = np.r_[0:64, S - 4096:S]
    cos, sin = oracle.cos_sin_table(CFG, rows)
    rq = oracle.rotate(np64(q[0, rows]), cos[:, None, :], sin[:, None, :])
    assert np.array_equal(np64(qo[0, rows]), rq)
    rk = oracle.rotate(np64(k[0, rows]), cos[:, None, :], sin[:, None, :])
    assert np.array_equal(np64(ko[0, rows]), rk)


@pytest.mark.parametrize("rd", [16, 32, 48])
def test_rope_qk_partial_rotary_bit_exact(rd):
    """rotary_dim < 64: the first rd dims rotate in pairs (i, i + rd/2), the rest are copied."""
    cfg = oracle.RopeConfig(rotary_dim=rd)
    table = gx.rope_table(1100, gx.rope_config(rotary_dim=rd))
    assert tuple(table.shape) == (1100, rd)
    # the table is rounded from fp64 sin/cos on both sides; a near-tie entry may round
    # the other way (at most a couple per 10^5). Positions whose row differs are
    # left out of the bit-exact comparison.
    same = (bits16(table) == oracle.bf16_bits(oracle.freqs_cis(cfg, 1100))).all(axis=1)
    assert int((~same).sum()) <= 2
    inp = wl.prefill_bshd(2, 1031, seed=300 + rd)
    say(f"[gpu] rope_qk partial rotary rd={rd} ({int((~same).sum())} table rows differ)")
    qo, ko = gx.rope_qk(inp.q.cuda(), inp.k.cuda(), table)
    rq, rk = oracle.rope_qk_bshd(np64(inp.q), np64(inp.k), cfg)
    keep = same[:1031]
    assert np.array_equal(np64(qo)[:, keep], rq[:, keep]) and np.array_equal(np64(ko)[:, keep], rk[:, keep])
    assert torch.equal(qo[..., rd:].cpu(), inp.q[..., rd:])
    t = wl.prefill_thd(0, 0, 0, seed=310 + rd, lengths=[7, 0, 300, 64])
    qo, ko = gx.rope_qk(t.q.cuda(), t.k.cuda(), table, cu_seqlens=t.cu_seqlens.cuda(), max_seqlen=t.max_seqlen)
    rq, rk = oracle.rope_qk_thd(np64(t.q), np64(t.k), t.cu_seqlens.numpy(), cfg)
    keep = same[oracle.thd_positions(t.cu_seqlens.numpy(), t.q.shape[0])]
    assert np.array_equal(np64(qo)[keep], rq[keep]) and np.array_equal(np64(ko)[keep], rk[keep])


def test_partial_rotary_attention_through_pre_rotation():
    """Prefill with rotary_dim 32: q and k rotated by rope_qk, then attention with table=None,
    against the oracle's prefill with the same partial rotary."""
    from helpers import assert_close
    cfg = oracle.RopeConfig(rotary_dim=32)
    table = gx.rope_table(400, gx.rope_config(rotary_dim=32))
    inp = wl.prefill_bshd(2, 333, seed=320)
    s = inp.sinks.cuda()
    qr, kr = gx.rope_qk(inp.q.cuda(), inp.k.cuda(), table)
    for w in (0, 128):
        out = gx.attn_prefill(qr, kr, inp.v.cuda(), s, window=w, table=None)
        ref = oracle.prefill_bshd(np64(inp.q), np64(inp.k), np64(inp.v), np64(inp.sinks), 0.125, w, cfg)
        assert_close(out, ref, f"partial rotary rd=32 W={w}")


def test_kv_append_partial_rotary_bit_exact():
    from oracle import kvcache as kv
    cfg = oracle.RopeConfig(rotary_dim=32)
    table = gx.rope_table(200, gx.rope_config(rotary_dim=32))
    kn, vn = wl.new_tokens(3, 5, 330)
    kc = torch.zeros((3, 160, 8, 64), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    kg, vg = kc.cuda(), vc.cuda()
    lens = [5, 77, 160]
    gx.kv_append(kg, vg, kn.cuda(), vn.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table=table,
                 max_seqlen=160)
    rk, rv = kv.append(kv.KVLayout(kv.CONTIGUOUS, 160), np64(kc), np64(vc), np64(kn), np64(vn), lens, cfg)
    same = (bits16(table) == oracle.bf16_bits(oracle.freqs_cis(cfg, 200))).all(axis=1)
    assert int((~same).sum()) <= 2
    g, r = np64(kg), rk
    for n, L in enumerate(lens):
        pos = np.arange(L - 5, L)
        pos = pos[same[pos]]
        assert np.array_equal(g[n, pos], r[n, pos])
    assert np.array_equal(np64(vg), rv)
