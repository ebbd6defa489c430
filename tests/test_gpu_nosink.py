"""GPU parity of rows without a sink term whose logits all lie far below zero.

With sigma = -inf the sink drops out of the softmax denominator and the layer is
plain causal / window softmax attention (page "nemo_automodel.components.models.
gpt_oss.layers", GptOssAttention.sinks; Transformers v4.55.0 release notes,
"Architecture": the sink is one more term of the denominator). Softmax is
invariant under a common shift of the logits, so rows whose logits are all near
-512 must give the same result as rows near 0. A kernel that normalises against
a fixed reference of 0 instead of the row's own scale underflows every exp()
there and writes 0 (or lse = -inf).

Inputs are already rotated (no table): q = -8 + a and k = +8 + b in every
dimension with a, b ~ c * N(0, 1), rounded to bf16, so tau <q, k> = -512 plus a
spread of several units (c = 0.5) or exactly -512 for every pair (c = 0, a
uniform softmax over the visible keys). Checked against oracle.prefill_bshd /
prefill_thd and oracle.context_parallel.shard_attention with rotate_qk=False.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd.workloads import far_below
from helpers import assert_close, np64, say
from oracle import context_parallel as cp

pytestmark = pytest.mark.gpu
TAU = 0.125
U = 2.0 ** -8


def _check_lse(got, ref, what):
    g = np64(got).reshape(ref.shape)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(g), inf), f"{what}: -inf rows differ"
    err = float(np.abs(g[~inf] - ref[~inf]).max()) if (~inf).any() else 0.0
    say(f"  {what} lse: max_abs={err:.3e}")
    assert err <= U + 1e-4, f"{what}: lse error {err}"


@pytest.mark.parametrize("spread", [0.0, 0.5])
@pytest.mark.parametrize("window", [0, 128])
def test_bshd_no_sink_far_below_zero(window, spread):
    q, k, v = far_below((2, 300), (2, 300), spread, seed=800 + window)
    sinks = torch.full((64,), -float("inf"))
    say(f"[gpu] no sink, logits near -512: bshd B=2 S=300 W={window} spread={spread}")
    out, lse = gx.attn_prefill_lse(q.cuda(), k.cuda(), v.cuda(), sinks.cuda(), window=window)
    ref = oracle.prefill_bshd(np64(q), np64(k), np64(v), np64(sinks), TAU, window, rotate_qk=False)
    assert_close(out, ref, f"bshd W={window}")
    # the same rows through the call without the LSE output
    assert torch.equal(gx.attn_prefill(q.cuda(), k.cuda(), v.cuda(), sinks.cuda(), window=window), out)
    _, rl = cp.shard_attention(np64(q), np64(k), np64(v), TAU, window, 0, 0, rotate_qk=False)
    _check_lse(lse, rl, f"bshd W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_mixed_sinks_far_below_zero(window):
    """Heads with sigma = -inf next to heads with a finite sigma in the same GQA group and wave."""
    q, k, v = far_below((1, 200), (1, 200), 0.5, seed=810 + window)
    sinks = torch.where(torch.arange(64) % 3 == 0, torch.tensor(-float("inf")), torch.linspace(-600.0, 0.0, 64))
    say(f"[gpu] mixed sinks, logits near -512: W={window}")
    out = gx.attn_prefill(q.cuda(), k.cuda(), v.cuda(), sinks.cuda(), window=window)
    ref = oracle.prefill_bshd(np64(q), np64(k), np64(v), np64(sinks), TAU, window, rotate_qk=False)
    assert_close(out, ref, f"mixed sinks W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_thd_no_sink_far_below_zero(window):
    lengths = [37, 0, 300, 129, 1]
    T = sum(lengths)
    q, k, v = far_below((T,), (T,), 0.5, seed=820 + window)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    sinks = torch.full((64,), -float("inf"))
    say(f"[gpu] no sink, logits near -512: thd W={window}")
    out = gx.attn_prefill(q.cuda(), k.cuda(), v.cuda(), sinks.cuda(), window=window, cu_seqlens=cu.cuda(),
                          max_seqlen=max(lengths))
    ref = oracle.prefill_thd(np64(q), np64(k), np64(v), cu.numpy(), np64(sinks), TAU, window, rotate_qk=False)
    assert_close(out, ref, f"thd W={window}")


@pytest.mark.parametrize("Sq,Sk,qo,ko,window", [
    (128, 128, 256, 256, 0),      # the diagonal block of a ring
    (100, 77, 500, 100, 0),       # every key visible, ragged sizes
    (96, 160, 300, 200, 128),     # window: a band of the keys
    (200, 300, 250, 0, 64),       # window starting inside the shard
])
def test_shard_far_below_zero(Sq, Sk, qo, ko, window):
    """A shard never has a sink term: its o and lse against the oracle."""
    q, k, v = far_below((2, Sq), (2, Sk), 0.5, seed=830 + Sq + Sk)
    say(f"[gpu] shard, logits near -512: Sq={Sq} Sk={Sk} q_offset={qo} kv_offset={ko} W={window}")
    out, lse = gx.attn_prefill_shard(q.cuda(), k.cuda(), v.cuda(), qo, ko, window=window)
    ro, rl = cp.shard_attention(np64(q), np64(k), np64(v), TAU, window, qo, ko, rotate_qk=False)
    assert_close(out, ro, "shard o")
    _check_lse(lse, rl, "shard")


@pytest.mark.parametrize("window", [0, 128])
def test_ring_far_below_zero(window):
    """Two contiguous shards per query shard, merged with a -inf sink, equal the prefill definition."""
    S = 512
    q, k, v = far_below((1, S), (1, S), 0.5, seed=840 + window)
    sinks = torch.full((64,), -float("inf"))
    qc, kc, vc, sc = q.cuda(), k.cuda(), v.cuda(), sinks.cuda()
    ref = oracle.prefill_bshd(np64(q), np64(k), np64(v), np64(sinks), TAU, window, rotate_qk=False)
    say(f"[gpu] ring of 2 shards, logits near -512, W={window}")
    for lo, hi in ((0, 256), (256, 512)):
        parts_o, parts_l = [], []
        for a, b in ((0, 256), (256, 512)):
            o, l = gx.attn_prefill_shard(qc[:, lo:hi].contiguous(), kc[:, a:b].contiguous(),
                                         vc[:, a:b].contiguous(), lo, a, window=window)
            parts_o.append(o.reshape(-1, 64, 64))
            parts_l.append(l.reshape(-1))
        merged = gx.attn_merge(torch.stack(parts_o), torch.stack(parts_l), sc)
        assert_close(merged.reshape(1, hi - lo, 64, 64), ref[:, lo:hi], f"ring rows {lo}..{hi - 1}")
