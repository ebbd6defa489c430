"""Parity at the full workload sizes, in the launch configuration bench.py times.

The GPU computes every output; the oracle recomputes seeded samples of them one
row (query token, all heads) at a time:
  * dense BSHD prefill B=4, S=4096, full-causal and window-128: in batch 0 every row on
    either side of a 32-row boundary (31, 32, 63, 64, ..., 4095) plus 64 seeded rows, in
    batches 1-3 64 seeded rows each;
  * packed THD prefill, 16 sequences with lengths uniform in [128, 8192];
  * long-context prefill B=1, S=131072: the 512 sampled rows (0, 1, 127, 128, 131071 and
    the first 507 other entries of a seeded permutation), both layers;
  * decode, 64 sequences with cache lengths uniform in [1024, 32768] (all rows).
Tolerance as in helpers.py.
"""

import numpy as np
import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
TAU = 0.125


def _rows(S, n, seed, must=()):
    rng = np.random.default_rng(seed)
    r = set(int(x) for x in must if 0 <= x < S)
    r.update(int(x) for x in rng.choice(S, size=min(n, S), replace=False))
    return np.array(sorted(r))


class _Rows:
    """Indexable view of a CPU bf16 tensor that converts only the requested rows to fp64."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return np64(self.t[torch.as_tensor(np.asarray(idx))])


def _check_rows(out, q, k, v, sinks, window, rows, what, positions=None):
    """out/q/k/v: one sequence ([S, H, D] tensors on CPU); rows: indices into it."""
    ref = oracle.prefill_rows(_Rows(q), _Rows(k), _Rows(v), np64(sinks), TAU, window, rows, positions=positions)
    assert_close(out[rows], ref, what)


@pytest.mark.parametrize("window", [0, 128])
def test_dense_bshd(window):
    say(f"[gpu] dense B=4 S=4096 window={window}")
    inp = wl.dense()
    table = gx.rope_table(4096)
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window,
                          table=table).cpu()
    edges = [r for m in range(0, 4096 + 32, 32) for r in (m - 1, m)]   # both sides of every 32-row boundary
    for b in range(4):
        rows = _rows(4096, 64, 100 + b, must=edges if b == 0 else ())
        say(f"  batch {b}: {len(rows)} rows")
        _check_rows(out[b], inp.q[b], inp.k[b], inp.v[b], inp.sinks, window, rows, f"dense b={b} W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_thd_16_sequences(window):
    say(f"[gpu] THD 16 sequences window={window}")
    inp = wl.thd()
    assert inp.q.shape[0] == sum(inp.lengths)
    table = gx.rope_table(8192)
    out = gx.attn_prefill(inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda(), window=window, table=table,
                          cu_seqlens=inp.cu_seqlens.cuda(), max_seqlen=inp.max_seqlen).cpu()
    cu = inp.cu_seqlens.tolist()
    for n, L in enumerate(inp.lengths):
        a, b = cu[n], cu[n + 1]
        rows = _rows(L, 3, 200 + n, must=(0, L - 1))
        _check_rows(out[a:b], inp.q[a:b], inp.k[a:b], inp.v[a:b], inp.sinks, window, rows,
                    f"thd seq {n} (L={L}) W={window}")


@pytest.fixture(scope="module")
def long_outputs():
    """Both layers of the 131072-token sequence on the GPU; the sampled rows of their outputs."""
    say("[gpu] long S=131072: both layers")
    inp = wl.long_context()
    table = gx.rope_table(131072)
    q, k, v, s = inp.q.cuda(), inp.k.cuda(), inp.v.cuda(), inp.sinks.cuda()
    rows = np.array(wl.long_context_rows())
    outs = {w: gx.attn_prefill(q, k, v, s, window=w, table=table)[0][torch.as_tensor(rows).cuda()].cpu()
            for w in (0, 128)}
    del q, k, v, s
    return inp, rows, outs


def test_long_context_window(long_outputs):
    """Window-128 layer: all 512 sampled rows, one oracle call per row (each sees 128 keys)."""
    inp, rows, outs = long_outputs
    say("  window=128, 512 rows")
    ref = np.concatenate([oracle.prefill_rows(_Rows(inp.q[0]), _Rows(inp.k[0]), _Rows(inp.v[0]), np64(inp.sinks),
                                              TAU, 128, [r]) for r in rows])
    assert_close(outs[128], ref, "long W=128 (512 rows)")


def test_long_context_full(long_outputs):
    """Full-causal layer: all 512 sampled rows in one oracle call (each sees up to 131072 keys)."""
    inp, rows, outs = long_outputs
    say("  window=0, 512 rows")
    ref = oracle.prefill_rows(_Rows(inp.q[0]), _Rows(inp.k[0]), _Rows(inp.v[0]), np64(inp.sinks), TAU, 0, rows)
    assert_close(outs[0], ref, "long W=0 (512 rows)")


def test_over_2g_elements():
    """B=4, S=131072: q and the output hold 2^31 elements each (4 GiB), past any 32-bit element
    offset. The inputs are drawn on the GPU from a seeded generator; sampled rows of the last
    sequence (the largest offsets) are checked against the oracle for the window layer (64 rows)
    and the full-causal layer (8 rows)."""
    B, S = 4, 131072
    g = torch.Generator(device="cuda").manual_seed(77)

    def draw(shape):
        t = torch.empty((B,) + shape, dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            t[b] = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        return t

    q, k, v = draw((S, 64, 64)), draw((S, 8, 64)), draw((S, 8, 64))
    s = torch.randn(64, generator=g, device="cuda", dtype=torch.float32)
    assert q.numel() == 2 ** 31
    table = gx.rope_table(S)
    rows = [0, 1, 127, 128, 65536, S - 1] + torch.randperm(S, generator=torch.Generator().manual_seed(78))[:58].tolist()
    rows = np.array(sorted(set(rows)))
    q3, k3, v3, s3 = q[3].cpu(), k[3].cpu(), v[3].cpu(), s.cpu()
    say("[gpu] B=4 S=131072 (2^31-element q) window=128")
    out = gx.attn_prefill(q, k, v, s, window=128, table=table)
    _check_rows(out[3].cpu(), q3, k3, v3, s3, 128, rows, "B=4 S=131072 W=128, last sequence")
    del out
    say("[gpu] B=4 S=131072 (2^31-element q) window=0")
    out = gx.attn_prefill(q, k, v, s, window=0, table=table)
    _check_rows(out[3].cpu(), q3, k3, v3, s3, 0, rows[[0, 1, 2, 3, 4, -3, -2, -1]], "B=4 S=131072 W=0, last sequence")


@pytest.mark.parametrize("window", [0, 128])
def test_decode_64_sequences(window):
    say(f"[gpu] decode 64 sequences window={window}")
    inp = wl.decode64()
    table = gx.rope_table(32768)
    out = gx.attn_decode(inp.q.cuda(), inp.k_cache.cuda(), inp.v_cache.cuda(), inp.cache_seqlens.cuda(),
                         inp.sinks.cuda(), window=window, table=table).cpu()
    ref = np.zeros((64, 64, 64))
    for n, L in enumerate(inp.lengths):
        ref[n] = oracle.decode(np64(inp.q[n:n + 1]), np64(inp.k_cache[n:n + 1, :L]), np64(inp.v_cache[n:n + 1, :L]),
                               [L], np64(inp.sinks), TAU, window)[0]
    assert_close(out, ref, f"decode64 W={window}")
