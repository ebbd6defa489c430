"""GPU checks of gptoss_attn_decode_kv_noalloc, the decode entry point that
allocates nothing (its split partials and plan live in a fixed per-GPU scratch
array inside the library), against gptoss_attn_decode_kv with a workspace and
against oracle.kvcache, through the C ABI.

Calls run back to back on the one scratch array, each followed by a smaller
one, so a call that read a previous call's partials or plan would show. Where
the default split plan fits the scratch the two entry points run the same
kernels on the same plan and must agree bit for bit; where the scratch forces
longer splits the result is checked against the oracle with the elementwise
tolerance of helpers.py.
"""

import pytest
import torch

import attention_yarn_rope_amd as gx
import oracle
from attention_yarn_rope_amd import workloads as wl
from helpers import assert_close, np64, say
from oracle import kvcache as kv

pytestmark = pytest.mark.gpu
CFG = oracle.RopeConfig()
TAU = 0.125


@pytest.fixture(scope="module")
def table():
    return gx.rope_table(8192)


def _paged(w):
    return dict(kind="paged", block_table=w.block_table.cuda())


def _ref(w, window):
    lay = kv.KVLayout(kv.PAGED, w.k_pool.shape[1], w.block_table.numpy())
    return kv.decode(lay, np64(w.q), w.k_pool.float().numpy(), w.v_pool.float().numpy(), w.lengths, np64(w.sinks),
                     TAU, window, CFG)


def _both(w, table, window, max_seqlen, splits=0):
    q, kp, vp, lens, s = w.q.cuda(), w.k_pool.cuda(), w.v_pool.cuda(), w.cache_seqlens.cuda(), w.sinks.cuda()
    a = gx.attn_decode_kv_noalloc(q, kp, vp, lens, s, window=window, table=table, max_seqlen=max_seqlen,
                                  num_splits=splits, **_paged(w))
    b = gx.attn_decode_kv(q, kp, vp, lens, s, window=window, table=table, max_seqlen=max_seqlen,
                          num_splits=splits, **_paged(w))
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("window", [0, 128])
def test_two_calls_second_smaller(table, window):
    """A larger and then a smaller paged decode: bit-identical to the workspace entry point."""
    big = wl.paged_decode([5000, 1, 4096, 33, 2500, 700, 3000, 6000, 128, 129, 4097, 1500], 64, seed=900 + window)
    small = wl.paged_decode([300, 17, 1025], 64, seed=901 + window)
    for name, w, ms in (("large", big, 6000), ("smaller", small, 1025)):
        say(f"[gpu] no-alloc decode, {name} call, W={window}, {len(w.lengths)} sequences")
        a, b = _both(w, table, window, ms)
        assert torch.equal(a, b), f"{name}: differs from gptoss_attn_decode_kv"
        assert_close(a, _ref(w, window), f"no-alloc {name} W={window}")


def test_fixed_split_counts_back_to_back(table):
    """Caller-given split counts, largest first: each call reads only the partials it wrote."""
    w = wl.paged_decode([4096, 100, 2000, 3333], 64, seed=910)
    ref = _ref(w, 0)
    for splits in (8, 3, 1):
        say(f"[gpu] no-alloc decode, num_splits={splits}")
        a, b = _both(w, table, 0, 4096, splits)
        assert torch.equal(a, b), f"num_splits={splits}: differs from gptoss_attn_decode_kv"
        assert_close(a, ref, f"no-alloc splits={splits}")


def test_scratch_lengthens_splits(table):
    """256 sequences declared up to 4096 keys: the default plan's partials (34.6 MB) exceed the
    32 MiB scratch, so the shortest split grows from 512 to 640 keys. Then a smaller call."""
    g = torch.Generator().manual_seed(920)
    lengths = torch.randint(1, 1501, (256,), generator=g).tolist()
    w = wl.paged_decode(lengths, 64, seed=921)
    bt = torch.zeros((256, 64), dtype=torch.int32)   # room for 4096 keys; entries past a sequence's pages name page 0
    bt[:, :w.block_table.shape[1]] = w.block_table
    w.block_table = bt
    say("[gpu] no-alloc decode, 256 sequences, max_seqlen 4096 (longer splits than the workspace call)")
    a, b = _both(w, table, 0, 4096)
    ref = _ref(w, 0)
    assert_close(a, ref, "no-alloc 256 sequences")
    assert_close(b, ref, "workspace 256 sequences")
    small = wl.paged_decode([900, 2, 64], 64, seed=922)
    say("[gpu] no-alloc decode, smaller call after it")
    a, b = _both(small, table, 0, 900)
    assert torch.equal(a, b)
    assert_close(a, _ref(small, 0), "no-alloc after the large call")


def test_rejects_what_cannot_fit(table):
    """2048 sequences x 64 heads need 34.6 MB of partials even with one split each: the call is
    refused before any launch and leaves the output untouched."""
    N = 2048
    q = torch.zeros((N, 64, 64), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((N, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(N, dtype=torch.int32, device="cuda")
    out = torch.full((N, 64, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gx.GptossError) as e:
        gx.attn_decode_kv_noalloc(q, kc, kc, lens, torch.zeros(64, device="cuda"), table=table, out=out)
    assert e.value.status == 4   # GPTOSS_ERR_WORKSPACE
    assert torch.all(out == 7.0)
