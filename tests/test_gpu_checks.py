"""GPU test of gptoss_check_lengths, the device-side check of the lengths the attention
calls trust: THD offsets (cu_seqlens starting at 0, non-decreasing, ending at the token
count; the packed-sequence format of the rope_utils page's apply_rotary_emb_qk) and decode
cache lengths (1 .. max_cache_len). The expected bits and first indices come from the rules
written out in Python below, applied to the same arrays."""

import pytest
import torch

import attention_yarn_rope_amd as gx
from helpers import say

pytestmark = pytest.mark.gpu
F = gx.LENGTH_FAULTS


def _expect(cu, total, cl, max_len):
    mask, first_cu, first_cl = 0, -1, -1
    if cu is not None:
        for i, v in enumerate(cu):
            bad = 0
            if i == 0 and v != 0:
                bad |= F["cu_start"]
            if i > 0 and v < cu[i - 1]:
                bad |= F["cu_order"]
            if i == len(cu) - 1 and total >= 0 and v != total:
                bad |= F["cu_total"]
            if bad:
                mask |= bad
                first_cu = i if first_cu < 0 else first_cu
    if cl is not None:
        for i, v in enumerate(cl):
            if v < 1 or v > max_len:
                mask |= F["cache"]
                first_cl = i if first_cl < 0 else first_cl
    return [mask, first_cu, first_cl]


def _run(cu, total, cl, max_len):
    t_cu = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    t_cl = torch.tensor(cl, dtype=torch.int32, device="cuda") if cl is not None else None
    return gx.check_lengths(t_cu, total, t_cl, max_len).cpu().tolist()


CU_CASES = [
    ([0, 37, 38, 38, 338, 466], 466),          # valid, with an empty sequence
    ([0], 0),                                  # no sequences
    ([1, 37, 38], 38),                         # does not start at 0
    ([0, 37, 20, 40], 40),                     # decreases at index 2
    ([0, 10, 20], 25),                         # ends before the token count
    ([0, 10, 20], -1),                         # total not checked
    ([5, 3, 2, 9], 10),                        # every rule broken
]


@pytest.mark.parametrize("cu,total", CU_CASES)
def test_cu_seqlens_rules(cu, total):
    say(f"[gpu] check_lengths cu={cu} total={total}")
    assert _run(cu, total, None, 1) == _expect(cu, total, None, 1)


def test_cu_seqlens_long_array():
    """More entries than the kernel's threads: a decrease near the end is still found."""
    cu = list(range(0, 3 * 4096, 3))
    cu[3000] = cu[2999] - 1
    say("[gpu] check_lengths long cu_seqlens")
    got = _run(cu, cu[-1], None, 1)
    assert got == _expect(cu, cu[-1], None, 1) and got[1] == 3000


@pytest.mark.parametrize("cl,max_len", [([1, 1024, 17], 1024), ([0, 5, 2000, 7], 1024), ([3, -4], 8),
                                         ([], 8)])
def test_cache_seqlens_rules(cl, max_len):
    say(f"[gpu] check_lengths cache={cl} max={max_len}")
    assert _run(None, -1, cl, max_len) == _expect(None, -1, cl, max_len)


def test_both_arrays_and_the_workload_lengths():
    """Both arrays in one call, and the lengths of the THD and decode workloads pass."""
    from attention_yarn_rope_amd import workloads as wl
    thd = wl.prefill_thd(0, 0, 0, seed=3, lengths=[128, 4096, 300, 8192])
    cu, cl = thd.cu_seqlens.tolist(), [int(x) for x in wl.decode64_lengths()]
    say("[gpu] check_lengths workloads")
    assert _run(cu, cu[-1], cl, 32768) == [0, -1, -1]
    bad_cl = list(cl)
    bad_cl[40] = 32769
    assert _run([0, 5, 3], 3, bad_cl, 32768) == [F["cu_order"] | F["cache"], 2, 40]
