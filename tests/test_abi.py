"""CPU checks of the C ABI: the library loads, exports every declared symbol,
computes the host-side YaRN parameters exactly like the oracle, and rejects bad
arguments with the documented status codes before launching anything.

No call here reaches a kernel launch (each returns on argument checks first):
the argument checks pass fake device pointers, so they are skipped where a GPU
is visible, and every call's status is checked against GPTOSS_ERR_HIP (what a
launch attempt returns on a host without a GPU).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from attention_yarn_rope_amd import _lib
from attention_yarn_rope_amd._lib import I64x2, I64x3, KVLayout, RopeConfig, SeqDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptoss_attn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4, 5


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


class _NoLaunch:
    """The library with every status-returning call checked: GPTOSS_ERR_HIP means the call got
    past its argument checks to a kernel launch, which a fake-pointer check must never do."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(self._lib, name)
        if not name.startswith("gptoss_") or fn.restype is not ctypes.c_int:
            return fn

        def call(*args):
            st = fn(*args)
            assert st != ERR_HIP, f"{name} got past its argument checks to a kernel launch"
            return st
        return call


def _load():
    if not os.path.exists(_lib.LIB_PATH):
        from attention_yarn_rope_amd import build
        build.build(verbose=False)
    return _lib.load()


@pytest.fixture(scope="module")
def real_lib():
    return _load()


@pytest.fixture(scope="module")
def lib():
    if _gpu_visible():
        pytest.skip("argument checks with fake device pointers run on a host without a GPU")
    return _NoLaunch(_load())


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptoss_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(real_lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(real_lib, n), f"{n} declared in gptoss_attn.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version_and_strings(real_lib):
    assert real_lib.gptoss_abi_version() == 6
    for code in range(6):
        assert real_lib.gptoss_status_string(code)
    assert real_lib.gptoss_status_string(99) == b"unknown status"


def _cfg(**kw):
    base = dict(head_dim=64, rotary_dim=64, base=150000.0, scaling_factor=32.0, initial_context_length=4096,
                ntk_alpha=1.0, ntk_beta=32.0)
    base.update(kw)
    return RopeConfig(**base)


@pytest.mark.parametrize("kw", [{}, {"scaling_factor": 1.0}, {"base": 10000.0, "scaling_factor": 4.0},
                                {"rotary_dim": 32}])
def test_yarn_params_match_oracle_exactly(lib, kw):
    c = _cfg(**kw)
    n = c.rotary_dim // 2
    om = (ctypes.c_double * n)()
    conc = ctypes.c_double()
    assert lib.gptoss_yarn_params(ctypes.byref(c), om, ctypes.byref(conc)) == OK
    ref_om, ref_c, _ = oracle.yarn_params(oracle.RopeConfig(**kw))
    assert np.array_equal(np.array(list(om)), ref_om)
    assert conc.value == ref_c


def test_yarn_param_errors(lib):
    om = (ctypes.c_double * 32)()
    assert lib.gptoss_yarn_params(None, om, None) == ERR_NULL
    assert lib.gptoss_yarn_params(ctypes.byref(_cfg(rotary_dim=63)), om, None) == ERR_SHAPE
    assert lib.gptoss_yarn_params(ctypes.byref(_cfg(rotary_dim=128)), om, None) == ERR_SHAPE
    assert lib.gptoss_yarn_params(ctypes.byref(_cfg(ntk_beta=0.5)), om, None) == ERR_SHAPE
    assert b"ntk" in lib.gptoss_last_error()


def test_table_init_errors(lib):
    assert lib.gptoss_rope_table_init(ctypes.byref(_cfg()), 10, None, None) == ERR_NULL
    fake = ctypes.c_void_p(0x1000)
    assert lib.gptoss_rope_table_init(ctypes.byref(_cfg()), 0, fake, None) == ERR_SHAPE
    assert lib.gptoss_rope_table_init(ctypes.byref(_cfg(rotary_dim=7)), 10, fake, None) == ERR_SHAPE


def _desc(**kw):
    d = dict(layout=0, batch=2, seqlen=128, max_seqlen=128, cu_seqlens=None, num_q_heads=64, num_kv_heads=8,
             head_dim=64)
    d.update(kw)
    return SeqDesc(**d)


P = ctypes.c_void_p(0x10000)     # aligned fake device pointers: never dereferenced on these paths
S3 = I64x3(128 * 64 * 64, 64 * 64, 64)
K3 = I64x3(128 * 8 * 64, 8 * 64, 64)


def _prefill(lib, desc, **kw):
    a = dict(q=P, qs=S3, k=P, ks=K3, v=P, vs=K3, sinks=P, scale=0.125, window=0, table=P, rows=4096, rd=64,
             out=P, os=S3, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.gptoss_attn_prefill(ctypes.byref(desc) if desc is not None else None, a["q"], a["qs"], a["k"],
                                   a["ks"], a["v"], a["vs"], a["sinks"], a["scale"], a["window"], a["table"],
                                   a["rows"], a["rd"], a["out"], a["os"], a["ws"], a["wsb"], None)


def test_prefill_argument_errors(lib):
    d = _desc()
    assert _prefill(lib, None) == ERR_NULL
    assert _prefill(lib, _desc(head_dim=128)) == ERR_UNSUPPORTED
    assert _prefill(lib, _desc(num_q_heads=60)) == ERR_UNSUPPORTED
    assert _prefill(lib, _desc(layout=7)) == ERR_SHAPE
    assert _prefill(lib, _desc(layout=1, batch=2, seqlen=100, max_seqlen=50)) == ERR_NULL   # no cu_seqlens
    assert _prefill(lib, d, q=None) == ERR_NULL
    assert _prefill(lib, d, window=-1) == ERR_SHAPE
    assert _prefill(lib, d, scale=float("nan")) == ERR_SHAPE
    assert _prefill(lib, d, scale=-0.125) == ERR_SHAPE
    assert _prefill(lib, d, scale=0.0, wsb=16) == ERR_WORKSPACE     # 0 = head_dim ** -0.5: passes the check
    assert _prefill(lib, d, rd=24) == ERR_UNSUPPORTED             # not a multiple of 16
    assert _prefill(lib, d, rows=100) == ERR_SHAPE               # table shorter than the sequence
    assert _prefill(lib, d, qs=I64x3(128 * 64 * 64, 64 * 64, 65)) == ERR_UNSUPPORTED   # misaligned stride
    assert _prefill(lib, d, q=ctypes.c_void_p(0x10002)) == ERR_UNSUPPORTED             # misaligned pointer
    assert _prefill(lib, d, wsb=16) == ERR_WORKSPACE
    assert _prefill(lib, d, ws=None) == ERR_WORKSPACE
    assert _prefill(lib, d, ws=ctypes.c_void_p(0x10010)) == ERR_WORKSPACE               # not 256-byte aligned
    assert _prefill(lib, _desc(batch=0)) == OK                   # nothing to do, nothing launched


def test_prefill_workspace_size(lib):
    d = _desc(batch=4, seqlen=4096, max_seqlen=4096)
    assert lib.gptoss_attn_prefill_workspace_size(ctypes.byref(d)) == 4 * 4096 * 8 * 64 * 2
    t = _desc(layout=1, batch=16, seqlen=65171, max_seqlen=8179, cu_seqlens=P)
    ws = lib.gptoss_attn_prefill_workspace_size(ctypes.byref(t))
    assert ws >= 65171 * 8 * 64 * 2 + ((65171 + 31) // 32 + 16) * 8
    assert lib.gptoss_attn_prefill_workspace_size(ctypes.byref(_desc(head_dim=80))) == 0


def _decode(lib, **kw):
    a = dict(n=4, hq=64, hkv=8, d=64, q=P, qs=I64x2(64 * 64, 64), k=P, v=P, kvs=I64x3(1024 * 8 * 64, 8 * 64, 64),
             lens=P, lmax=1024, sinks=P, scale=0.125, window=0, table=P, rows=1024, rd=64, out=P,
             os=I64x2(64 * 64, 64), ws=P, wsb=1 << 30, splits=0)
    a.update(kw)
    return lib.gptoss_attn_decode(a["n"], a["hq"], a["hkv"], a["d"], a["q"], a["qs"], a["k"], a["v"], a["kvs"],
                                  a["lens"], a["lmax"], a["sinks"], a["scale"], a["window"], a["table"], a["rows"],
                                  a["rd"], a["out"], a["os"], a["ws"], a["wsb"], a["splits"], None)


def test_decode_argument_errors(lib):
    assert _decode(lib, d=128) == ERR_UNSUPPORTED
    assert _decode(lib, hq=32) == ERR_UNSUPPORTED
    assert _decode(lib, lmax=0) == ERR_SHAPE
    assert _decode(lib, splits=-1) == ERR_SHAPE
    assert _decode(lib, window=-5) == ERR_SHAPE
    assert _decode(lib, lens=None) == ERR_NULL
    assert _decode(lib, rows=1000) == ERR_SHAPE
    assert _decode(lib, wsb=8) == ERR_WORKSPACE
    assert _decode(lib, kvs=I64x3(1024 * 8 * 64, 8 * 64, 63)) == ERR_UNSUPPORTED
    assert _decode(lib, n=0) == OK


def test_decode_workspace_size(lib):
    # 64 sequences x 64 heads x ceil(32768 / 512) splits x (64 + 2) floats, plus the
    # split plan: 2 ints and one (sequence, split) int pair per item, rounded to 256 bytes
    ws = lib.gptoss_attn_decode_workspace_size(64, 64, 32768, 0)
    plan = (2 * 4 + 64 * 64 * 8 + 255) // 256 * 256
    assert ws == 64 * 64 * 64 * 64 * 4 + 64 * 64 * 64 * 2 * 4 + plan
    assert lib.gptoss_attn_decode_workspace_size(2, 64, 1000, 3) >= 2 * 64 * 3 * 66 * 4
    assert lib.gptoss_attn_decode_workspace_size(2, 64, 0, 0) == 0


def test_rope_qk_argument_errors(lib):
    d = _desc()
    f = lib.gptoss_rope_qk
    assert f(ctypes.byref(d), P, S3, P, K3, P, P, None, 4096, 64, None) == ERR_NULL
    assert f(ctypes.byref(d), P, S3, P, K3, P, P, P, 10, 64, None) == ERR_SHAPE
    assert f(ctypes.byref(_desc(head_dim=32)), P, S3, P, K3, P, P, P, 4096, 64, None) == ERR_UNSUPPORTED
    assert f(ctypes.byref(_desc(seqlen=0)), P, S3, P, K3, P, P, P, 4096, 64, None) == OK
    for rd in (8, 24, 40, 66):   # partial rotary: multiples of 16 only
        assert f(ctypes.byref(d), P, S3, P, K3, P, P, P, 4096, rd, None) == ERR_UNSUPPORTED


def test_attention_rotary_dims(lib):
    # the attention calls rotate 16, 32, 48 or 64 dims; other widths are refused before any launch
    assert _prefill(lib, _desc_bshd(), rd=24) == ERR_UNSUPPORTED
    assert _prefill(lib, _desc_bshd(), rd=80) == ERR_UNSUPPORTED
    assert _decode(lib, rd=8) == ERR_UNSUPPORTED
    # 32 passes the table check (the call then stops at the too-small workspace)
    assert _prefill(lib, _desc_bshd(), rd=32, wsb=16) == ERR_WORKSPACE
    assert _decode(lib, rd=32, wsb=16) == ERR_WORKSPACE
    # the gradients rotate back all 64 dims only
    assert _backward(lib, _desc_bshd(), rd=32) == ERR_UNSUPPORTED


def test_prefill_ex_rejects_unknown_k_rotation(lib):
    d = _desc()
    st = lib.gptoss_attn_prefill_ex(ctypes.byref(d), P, S3, P, K3, P, K3, P, 0.125, 0, P, 4096, 64, P, S3, P,
                                    1 << 30, 9, None)
    assert st == ERR_SHAPE


def _desc_bshd(B=2, S=128):
    return SeqDesc(0, B, S, S, None, 64, 8, 64)


def _backward(lib, desc, **kw):
    a = dict(q=P, qs=I64x3(128 * 64 * 64, 64 * 64, 64), k=P, ks=I64x3(128 * 8 * 64, 8 * 64, 64), v=P,
             vs=I64x3(128 * 8 * 64, 8 * 64, 64), sinks=P, scale=0.125, window=0, table=P, rows=128, rd=64,
             out=P, os=I64x3(128 * 64 * 64, 64 * 64, 64), dout=P, dos=I64x3(128 * 64 * 64, 64 * 64, 64), lse=P,
             dq=P, dk=P, dv=P, ds=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.gptoss_attn_prefill_backward(ctypes.byref(desc) if desc is not None else None, a["q"], a["qs"],
                                            a["k"], a["ks"], a["v"], a["vs"], a["sinks"], a["scale"], a["window"],
                                            a["table"], a["rows"], a["rd"], a["out"], a["os"], a["dout"], a["dos"],
                                            a["lse"], a["dq"], a["dk"], a["dv"], a["ds"], a["ws"], a["wsb"], None)


def test_backward_argument_errors(lib):
    d = _desc_bshd()
    assert _backward(lib, None) == ERR_NULL
    assert _backward(lib, _desc_bshd(), ds=None) == ERR_NULL
    assert _backward(lib, d, dout=None) == ERR_NULL
    assert _backward(lib, d, lse=None) == ERR_NULL
    assert _backward(lib, d, window=-1) == ERR_SHAPE
    assert _backward(lib, d, scale=-0.125) == ERR_SHAPE
    assert _backward(lib, d, scale=float("inf")) == ERR_SHAPE
    assert _backward(lib, d, scale=0.0, wsb=16) == ERR_WORKSPACE     # 0 = head_dim ** -0.5: passes the check
    assert _backward(lib, d, rows=100) == ERR_SHAPE                     # table shorter than the sequence
    assert _backward(lib, d, dos=I64x3(128 * 64 * 64, 64 * 64, 65)) == ERR_UNSUPPORTED
    assert _backward(lib, d, lse=ctypes.c_void_p(0x10004)) == ERR_UNSUPPORTED
    assert _backward(lib, d, wsb=16) == ERR_WORKSPACE
    assert _backward(lib, SeqDesc(0, 2, 128, 128, None, 64, 8, 128)) == ERR_UNSUPPORTED   # head_dim 128


def test_backward_workspace_size(lib):
    d = _desc_bshd(4, 4096)
    T = 4 * 4096
    # rotated q and k, (lse, -D) per row and head, one dsigma partial per head and dq work item (4 x 128)
    assert lib.gptoss_attn_prefill_backward_workspace_size(ctypes.byref(d)) == (
        T * 64 * 64 * 2 + T * 8 * 64 * 2 + 2 * T * 64 * 4 + 4 * 128 * 64 * 4)
    t = SeqDesc(1, 16, 65171, 8179, P, 64, 8, 64)
    ws = lib.gptoss_attn_prefill_backward_workspace_size(ctypes.byref(t))
    assert ws >= 65171 * (64 * 64 * 2 + 8 * 64 * 2 + 2 * 64 * 4) + ((65171 + 31) // 32 + 16) * 8
    assert lib.gptoss_attn_prefill_backward_workspace_size(ctypes.byref(SeqDesc(0, 1, 8, 8, None, 60, 8, 64))) == 0


def test_prefill_lse_requires_lse(lib):
    d = _desc_bshd()
    st = lib.gptoss_attn_prefill_lse(ctypes.byref(d), P, I64x3(128 * 64 * 64, 64 * 64, 64), P,
                                     I64x3(128 * 8 * 64, 8 * 64, 64), P, I64x3(128 * 8 * 64, 8 * 64, 64), P, 0.125, 0,
                                     P, 128, 64, P, I64x3(128 * 64 * 64, 64 * 64, 64), None, P, 1 << 30, None)
    assert st == ERR_NULL


def _layout(kind=0, cap=1024, strides=(1024 * 8 * 64, 8 * 64, 64), bt=None, max_pages=0, num_pages=0):
    lay = KVLayout()
    lay.kind, lay.capacity, lay.strides = kind, cap, I64x3(*strides)
    lay.block_table, lay.max_pages, lay.num_pages = bt, max_pages, num_pages
    return lay


def _append(lib, lay, **kw):
    a = dict(k=P, v=P, n=4, hkv=8, d=64, t=1, kn=P, kns=I64x3(8 * 64, 8 * 64, 64), vn=P, vns=I64x3(8 * 64, 8 * 64, 64),
             lens=P, maxlen=1024, table=P, rows=1024, rd=64)
    a.update(kw)
    return lib.gptoss_kv_append(ctypes.byref(lay) if lay is not None else None, a["k"], a["v"], a["n"], a["hkv"],
                                a["d"], a["t"], a["kn"], a["kns"], a["vn"], a["vns"], a["lens"], a["maxlen"],
                                a["table"], a["rows"], a["rd"], None)


def test_kv_append_argument_errors(lib):
    assert _append(lib, None) == ERR_NULL
    assert _append(lib, _layout(kind=3)) == ERR_SHAPE
    assert _append(lib, _layout(cap=0)) == ERR_SHAPE
    assert _append(lib, _layout(), d=128) == ERR_UNSUPPORTED
    assert _append(lib, _layout(), t=-1) == ERR_SHAPE
    assert _append(lib, _layout(strides=(1024 * 8 * 64, 8 * 64, 65))) == ERR_UNSUPPORTED
    assert _append(lib, _layout(kind=1, cap=48, bt=P, max_pages=4, num_pages=8)) == ERR_UNSUPPORTED   # page size
    assert _append(lib, _layout(kind=1, cap=16, bt=P, max_pages=4, num_pages=8)) == ERR_UNSUPPORTED   # below 32
    assert _append(lib, _layout(kind=1, cap=64, bt=None, max_pages=4, num_pages=8)) == ERR_NULL
    assert _append(lib, _layout(kind=1, cap=64, bt=P, max_pages=0, num_pages=8)) == ERR_SHAPE
    assert _append(lib, _layout(), kn=None) == ERR_NULL
    assert _append(lib, _layout(), lens=None) == ERR_NULL
    assert _append(lib, _layout(), kns=I64x3(8 * 64, 8 * 64, 60)) == ERR_UNSUPPORTED
    assert _append(lib, _layout(), rows=100) == ERR_SHAPE          # table shorter than max_seqlen
    assert _append(lib, _layout(), t=0) == OK
    assert _append(lib, _layout(), n=0) == OK


def _decode_kv(lib, lay, **kw):
    a = dict(n=4, hq=64, hkv=8, d=64, q=P, qs=I64x2(64 * 64, 64), k=P, v=P, lens=P, maxlen=1024, sinks=P,
             scale=0.125, window=0, table=P, rows=1024, rd=64, out=P, os=I64x2(64 * 64, 64), ws=P, wsb=1 << 30,
             splits=0)
    a.update(kw)
    return lib.gptoss_attn_decode_kv(ctypes.byref(lay) if lay is not None else None, a["n"], a["hq"], a["hkv"],
                                     a["d"], a["q"], a["qs"], a["k"], a["v"], a["lens"], a["maxlen"], a["sinks"],
                                     a["scale"], a["window"], a["table"], a["rows"], a["rd"], a["out"], a["os"],
                                     a["ws"], a["wsb"], a["splits"], None)


def test_decode_kv_argument_errors(lib):
    assert _decode_kv(lib, None) == ERR_NULL
    assert _decode_kv(lib, _layout(), maxlen=2048, rows=4096) == ERR_SHAPE            # beyond the cache's rows
    assert _decode_kv(lib, _layout(kind=2, cap=128), window=0) == ERR_UNSUPPORTED    # ring needs window = capacity
    assert _decode_kv(lib, _layout(kind=2, cap=128), window=64) == ERR_UNSUPPORTED
    paged = _layout(kind=1, cap=64, strides=(64 * 8 * 64, 8 * 64, 64), bt=P, max_pages=8, num_pages=100)
    assert _decode_kv(lib, paged, maxlen=1024) == ERR_SHAPE                          # 8 pages x 64 rows = 512
    assert _decode_kv(lib, _layout(kind=1, cap=100, bt=P, max_pages=8, num_pages=9), maxlen=512) == ERR_UNSUPPORTED
    assert _decode_kv(lib, paged, maxlen=512, wsb=16) == ERR_WORKSPACE
    assert _decode_kv(lib, _layout(), d=128) == ERR_UNSUPPORTED
    assert _decode_kv(lib, _layout(), lens=None) == ERR_NULL
    assert _decode_kv(lib, _layout(kind=2, cap=128), window=128, wsb=16) == ERR_WORKSPACE
    assert _decode_kv(lib, _layout(), n=0) == OK


def _decode_noalloc(lib, lay, **kw):
    a = dict(n=4, hq=64, hkv=8, d=64, q=P, qs=I64x2(64 * 64, 64), k=P, v=P, lens=P, maxlen=1024, sinks=P,
             scale=0.125, window=0, table=P, rows=1024, rd=64, out=P, os=I64x2(64 * 64, 64), splits=0)
    a.update(kw)
    return lib.gptoss_attn_decode_kv_noalloc(ctypes.byref(lay) if lay is not None else None, a["n"], a["hq"],
                                             a["hkv"], a["d"], a["q"], a["qs"], a["k"], a["v"], a["lens"],
                                             a["maxlen"], a["sinks"], a["scale"], a["window"], a["table"], a["rows"],
                                             a["rd"], a["out"], a["os"], a["splits"], None)


def test_decode_noalloc_argument_errors(lib):
    """The allocation-free decode checks its arguments like gptoss_attn_decode_kv and refuses,
    before any launch, calls whose partials cannot fit its fixed 32 MiB scratch."""
    assert _decode_noalloc(lib, None) == ERR_NULL
    assert _decode_noalloc(lib, _layout(), d=128) == ERR_UNSUPPORTED
    assert _decode_noalloc(lib, _layout(kind=2, cap=128), window=64) == ERR_UNSUPPORTED
    assert _decode_noalloc(lib, _layout(), lens=None) == ERR_NULL
    assert _decode_noalloc(lib, _layout(), n=0) == OK
    # one split per sequence already needs 2048 * 64 * 264 bytes > 32 MiB
    assert _decode_noalloc(lib, _layout(cap=1), n=2048, maxlen=1, rows=1) == ERR_WORKSPACE
    assert b"32 MiB" in lib.gptoss_last_error() or b"33554432" in lib.gptoss_last_error()
    # a caller-given split count is not shortened: 64 splits of 64 sequences need 66 MiB
    assert _decode_noalloc(lib, _layout(cap=32768), n=64, maxlen=32768, rows=32768, splits=64) == ERR_WORKSPACE


def test_decode_kv_workspace_size(lib):
    # contiguous == the plain decode's size; a ring is sized by its slots; a paged window
    # layer by window + 31 keys (its reads start at a 32-key boundary)
    cont = _layout(cap=32768)
    assert lib.gptoss_attn_decode_kv_workspace_size(ctypes.byref(cont), 64, 64, 32768, 0, 0) == \
        lib.gptoss_attn_decode_workspace_size(64, 64, 32768, 0)
    ring = _layout(kind=2, cap=128)
    assert lib.gptoss_attn_decode_kv_workspace_size(ctypes.byref(ring), 64, 64, 1 << 20, 128, 0) == \
        lib.gptoss_attn_decode_workspace_size(64, 64, 128, 0)
    paged = _layout(kind=1, cap=64, bt=P, max_pages=512, num_pages=4096)
    assert lib.gptoss_attn_decode_kv_workspace_size(ctypes.byref(paged), 64, 64, 32768, 128, 0) == \
        lib.gptoss_attn_decode_workspace_size(64, 64, 159, 0)
    assert lib.gptoss_attn_decode_kv_workspace_size(None, 64, 64, 32768, 0, 0) == 0


def _proj(lib, desc, **kw):
    a = dict(x=P, xs=2880, hidden=2880, wq=P, bq=P, wk=P, bk=P, wv=P, bv=P, table=P, rows=4096, rd=64, q=P, k=P,
             v=P)
    a.update(kw)
    return lib.gptoss_qkv_proj_rope(ctypes.byref(desc) if desc is not None else None, a["x"], a["xs"], a["hidden"],
                                    a["wq"], a["bq"], a["wk"], a["bk"], a["wv"], a["bv"], a["table"], a["rows"],
                                    a["rd"], a["q"], a["k"], a["v"], None)


def test_projection_argument_errors(lib):
    d = _desc_bshd()
    assert _proj(lib, None) == ERR_NULL
    assert _proj(lib, d, hidden=100) == ERR_UNSUPPORTED                     # not a multiple of 64
    assert _proj(lib, SeqDesc(0, 2, 128, 128, None, 16, 2, 64)) == ERR_UNSUPPORTED   # Hkv not a multiple of 4
    assert _proj(lib, d, wk=None) == ERR_NULL
    assert _proj(lib, d, xs=2000) == ERR_UNSUPPORTED                        # row stride below hidden
    assert _proj(lib, d, bq=ctypes.c_void_p(0x10001)) == ERR_UNSUPPORTED
    assert _proj(lib, d, rd=48) == ERR_UNSUPPORTED                          # epilogue rotates 64 or 32 dims
    assert _proj(lib, d, rows=100) == ERR_SHAPE                             # table shorter than the sequence
    assert _proj(lib, SeqDesc(0, 0, 128, 128, None, 64, 8, 64)) == OK       # no tokens


def test_shard_and_merge_argument_errors(lib):
    d = _desc_bshd()
    f = lib.gptoss_attn_prefill_shard
    args = lambda **kw: dict(dict(q=P, k=P, v=P, kvl=128, qo=0, ko=0, lse=P, ws=P, wsb=1 << 30, rows=4096), **kw)
    call = lambda desc, **kw: (lambda a: f(ctypes.byref(desc), a["q"], S3, a["k"], K3, a["v"], K3, a["kvl"], a["qo"],
                                           a["ko"], 0.125, 0, P, a["rows"], 64, P, S3, a["lse"], a["ws"], a["wsb"],
                                           None))(args(**kw))
    assert call(SeqDesc(1, 2, 100, 50, P, 64, 8, 64)) == ERR_UNSUPPORTED     # THD
    assert call(d, kvl=-1) == ERR_SHAPE
    assert call(d, qo=-5) == ERR_SHAPE
    assert call(d, lse=None) == ERR_NULL
    assert call(d, lse=ctypes.c_void_p(0x10004)) == ERR_UNSUPPORTED
    assert call(d, qo=4000, rows=4096) == ERR_SHAPE                          # table must cover q_offset + S
    assert call(d, wsb=16) == ERR_WORKSPACE
    assert lib.gptoss_attn_prefill_shard_workspace_size(ctypes.byref(d), 256) == 2 * 256 * 8 * 64 * 2
    m = lib.gptoss_attn_merge
    st4 = (ctypes.c_int64 * 4)(128 * 64 * 64, 64 * 64, 64, 1)
    assert m(2, 128, 64, 128, P, st4, P, P, P, I64x2(64 * 64, 64), None, None) == ERR_UNSUPPORTED   # head_dim
    assert m(2, 128, 64, 64, None, st4, P, P, P, I64x2(64 * 64, 64), None, None) == ERR_NULL
    assert m(2, 128, 64, 64, P, (ctypes.c_int64 * 4)(1, 1, 1, 2), P, P, P, I64x2(64 * 64, 64), None, None) == \
        ERR_UNSUPPORTED
    assert m(2, 0, 64, 64, P, st4, P, P, P, I64x2(64 * 64, 64), None, None) == OK
