"""Python binding of the C ABI: torch tensors in, torch tensors out.

Argument marshalling only -- shapes and strides are read off the tensors, device
memory comes from torch's allocator, work is enqueued on torch's current stream.
Every step of the computation runs in the HIP kernels of libgptoss_attn.so.
"""

import ctypes

import torch

from . import _lib
from ._lib import RopeConfig, SeqDesc, KVLayout, I64x2, I64x3, check

HEAD_DIM = 64


def rope_config(head_dim=64, rotary_dim=None, base=150000.0, scaling_factor=32.0,
                initial_context_length=4096, ntk_alpha=1.0, ntk_beta=32.0):
    """RoPE settings; defaults are GPT-OSS's (RotaryEmbedding on the rope_utils page)."""
    return RopeConfig(head_dim, head_dim if rotary_dim is None else rotary_dim, float(base),
                      float(scaling_factor), int(initial_context_length), float(ntk_alpha), float(ntk_beta))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _bf16(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA bfloat16 tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t


def _strides3(t, layout):
    s = t.stride()
    return I64x3(s[0], s[1], s[2]) if layout == _lib.BSHD else I64x3(0, s[0], s[1])


def yarn_params(cfg=None):
    """Host fp64 YaRN frequencies (rotary_dim/2 values) and concentration."""
    cfg = cfg or rope_config()
    n = cfg.rotary_dim // 2
    om = (ctypes.c_double * n)()
    c = ctypes.c_double()
    check("gptoss_yarn_params", _lib.load().gptoss_yarn_params(ctypes.byref(cfg), om, ctypes.byref(c)))
    return list(om), c.value


def rope_table(num_positions, cfg=None, device="cuda", out=None):
    """bf16 [num_positions, rotary_dim] table: cos half then sin half, concentration applied."""
    cfg = cfg or rope_config()
    t = out if out is not None else torch.empty((num_positions, cfg.rotary_dim), dtype=torch.bfloat16,
                                                device=device)
    _bf16(t, "table")
    if tuple(t.shape) != (num_positions, cfg.rotary_dim) or not t.is_contiguous():
        raise ValueError("out must be a contiguous [num_positions, rotary_dim] tensor")
    check("gptoss_rope_table_init",
          _lib.load().gptoss_rope_table_init(ctypes.byref(cfg), num_positions, _ptr(t), _stream()))
    return t


def _desc(q, k, cu_seqlens, max_seqlen):
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("BSHD q must be [B, S, Hq, D]")
        B, S, Hq, D = q.shape
        return SeqDesc(_lib.BSHD, B, S, S, None, Hq, k.shape[2], D), _lib.BSHD
    if q.dim() != 3:
        raise ValueError("THD q must be [T, Hq, D]")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous CUDA int32 tensor")
    T, Hq, D = q.shape
    if max_seqlen is None:
        raise ValueError("THD needs max_seqlen (a host-side bound of the sequence lengths)")
    return SeqDesc(_lib.THD, cu_seqlens.numel() - 1, T, int(max_seqlen), ctypes.c_void_p(cu_seqlens.data_ptr()),
                   Hq, k.shape[1], D), _lib.THD


def rope_qk(q, k, table, cu_seqlens=None, max_seqlen=None):
    """Rotate q and k (BSHD [B,S,H,D] or THD [T,H,D] with cu_seqlens) into new contiguous tensors."""
    _bf16(q, "q"), _bf16(k, "k"), _bf16(table, "table")
    desc, layout = _desc(q, k, cu_seqlens, max_seqlen)
    q_out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    k_out = torch.empty(k.shape, dtype=k.dtype, device=k.device)
    check("gptoss_rope_qk", _lib.load().gptoss_rope_qk(
        ctypes.byref(desc), _ptr(q), _strides3(q, layout), _ptr(k), _strides3(k, layout),
        _ptr(q_out), _ptr(k_out), _ptr(table), table.shape[0], table.shape[1], _stream()))
    return q_out, k_out


def prefill_workspace_size(q, k, cu_seqlens=None, max_seqlen=None):
    desc, _ = _desc(q, k, cu_seqlens, max_seqlen)
    return _lib.load().gptoss_attn_prefill_workspace_size(ctypes.byref(desc))


def attn_prefill(q, k, v, sinks, window=0, table=None, softmax_scale=None, cu_seqlens=None, max_seqlen=None,
                 out=None, workspace=None, k_rotation="auto"):
    """Sink + GQA + causal/sliding-window attention over BSHD or packed THD inputs.

    With ``table`` q and k are rotated on the fly; without it they are taken as
    already rotated. Returns ``out`` (bf16, q's shape).
    """
    _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    if sinks.dtype != torch.float32 or not sinks.is_cuda or not sinks.is_contiguous():
        raise TypeError("sinks must be a contiguous CUDA float32 tensor")
    desc, layout = _desc(q, k, cu_seqlens, max_seqlen)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _bf16(out, "out")
    lib = _lib.load()
    need = lib.gptoss_attn_prefill_workspace_size(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    if table is not None:
        _bf16(table, "table")
    check("gptoss_attn_prefill_ex", lib.gptoss_attn_prefill_ex(
        ctypes.byref(desc), _ptr(q), _strides3(q, layout), _ptr(k), _strides3(k, layout),
        _ptr(v), _strides3(v, layout), _ptr(sinks), float(scale), int(window), tptr, trows, tdim,
        _ptr(out), _strides3(out, layout), _ptr(workspace), workspace.numel(), _lib.KROT[k_rotation],
        _stream()))
    return out


def _sinks(sinks):
    if sinks.dtype != torch.float32 or not sinks.is_cuda or not sinks.is_contiguous():
        raise TypeError("sinks must be a contiguous CUDA float32 tensor")
    return sinks


def attn_prefill_lse(q, k, v, sinks, window=0, table=None, softmax_scale=None, cu_seqlens=None, max_seqlen=None,
                     out=None, lse=None, workspace=None):
    """attn_prefill that also returns each row's log-sum-exp: (out, lse fp32 [tokens, Hq])."""
    _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _sinks(sinks)
    desc, layout = _desc(q, k, cu_seqlens, max_seqlen)
    tokens = q.shape[0] * q.shape[1] if layout == _lib.BSHD else q.shape[0]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((tokens, q.shape[-2]), dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != tokens * q.shape[-2]:
        raise ValueError("lse must be a contiguous float32 [tokens, Hq] tensor")
    _bf16(out, "out")
    lib = _lib.load()
    need = lib.gptoss_attn_prefill_workspace_size(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_attn_prefill_lse", lib.gptoss_attn_prefill_lse(
        ctypes.byref(desc), _ptr(q), _strides3(q, layout), _ptr(k), _strides3(k, layout),
        _ptr(v), _strides3(v, layout), _ptr(sinks), float(scale), int(window), tptr, trows, tdim,
        _ptr(out), _strides3(out, layout), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


def prefill_backward_workspace_size(q, k, cu_seqlens=None, max_seqlen=None):
    desc, _ = _desc(q, k, cu_seqlens, max_seqlen)
    return _lib.load().gptoss_attn_prefill_backward_workspace_size(ctypes.byref(desc))


def attn_prefill_backward(q, k, v, sinks, out, dout, lse, window=0, table=None, softmax_scale=None,
                          cu_seqlens=None, max_seqlen=None, workspace=None, grads=None):
    """Gradients of attn_prefill: (dq, dk, dv bf16 contiguous in q/k/v's layout, dsinks fp32 [Hq]).

    q, k, v, sinks, window, table, softmax_scale as given to the forward; out and lse
    from attn_prefill_lse; dout = dL/d out. ``grads`` may pass preallocated (dq, dk, dv, dsinks).
    """
    _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v"), _bf16(out, "out"), _bf16(dout, "dout"), _sinks(sinks)
    desc, layout = _desc(q, k, cu_seqlens, max_seqlen)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    if grads is None:
        grads = (torch.empty(q.shape, dtype=torch.bfloat16, device=q.device),
                 torch.empty(k.shape, dtype=torch.bfloat16, device=q.device),
                 torch.empty(v.shape, dtype=torch.bfloat16, device=q.device),
                 torch.empty(q.shape[-2], dtype=torch.float32, device=q.device))
    dq, dk, dv, dsinks = grads
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t.shape != ref.shape or not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 tensor shaped like its input")
    lib = _lib.load()
    need = lib.gptoss_attn_prefill_backward_workspace_size(ctypes.byref(desc))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_attn_prefill_backward", lib.gptoss_attn_prefill_backward(
        ctypes.byref(desc), _ptr(q), _strides3(q, layout), _ptr(k), _strides3(k, layout),
        _ptr(v), _strides3(v, layout), _ptr(sinks), float(scale), int(window), tptr, trows, tdim,
        _ptr(out), _strides3(out, layout), _ptr(dout), _strides3(dout, layout), _ptr(lse),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks), _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dsinks


def decode_workspace_size(num_seqs, num_q_heads, max_cache_len, num_splits=0):
    return _lib.load().gptoss_attn_decode_workspace_size(num_seqs, num_q_heads, max_cache_len, num_splits)


def attn_decode(q, k_cache, v_cache, cache_seqlens, sinks, window=0, table=None, softmax_scale=None,
                num_splits=0, out=None, workspace=None):
    """One query token per sequence: q [N,Hq,D], caches [N,Lmax,Hkv,D], cache_seqlens int32 [N]."""
    _bf16(q, "q"), _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache")
    if k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must share strides")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be a CUDA int32 tensor")
    if sinks.dtype != torch.float32 or not sinks.is_cuda or not sinks.is_contiguous():
        raise TypeError("sinks must be a contiguous CUDA float32 tensor")
    N, Hq, D = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lib = _lib.load()
    need = lib.gptoss_attn_decode_workspace_size(N, Hq, Lmax, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    ks = k_cache.stride()
    check("gptoss_attn_decode", lib.gptoss_attn_decode(
        N, Hq, Hkv, D, _ptr(q), I64x2(q.stride(0), q.stride(1)), _ptr(k_cache), _ptr(v_cache),
        I64x3(ks[0], ks[1], ks[2]), _ptr(cache_seqlens), Lmax, _ptr(sinks), float(scale), int(window),
        tptr, trows, tdim, _ptr(out), I64x2(out.stride(0), out.stride(1)), _ptr(workspace),
        workspace.numel(), int(num_splits), _stream()))
    return out


def kv_layout(k_cache, kind="contiguous", block_table=None):
    """The gptoss_kv_layout of a cache tensor. Contiguous and ring caches are
    [N, capacity, Hkv, D]; a paged pool is [num_pages, page_size, Hkv, D] with a
    device int32 block_table [N, max_pages]."""
    if kind not in _lib.CACHE_KINDS:
        raise ValueError(f"kind must be one of {sorted(_lib.CACHE_KINDS)}")
    if k_cache.dim() != 4:
        raise ValueError("a cache is a 4-d tensor")
    s = k_cache.stride()
    lay = KVLayout()
    lay.kind = _lib.CACHE_KINDS[kind]
    lay.capacity = k_cache.shape[1]
    lay.strides = I64x3(s[0], s[1], s[2])
    if kind == "paged":
        if block_table is None or block_table.dtype != torch.int32 or not block_table.is_cuda or \
                block_table.dim() != 2 or not block_table.is_contiguous():
            raise TypeError("a paged cache needs a contiguous CUDA int32 block_table [N, max_pages]")
        lay.block_table = block_table.data_ptr()
        lay.max_pages = block_table.shape[1]
        lay.num_pages = k_cache.shape[0]
    return lay


def _cache_max_seqlen(kind, k_cache, block_table, table):
    if kind == "contiguous":
        return k_cache.shape[1]
    if kind == "paged":
        return block_table.shape[1] * k_cache.shape[1]
    return table.shape[0] if table is not None else 2 ** 30


def kv_append(k_cache, v_cache, k_new, v_new, cache_seqlens, kind="contiguous", block_table=None, table=None,
              max_seqlen=None):
    """Store the newest tokens of every sequence: k_new / v_new [N, T, Hkv, D] (or [N, Hkv, D] for
    one token) at positions cache_seqlens - T .. cache_seqlens - 1, k rotated there with the table."""
    _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache"), _bf16(k_new, "k_new"), _bf16(v_new, "v_new")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_new.dim() == 3:
        k_new, v_new = k_new.unsqueeze(1), v_new.unsqueeze(1)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have one shape")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be a CUDA int32 tensor")
    N, T, Hkv, D = k_new.shape
    lay = kv_layout(k_cache, kind, block_table)
    if max_seqlen is None:
        max_seqlen = _cache_max_seqlen(kind, k_cache, block_table, table)
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    kn, vn = k_new.stride(), v_new.stride()
    check("gptoss_kv_append", _lib.load().gptoss_kv_append(
        ctypes.byref(lay), _ptr(k_cache), _ptr(v_cache), N, Hkv, D, T, _ptr(k_new), I64x3(kn[0], kn[1], kn[2]),
        _ptr(v_new), I64x3(vn[0], vn[1], vn[2]), _ptr(cache_seqlens), int(max_seqlen), tptr, trows, tdim, _stream()))


def decode_kv_workspace_size(q, k_cache, kind="contiguous", block_table=None, window=0, max_seqlen=None,
                             table=None, num_splits=0):
    lay = kv_layout(k_cache, kind, block_table)
    if max_seqlen is None:
        max_seqlen = _cache_max_seqlen(kind, k_cache, block_table, table)
    return _lib.load().gptoss_attn_decode_kv_workspace_size(ctypes.byref(lay), q.shape[0], q.shape[1],
                                                             int(max_seqlen), int(window), int(num_splits))


def attn_decode_kv(q, k_cache, v_cache, cache_seqlens, sinks, kind="contiguous", block_table=None, window=0,
                   table=None, max_seqlen=None, softmax_scale=None, num_splits=0, out=None, workspace=None):
    """attn_decode over a contiguous, paged or ring cache (kind); a ring needs window == its slot count."""
    _bf16(q, "q"), _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be a CUDA int32 tensor")
    if sinks.dtype != torch.float32 or not sinks.is_cuda or not sinks.is_contiguous():
        raise TypeError("sinks must be a contiguous CUDA float32 tensor")
    N, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    lay = kv_layout(k_cache, kind, block_table)
    if max_seqlen is None:
        max_seqlen = _cache_max_seqlen(kind, k_cache, block_table, table)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lib = _lib.load()
    need = lib.gptoss_attn_decode_kv_workspace_size(ctypes.byref(lay), N, Hq, int(max_seqlen), int(window),
                                                    int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_attn_decode_kv", lib.gptoss_attn_decode_kv(
        ctypes.byref(lay), N, Hq, Hkv, D, _ptr(q), I64x2(q.stride(0), q.stride(1)), _ptr(k_cache), _ptr(v_cache),
        _ptr(cache_seqlens), int(max_seqlen), _ptr(sinks), float(scale), int(window), tptr, trows, tdim,
        _ptr(out), I64x2(out.stride(0), out.stride(1)), _ptr(workspace), workspace.numel(), int(num_splits),
        _stream()))
    return out


def attn_decode_kv_noalloc(q, k_cache, v_cache, cache_seqlens, sinks, kind="contiguous", block_table=None,
                           window=0, table=None, max_seqlen=None, softmax_scale=None, num_splits=0, out=None):
    """attn_decode_kv with no workspace: the library keeps the split partials in its own fixed
    per-GPU scratch (gptoss_attn_decode_kv_noalloc). Allocates only ``out`` when it is not given."""
    _bf16(q, "q"), _bf16(k_cache, "k_cache"), _bf16(v_cache, "v_cache")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_cuda:
        raise TypeError("cache_seqlens must be a CUDA int32 tensor")
    _sinks(sinks)
    N, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    lay = kv_layout(k_cache, kind, block_table)
    if max_seqlen is None:
        max_seqlen = _cache_max_seqlen(kind, k_cache, block_table, table)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_attn_decode_kv_noalloc", _lib.load().gptoss_attn_decode_kv_noalloc(
        ctypes.byref(lay), N, Hq, Hkv, D, _ptr(q), I64x2(q.stride(0), q.stride(1)), _ptr(k_cache), _ptr(v_cache),
        _ptr(cache_seqlens), int(max_seqlen), _ptr(sinks), float(scale), int(window), tptr, trows, tdim,
        _ptr(out), I64x2(out.stride(0), out.stride(1)), int(num_splits), _stream()))
    return out


def qkv_proj_rope(x, wq, bq, wk, bk, wv, bv, table=None, cu_seqlens=None, max_seqlen=None, out=None):
    """q, k, v = x W^T + b (rounded to bf16), q and k then rotated with the table (None: not rotated).

    x: [B, S, hidden] (BSHD) or [T, hidden] with cu_seqlens (THD); weights [out, hidden] (Linear
    layout), biases [out] or None. Returns q [.., Hq, 64], k and v [.., Hkv, 64] in x's layout."""
    _bf16(x, "x")
    for name, w in (("wq", wq), ("wk", wk), ("wv", wv)):
        _bf16(w, name)
        if not w.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, b in (("bq", bq), ("bk", bk), ("bv", bv)):
        if b is not None:
            _bf16(b, name)
    hidden = x.shape[-1]
    hq, hkv = wq.shape[0] // HEAD_DIM, wk.shape[0] // HEAD_DIM
    if cu_seqlens is None:
        if x.dim() != 3:
            raise ValueError("BSHD x must be [B, S, hidden]")
        B, S = x.shape[0], x.shape[1]
        if x.stride(0) != S * x.stride(1):
            raise ValueError("x's rows must be evenly spaced ([B, S] flattened)")
        desc = SeqDesc(_lib.BSHD, B, S, S, None, hq, hkv, HEAD_DIM)
        lead = (B, S)
    else:
        if x.dim() != 2:
            raise ValueError("THD x must be [T, hidden]")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
            raise TypeError("cu_seqlens must be a contiguous CUDA int32 tensor")
        T = x.shape[0]
        if max_seqlen is None:
            cu = cu_seqlens.cpu()
            max_seqlen = int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0
        desc = SeqDesc(_lib.THD, cu_seqlens.numel() - 1, T, int(max_seqlen), _ptr(cu_seqlens), hq, hkv, HEAD_DIM)
        lead = (T,)
    if out is None:
        out = (torch.empty(lead + (hq, HEAD_DIM), dtype=torch.bfloat16, device=x.device),
               torch.empty(lead + (hkv, HEAD_DIM), dtype=torch.bfloat16, device=x.device),
               torch.empty(lead + (hkv, HEAD_DIM), dtype=torch.bfloat16, device=x.device))
    q, k, v = out
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_qkv_proj_rope", _lib.load().gptoss_qkv_proj_rope(
        ctypes.byref(desc), _ptr(x), x.stride(-2), hidden, _ptr(wq), _ptr(bq), _ptr(wk), _ptr(bk), _ptr(wv),
        _ptr(bv), tptr, trows, tdim, _ptr(q), _ptr(k), _ptr(v), _stream()))
    return q, k, v


def prefill_shard_workspace_size(q, k):
    """Workspace bytes of attn_prefill_shard for a query shard q [B, Sq, Hq, D] and key shard k [B, Sk, Hkv, D]."""
    B, S, Hq, D = q.shape
    desc = SeqDesc(_lib.BSHD, B, S, S, None, Hq, k.shape[2], D)
    return _lib.load().gptoss_attn_prefill_shard_workspace_size(ctypes.byref(desc), k.shape[1])


def attn_prefill_shard(q, k, v, q_offset, kv_offset, window=0, table=None, softmax_scale=None, out=None, lse=None,
                       workspace=None):
    """One step of a context-parallel prefill: q [B, Sq, Hq, D] at positions q_offset + s against
    k, v [B, Sk, Hkv, D] at kv_offset + j, no sink. Returns (out, lse [B * Sq, Hq])."""
    _bf16(q, "q"), _bf16(k, "k"), _bf16(v, "v")
    if q.dim() != 4:
        raise ValueError("shards are BSHD: q [B, S, Hq, D]")
    B, S, Hq, D = q.shape
    desc = SeqDesc(_lib.BSHD, B, S, S, None, Hq, k.shape[2], D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B * S, Hq), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    if workspace is None:
        workspace = torch.empty(max(prefill_shard_workspace_size(q, k), 1), dtype=torch.uint8, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale   # 0: the library's head_dim ** -0.5
    tptr, trows, tdim = (_ptr(table), table.shape[0], table.shape[1]) if table is not None else (None, 0, 0)
    check("gptoss_attn_prefill_shard", lib.gptoss_attn_prefill_shard(
        ctypes.byref(desc), _ptr(q), _strides3(q, _lib.BSHD), _ptr(k), _strides3(k, _lib.BSHD), _ptr(v),
        _strides3(v, _lib.BSHD), k.shape[1], int(q_offset), int(kv_offset), float(scale), int(window), tptr, trows,
        tdim, _ptr(out), _strides3(out, _lib.BSHD), _ptr(lse), _ptr(workspace), workspace.numel(), _stream()))
    return out, lse


def attn_merge(o_parts, lse_parts, sinks=None, out=None, lse_out=None):
    """Merge partial results: o_parts [P, T, Hq, D] bf16, lse_parts [P, T * Hq] fp32 -> out [T, Hq, D]
    (and lse [T * Hq] when lse_out is given); the sink is added once."""
    _bf16(o_parts, "o_parts")
    P, T, Hq, D = o_parts.shape
    if lse_parts.dtype != torch.float32 or not lse_parts.is_contiguous() or lse_parts.numel() != P * T * Hq:
        raise ValueError("lse_parts must be a contiguous float32 [P, T * Hq] tensor")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=o_parts.device)
    ps = o_parts.stride()
    check("gptoss_attn_merge", _lib.load().gptoss_attn_merge(
        P, T, Hq, D, _ptr(o_parts), (ctypes.c_int64 * 4)(ps[0], ps[1], ps[2], ps[3]), _ptr(lse_parts),
        _ptr(sinks), _ptr(out), I64x2(out.stride(0), out.stride(1)), _ptr(lse_out), _stream()))
    return out


LENGTH_FAULTS = {"cu_start": 1, "cu_order": 2, "cu_total": 4, "cache": 8}


def check_lengths(cu_seqlens=None, total_tokens=-1, cache_seqlens=None, max_cache_len=1, result=None):
    """Check device-resident lengths on the device (no synchronisation): returns an int32 [3]
    device tensor: OR of the LENGTH_FAULTS bits of the broken rules (0: all hold), the first
    offending cu_seqlens index and the first offending cache_seqlens index (-1: none)."""
    for name, t in (("cu_seqlens", cu_seqlens), ("cache_seqlens", cache_seqlens)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor on the device")
    dev = (cu_seqlens if cu_seqlens is not None else cache_seqlens)
    if result is None:
        result = torch.empty(3, dtype=torch.int32, device=dev.device if dev is not None else "cuda")
    batch = cu_seqlens.numel() - 1 if cu_seqlens is not None else 0
    n = cache_seqlens.numel() if cache_seqlens is not None else 0
    check("gptoss_check_lengths", _lib.load().gptoss_check_lengths(
        _ptr(cu_seqlens), batch, int(total_tokens), _ptr(cache_seqlens), n, int(max_cache_len), _ptr(result),
        _stream()))
    return result
