"""ctypes declarations of libgptoss_attn.so (the C ABI in include/gptoss_attn.h).

The library is loaded on first use. A missing library is an error: there is no
fallback implementation.
"""

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GPTOSS_ATTN_LIB", os.path.join(_HERE, "libgptoss_attn.so"))

c_i32, c_i64, c_f32, c_f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
c_vp, c_size = ctypes.c_void_p, ctypes.c_size_t
I64x3 = c_i64 * 3
I64x2 = c_i64 * 2

BSHD, THD = 0, 1
KROT = {"auto": 0, "fused": 1, "separate": 2}


class RopeConfig(ctypes.Structure):
    _fields_ = [("head_dim", c_i32), ("rotary_dim", c_i32), ("base", c_f64), ("scaling_factor", c_f64),
                ("initial_context_length", c_i32), ("ntk_alpha", c_f64), ("ntk_beta", c_f64)]


class SeqDesc(ctypes.Structure):
    _fields_ = [("layout", c_i32), ("batch", c_i32), ("seqlen", c_i32), ("max_seqlen", c_i32),
                ("cu_seqlens", c_vp), ("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32)]


class KVLayout(ctypes.Structure):
    _fields_ = [("kind", c_i32), ("capacity", c_i32), ("strides", I64x3), ("block_table", c_vp),
                ("max_pages", c_i32), ("num_pages", c_i32)]


CACHE_KINDS = {"contiguous": 0, "paged": 1, "ring": 2}

# name -> (restype, argtypes); every symbol include/gptoss_attn.h declares
SIGNATURES = {
    "gptoss_abi_version": (ctypes.c_int, []),
    "gptoss_check_lengths": (ctypes.c_int, [c_vp, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp]),
    "gptoss_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gptoss_last_error": (ctypes.c_char_p, []),
    "gptoss_yarn_params": (ctypes.c_int, [ctypes.POINTER(RopeConfig), ctypes.POINTER(c_f64),
                                          ctypes.POINTER(c_f64)]),
    "gptoss_rope_table_init": (ctypes.c_int, [ctypes.POINTER(RopeConfig), c_i32, c_vp, c_vp]),
    "gptoss_rope_qk": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, c_vp,
                                      c_vp, c_i32, c_i32, c_vp]),
    "gptoss_attn_prefill_workspace_size": (c_size, [ctypes.POINTER(SeqDesc)]),
    "gptoss_attn_prefill": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, I64x3,
                                           c_vp, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp, I64x3,
                                           c_vp, c_size, c_vp]),
    "gptoss_attn_prefill_ex": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, I64x3,
                                              c_vp, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp, I64x3,
                                              c_vp, c_size, c_i32, c_vp]),
    "gptoss_attn_prefill_lse": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, I64x3,
                                               c_vp, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp, I64x3, c_vp,
                                               c_vp, c_size, c_vp]),
    "gptoss_attn_prefill_backward_workspace_size": (c_size, [ctypes.POINTER(SeqDesc)]),
    "gptoss_attn_prefill_backward": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, I64x3,
                                                    c_vp, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp, I64x3,
                                                    c_vp, I64x3, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                    c_vp, c_size, c_vp]),
    "gptoss_attn_decode_workspace_size": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "gptoss_attn_prefill_shard_workspace_size": (c_size, [ctypes.POINTER(SeqDesc), c_i32]),
    "gptoss_attn_prefill_shard": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, I64x3, c_vp, I64x3, c_vp, I64x3,
                                                 c_i32, c_i32, c_i32, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp,
                                                 I64x3, c_vp, c_vp, c_size, c_vp]),
    "gptoss_attn_merge": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_vp, c_i64 * 4, c_vp, c_vp, c_vp, I64x2,
                                         c_vp, c_vp]),
    "gptoss_qkv_proj_rope": (ctypes.c_int, [ctypes.POINTER(SeqDesc), c_vp, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "gptoss_kv_append": (ctypes.c_int, [ctypes.POINTER(KVLayout), c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, I64x3,
                                        c_vp, I64x3, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp]),
    "gptoss_attn_decode_kv_workspace_size": (c_size, [ctypes.POINTER(KVLayout), c_i32, c_i32, c_i32, c_i32, c_i32]),
    "gptoss_attn_decode_kv": (ctypes.c_int, [ctypes.POINTER(KVLayout), c_i32, c_i32, c_i32, c_i32, c_vp, I64x2,
                                             c_vp, c_vp, c_vp, c_i32, c_vp, c_f32, c_i32, c_vp, c_i32, c_i32,
                                             c_vp, I64x2, c_vp, c_size, c_i32, c_vp]),
    "gptoss_attn_decode_kv_noalloc": (ctypes.c_int, [ctypes.POINTER(KVLayout), c_i32, c_i32, c_i32, c_i32, c_vp,
                                                     I64x2, c_vp, c_vp, c_vp, c_i32, c_vp, c_f32, c_i32, c_vp,
                                                     c_i32, c_i32, c_vp, I64x2, c_i32, c_vp]),
    "gptoss_attn_decode": (ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_vp, I64x2, c_vp, c_vp, I64x3,
                                          c_vp, c_i32, c_vp, c_f32, c_i32, c_vp, c_i32, c_i32, c_vp, I64x2,
                                          c_vp, c_size, c_i32, c_vp]),
}

_lib = None
_lock = threading.Lock()


def load(path=None):
    """Load (once) and return the library handle; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(
                    f"libgptoss_attn.so not found at {p}; build it with "
                    "`python -m attention_yarn_rope_amd.build` (there is no fallback path)")
            lib = ctypes.CDLL(p)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


class GptossError(RuntimeError):
    def __init__(self, fn, status):
        lib = load()
        msg = lib.gptoss_status_string(status).decode()
        detail = lib.gptoss_last_error().decode()
        super().__init__(f"{fn} failed with status {status} ({msg}): {detail}")
        self.status = status


def check(fn, status):
    if status != 0:
        raise GptossError(fn, status)
