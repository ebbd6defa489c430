"""GPT-OSS attention hot path on MI355X: YaRN RoPE, sink + GQA + sliding-window
prefill (BSHD and packed THD) with its backward pass and its context-parallel
shard + merge form, split-KV decode over
contiguous, paged or ring KV caches, the cache append, and the q/k/v
projections with the RoPE in their epilogue, as
hand-written gfx950 HIP kernels behind a C ABI (include/gptoss_attn.h). This
package is the thin torch binding; libgptoss_attn.so is loaded on first use and
is required.
"""

from .api import (  # noqa: F401
    rope_config,
    yarn_params,
    rope_table,
    rope_qk,
    attn_prefill,
    attn_prefill_lse,
    attn_prefill_backward,
    attn_decode,
    qkv_proj_rope,
    attn_prefill_shard,
    prefill_shard_workspace_size,
    attn_merge,
    kv_layout,
    kv_append,
    attn_decode_kv,
    attn_decode_kv_noalloc,
    decode_kv_workspace_size,
    prefill_workspace_size,
    prefill_backward_workspace_size,
    check_lengths,
    LENGTH_FAULTS,
    decode_workspace_size,
)
from ._lib import GptossError, load as load_library  # noqa: F401
