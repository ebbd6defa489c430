"""Plain fp64 CPU oracle for GPT-OSS attention: sink + GQA + sliding window + YaRN RoPE.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library and its Python
binding never call it. It shares no code with them: no kernels, headers,
helpers, tables or constant generators.

Everything is numpy float64 on the CPU. bf16 rounding (IEEE round-to-nearest-even
to an 8-bit significand) is applied only at the two points the rope_utils page
names: the cos/sin table is rounded to the q/k dtype, and the rotated q and k
keep that dtype. Everything after that (scores, sink softmax, the weighted sum of
v) is kept in fp64 and is the comparison target for the GPU's bf16 output.

Sources (the pages are cited by title and section):
  * "nemo_automodel.components.models.gpt_oss.rope_utils" (NeMo AutoModel docs
    v0.7): RotaryEmbedding and its constructor defaults,
    _compute_concentration_and_inv_freq (YaRN), _compute_cos_sin,
    _apply_rotary_emb_qk, apply_rotary_emb, apply_rotary_emb_qk (BSHD / THD,
    cu_seqlens), position_ids_to_freqs_cis.
  * "nemo_automodel.components.models.gpt_oss.layers" (NeMo AutoModel docs v0.4):
    GptOssAttention attributes sinks, sliding_window, softmax_scale,
    yarn_concentration, num_attention_heads, num_key_value_heads.
  * "Transformers v4.55.0" release notes, section "Architecture": RoPE with 128K
    context, alternating full and 128-token sliding-window layers, a learned
    per-head sink that adds a term to the softmax denominator.
  * "gpt-oss-20b 模型结构" (model-structure print-out): q_proj 2880->4096,
    k_proj / v_proj 2880->512, so 64 query heads and 8 KV heads of width 64.

``oracle.kvcache`` keeps the keys and values of the decode loop in contiguous,
paged and ring caches (append, and decode over a cache); no page specifies a
cache, so its layouts are readings, pinned against the prefill definition.

``oracle.backward`` adds the log-sum-exp of each row and the gradients of the
attention with respect to q, k, v and the sinks: the derivatives of the same
definition (no page prints a backward pass).

Parity unpinned: agreement with real GPT-OSS checkpoints. The pages print no
activations or outputs, and the RoPE pairing (half-split) and the YaRN ramp
shape (linear in the dimension index) are readings of the pages, not facts
they state. Every function here is otherwise pinned by tests/test_oracle_*.py.
"""

from .bf16 import round_bf16, bf16_bits, from_bf16_bits
from .yarn import RopeConfig, yarn_params, cos_sin_table, freqs_cis
from .rope import rotate, rope_qk_bshd, rope_qk_thd, thd_positions
from .attention import (
    sink_attention,
    prefill_bshd,
    prefill_thd,
    prefill_rows,
    decode,
)
from . import kvcache
from .backward import (rotate_transpose, sink_attention_backward, prefill_bshd_backward, prefill_thd_backward,
                       prefill_backward_rows)

__all__ = [
    "round_bf16", "bf16_bits", "from_bf16_bits",
    "RopeConfig", "yarn_params", "cos_sin_table", "freqs_cis",
    "rotate", "rope_qk_bshd", "rope_qk_thd", "thd_positions",
    "sink_attention", "prefill_bshd", "prefill_thd", "prefill_rows", "decode",
    "rotate_transpose", "sink_attention_backward", "prefill_bshd_backward", "prefill_thd_backward",
    "prefill_backward_rows", "kvcache",
]
