"""Writes tests/golden/yarn_table.json from the oracle alone (no HIP code involved).

Contents: the 32 YaRN frequencies and the concentration of GPT-OSS's RoPE
(base 150000, factor 32, original context 4096, ntk_alpha 1, ntk_beta 32, the
RotaryEmbedding entry of the rope_utils page) as exact hex floats, and the bf16
bit patterns of whole table rows at a few positions. It serves as a regression
fixture: any later change to the oracle's YaRN or table arithmetic shows up.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

cfg = oracle.RopeConfig()
om, c, (lo, hi) = oracle.yarn_params(cfg)
positions = [0, 1, 2, 127, 128, 4095, 4096, 65535, 131071]
table = oracle.freqs_cis(cfg, max(positions) + 1)[positions]
out = {
    "config": {"head_dim": cfg.head_dim, "rotary_dim": cfg.rotary_dim, "base": cfg.base,
               "scaling_factor": cfg.scaling_factor,
               "initial_context_length": cfg.initial_context_length,
               "ntk_alpha": cfg.ntk_alpha, "ntk_beta": cfg.ntk_beta},
    "omega_hex": [float(x).hex() for x in om],
    "concentration_hex": float(c).hex(),
    "ramp_lo_hi": [lo, hi],
    "positions": positions,
    "table_bits": oracle.bf16_bits(table).tolist(),
}
path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "yarn_table.json")
with open(path, "w") as f:
    json.dump(out, f, indent=1)
print("wrote", path)
