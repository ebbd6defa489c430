"""The oracle's YaRN table against values computed apart from it.

tests/golden/yarn_independent.json holds the frequencies, concentration, ramp
boundaries and bf16 table bits for GPT-OSS's configuration (page
"nemo_automodel.components.models.gpt_oss.rope_utils", RotaryEmbedding:
_compute_concentration_and_inv_freq and _compute_cos_sin; head_dim 64, base
150000, factor 32 over a 4096-token original context, ntk_beta 32, ntk_alpha 1),
from a calculation made separately from oracle/yarn.py. Unlike yarn_table.json
(written by the oracle itself, a regression fixture), these pin the oracle to an
outside computation: a wrong ramp boundary, the ramp taken linear in the
wavelength ratio instead of the dimension index (omega_9 would be 2.497e-02
instead of 3.171e-02), or the concentration applied twice (bf16 0x3fe8
instead of 0x3fac) or not at all would each move some of these values.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "yarn_independent.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return json.load(f)


def test_frequencies_concentration_and_boundaries(gold):
    omega, c, (lo, hi) = oracle.yarn_params(oracle.RopeConfig())
    assert c == pytest.approx(gold["concentration"], rel=1e-15)
    assert lo == pytest.approx(gold["lo"], rel=1e-14)
    assert hi == pytest.approx(gold["hi"], rel=1e-14)
    # 11 significant digits in the fixture
    assert np.allclose(omega[:9], gold["theta_0_8"], rtol=1e-10, atol=0)
    assert np.allclose(omega[9:18], gold["omega_9_17"], rtol=1e-10, atol=0)
    assert omega[18] == pytest.approx(gold["omega_18"], rel=1e-10)
    assert omega[31] == pytest.approx(gold["omega_31"], rel=1e-10)
    assert float(omega.sum()) == pytest.approx(gold["omega_sum"], rel=1e-14)
    gamma = np.clip((np.arange(9, 18) - lo) / (hi - lo), 0, 1)
    assert np.allclose(gamma, gold["gamma_9_17"], atol=5e-7)


def test_table_bits(gold):
    t = gold["table_bits"]
    cos, sin = oracle.cos_sin_table(oracle.RopeConfig(), t["positions"])
    bits = lambda x: np.vectorize(lambda v: "0x%04x" % int(oracle.bf16_bits(np.array([v]))[0]))(x)  # noqa: E731
    for r in range(len(t["positions"])):
        for j, i in enumerate(t["pairs"]):
            assert bits(cos[r, i]) == t["cos"][r][j], (t["positions"][r], i, "cos")
            assert bits(sin[r, i]) == t["sin"][r][j], (t["positions"][r], i, "sin")
    c_bits = oracle.bf16_bits(oracle.round_bf16(np.array([gold["concentration"]])))[0]
    assert "0x%04x" % int(c_bits) == gold["concentration_bf16_bits"]
