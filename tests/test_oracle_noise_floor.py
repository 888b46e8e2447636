"""bf16 rounding noise floor of the 7B-width 2-layer model (CPU, slow).

Runs the oracle twice: as is, and with every pre-rounding value perturbed by
a relative N(0, 1e-7) -- the size of the difference between fp32 and fp64
accumulation -- for three perturbation seeds.  The largest logit
disagreement is the floor below which no bf16 implementation with a
different summation order can be held.  Everything here is seeded, so the
floor is a fixed number; the test pins it (conftest.BF16_NOISE_FLOOR), and
the GPU's model-level bound (conftest.BF16_MODEL_LOGIT_TOL) is defined as
twice it, rounded up to 0.01.  If the oracle's arithmetic changes the floor,
this test fails and the bound has to be derived again.
"""
import math

import numpy as np
import pytest

import synthetic
from conftest import BF16_MODEL_LOGIT_TOL, BF16_NOISE_FLOOR
from oracle import numerics
from oracle.model import OracleModel


@pytest.mark.slow
def test_bf16_noise_floor_llama7b_2layer():
    dims = synthetic.PRESETS["llama7b_2l"]
    w = synthetic.model_weights(dims, 0)
    prompt = synthetic.markov_prompt(dims.vocab, 65, 0)
    base = OracleModel(dims, w)
    ref = base.sequence_logits(prompt)
    floors = []
    for seed in (1, 2, 3):
        rng = np.random.default_rng(seed)

        class Perturbed(OracleModel):
            def s(self, x):
                x = np.asarray(x, np.float64)
                return numerics.round_to(x * (1 + 1e-7 * rng.standard_normal(x.shape)), self.dims.dtype)

        other = Perturbed(dims, w)
        other._cache = base._cache
        d = np.abs(other.sequence_logits(prompt) - ref)
        floors.append(float(d.max()))
        print(f"perturbation seed {seed}: max {d.max():.4f} mean {d.mean():.5f}")
    floor = max(floors)
    assert floor == pytest.approx(BF16_NOISE_FLOOR, abs=1e-4)
    # already above the single-operator bound: 2e-2 cannot be held at model level
    assert floor > 2e-2
    assert BF16_MODEL_LOGIT_TOL == math.ceil(2 * floor * 100) / 100
