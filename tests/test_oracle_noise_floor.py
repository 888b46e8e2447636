"""bf16 rounding noise floor of the 7B-width 2-layer model (CPU, slow).

Runs the oracle twice: as is, and with every pre-rounding value perturbed by
a relative N(0, 1e-7) -- the size of the difference between fp32 and fp64
accumulation.  The logit disagreement between the two is the floor below
which no bf16 implementation with a different summation order can be held;
the GPU model-level tolerance is set at twice this floor.
"""
import numpy as np
import pytest

import synthetic
from oracle import numerics
from oracle.model import OracleModel


@pytest.mark.slow
def test_bf16_noise_floor_llama7b_2layer():
    dims = synthetic.PRESETS["llama7b_2l"]
    w = synthetic.model_weights(dims, 0)
    prompt = synthetic.markov_prompt(dims.vocab, 65, 0)
    base = OracleModel(dims, w)
    ref = base.sequence_logits(prompt)

    class Perturbed(OracleModel):
        def s(self, x):
            x = np.asarray(x, np.float64)
            return numerics.round_to(x * (1 + 1e-7 * rng.standard_normal(x.shape)), self.dims.dtype)

    rng = np.random.default_rng(1)
    other = Perturbed(dims, w)
    other._cache = base._cache
    d = np.abs(other.sequence_logits(prompt) - ref)
    print(f"noise floor: max {d.max():.4f} mean {d.mean():.4f}")
    assert 0.005 < d.max() < 0.04          # measured 0.035; the GPU bound (0.07) is twice this floor
