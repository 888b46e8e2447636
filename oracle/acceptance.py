"""Expected accepted tokens under the paper's survival model.

"M7.3 - Lookahead Decoding", 0x05C (and the paper summary, 4.2 / App. C):
one proposal of length gamma, each token surviving independently with
probability alpha, progress always including the ordinary token:
    E[R_1] = sum_{j=0..gamma} alpha^j = (1 - alpha^(gamma+1)) / (1 - alpha);
b independent candidates, maximum progress R_b:
    P(R_b >= i + 1) = 1 - (1 - alpha^i)^b,
    E[R_b] = (gamma + 1) - sum_{i=1..gamma} (1 - alpha^i)^b;
one good round in f:  S_steps = (f - 1 + E[R_b]) / f.
"""
from __future__ import annotations


def expected_single(alpha: float, gamma: int) -> float:
    return sum(alpha ** j for j in range(gamma + 1))


def expected_batch(alpha: float, gamma: int, b: int) -> float:
    return (gamma + 1) - sum((1 - alpha ** i) ** b for i in range(1, gamma + 1))


def step_compression(f: float, e_rb: float) -> float:
    return (f - 1 + e_rb) / f
