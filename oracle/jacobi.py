"""Jacobi and Gauss-Seidel schedules on a triangular system.

"M7.3 - Lookahead Decoding", 0x02 and 0x02C: a Jacobi sweep updates every
coordinate from the previous vector, y_i^(r+1) = T_i(y_<i^(r)); a
Gauss-Seidel sweep consumes coordinates already updated in the same sweep.
Toy operator: T1 = 2, T2 = (y1 + 1) mod 10, T3 = (y1 + y2) mod 10,
T4 = (y3 + 1) mod 10, starting from [9, 9, 9, 9]: Jacobi needs four sweeps,
Gauss-Seidel reaches [2, 3, 5, 6] in one.
"""
from __future__ import annotations


def toy_T(i: int, y_before):
    """T_i reads only coordinates < i (triangular dependence); 0-based i."""
    if i == 0:
        return 2
    if i == 1:
        return (y_before[0] + 1) % 10
    if i == 2:
        return (y_before[0] + y_before[1]) % 10
    if i == 3:
        return (y_before[2] + 1) % 10
    raise IndexError(i)


def jacobi_sweep(T, y):
    old = list(y)
    return [T(i, old[:i]) for i in range(len(old))]


def gauss_seidel_sweep(T, y):
    new = list(y)
    for i in range(len(new)):
        new[i] = T(i, new[:i])
    return new


def solve(T, y0, sweep, max_sweeps=100):
    """Iterate until a fixed point; returns (fixed point, trajectory of sweeps)."""
    traj = []
    y = list(y0)
    for _ in range(max_sweeps):
        y2 = sweep(T, y)
        traj.append(y2)
        if y2 == y:
            traj.pop()
            return y, traj
        y = y2
    raise RuntimeError("no fixed point")
