"""Jacobi trajectory window: depth admission, warmup fill, steady advance.

"M7.3 - Lookahead Decoding":
* 0x01A -- the pinned multilevel schedule is defined for integer N >= 3
  (S = R = N - 1); anything else is refused before any state is built;
* 0x03A -- warmup: level 0 starts with W + N - 3 cells; each fill shifts the
  existing levels left by one and turns the deepest level's outputs into a
  new, deeper level, which loses its first output where needed (the page's
  N=4, W=5 trace: sizes [6,-,-] -> [5,6,-] -> [4,5,5]); no verification
  meanwhile;
* 0x03C -- steady advance under ALWAYS_FWD_ONE: one column per round
  whatever was accepted, keeping the ragged sizes [W-1, W, ..., W]; the
  page also names, in words only, a variant that slices the levels by the
  accepted count and refills the emptied slots.

Coordinates used below (reading 18 of the build's notes): with the live token
at logical position p, level r holds the cell of column j at position
p + j + r; level 0 holds columns 1..W-1 (column 0 is the live token itself),
deeper levels columns 0..W-1.  Each rule is written as "which old cell (or
new output) lands at each new cell"; every cell keeps the position it was
predicted for.

Readings (the pages leave these open):
* initial level-0 content: the page only says the lookahead slots are seeded
  from the prompt; read as the last W + N - 3 prompt tokens, cycling when
  the prompt is shorter;
* the new warmup level loses its first output exactly when the level it was
  computed from has index >= 1 (the only reading that reproduces the page's
  [5,6,-] -> [4,5,5] and keeps positions);
* ALWAYS_FWD_ONE=False: after the one-column advance (the one position every
  round publishes), each level drops its first h cells (the h accepted
  tokens moved the live position h further) and is refilled at its tail with
  h copies of the newest committed token (the page lists copying the last
  token among the seed choices); sizes are kept.  Warmup fills are unchanged.
"""
from __future__ import annotations


def admitted_depth(N) -> int:
    """S = R = N - 1 for an admitted depth (0x01A).

    Depth 2 would leave one trajectory level, while the first warmup fill and
    the steady advance both read a second one; such a schedule (and any
    non-integer N) is refused before state exists.
    """
    if isinstance(N, bool) or not isinstance(N, int) or N < 3:
        raise ValueError(f"N={N!r}: the multilevel schedule takes an integer depth of at least 3")
    return N - 1


def _check_width(W):
    if isinstance(W, bool) or not isinstance(W, int) or W < 1:
        raise ValueError(f"W={W!r}: the window needs at least one column")


def init_window(prompt, W: int, N: int):
    R = admitted_depth(N)
    _check_width(W)
    n0 = W + N - 3
    P = len(prompt)
    level0 = [int(prompt[(P - n0 + i) % P]) for i in range(n0)]
    return [level0] + [None] * (R - 1)


def level_sizes(window):
    return [None if lv is None else len(lv) for lv in window]


def is_warm(window) -> bool:
    return all(lv is not None for lv in window)


def deepest_level(window) -> int:
    return max(r for r, lv in enumerate(window) if lv is not None)


def fill_window(window, z):
    """One warmup fill: shift existing levels left by one, append the new level."""
    d = deepest_level(window)
    assert d + 1 < len(window), "window already warm"
    new = [lv[1:] for lv in window[:d + 1]]
    new.append(list(z[1:]) if d >= 1 else list(z))
    return new + [None] * (len(window) - len(new))


def advance_one_column(window, z, N, W):
    """Steady advance by one column (ALWAYS_FWD_ONE).

    The live position moves from p to p + 1, so new cell (r, j) at position
    p + 1 + j + r is old cell (r + 1, j), and the deepest new level is the
    outputs z (old deepest cell (R - 1, j) predicted position p + j + R).
    Old level 0 and old cell (1, 0) -- the new live token's position -- drop
    out.  The warm ragged layout and W outputs are required.
    """
    R = admitted_depth(N)
    _check_width(W)
    want = [W - 1] + [W] * (R - 1)
    if len(window) != R or level_sizes(window) != want:
        raise ValueError(f"level sizes {level_sizes(window)} differ from the warm layout {want}")
    if len(z) != W:
        raise ValueError(f"{len(z)} outputs for a {W}-column window")

    def old(r, j):                 # old level r at column j (level 0 starts at column 1)
        return window[r][j - 1] if r == 0 else window[r][j]

    new = []
    for r in range(R):
        cols = range(1, W) if r == 0 else range(W)
        new.append([int(z[j]) if r == R - 1 else old(r + 1, j) for j in cols])
    return new


def advance_by_accepted(window, z, N, W, h: int, fill: int):
    """ALWAYS_FWD_ONE=False: the one-column advance, then every level drops
    its first h cells and is refilled at its tail with `fill`."""
    out = []
    for lv in advance_one_column(window, z, N, W):
        k = min(int(h), len(lv))
        out.append(lv[k:] + [int(fill)] * k)
    return out


def next_window(window, z, N, W, h: int = 0, fill=None):
    """Warmup fill while levels are missing, otherwise the steady advance
    (by the accepted count h when `fill` is given, ALWAYS_FWD_ONE=False)."""
    if is_warm(window):
        if fill is not None:
            return advance_by_accepted(window, z, N, W, h, fill)
        return advance_one_column(window, z, N, W)
    return fill_window(window, z)
