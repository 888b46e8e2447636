"""Jacobi trajectory window: depth admission, warmup fill, pinned advance.

"M7.3 - Lookahead Decoding":
* 0x01A -- the illustrated pinned schedule needs an integer N >= 3
  (S = R = N - 1), otherwise ValueError, before any state is built;
* 0x03A -- warmup: level 0 starts with W + N - 3 cells; at each fill the
  existing levels shift left by one and the deepest level's outputs become a
  new, deeper level, the new level dropping its first output where needed
  (N=4, W=5: [6,-,-] -> [5,6,-] -> [4,5,5]); no verification meanwhile;
* 0x03C -- steady advance with ALWAYS_FWD_ONE: new window is
  [past[1][1:]] + past[2:] + [z], keeping the ragged sizes [W-1, W, ..., W];
  its alternative (ALWAYS_FWD_ONE=False) slices each level by the accepted
  count and refills the tail (0x03C, 0x06C "drop positions consumed by
  committed output, shift the remaining future slots left, refill vacated
  slots from the configured seed/reset source").

Readings (the pages leave these open):
* initial level-0 content: "seeds lookahead slots from prompt tokens" is
  read as the last W + N - 3 prompt tokens, cycling if the prompt is short;
* "drops its first output where needed" is read as: the new level drops its
  first output exactly when the level it was computed from has index >= 1
  (the only reading that reproduces [5,6,-] -> [4,5,5] and keeps every cell
  at the position it was predicted for);
* ALWAYS_FWD_ONE=False: after the pinned advance, which accounts for the
  one position every round publishes, each level drops its first h entries
  (the h accepted tokens moved the live position h further) and appends h
  copies of the newest committed token (the page lists "copy the last
  token" among the seed choices); the ragged sizes are kept, and every
  surviving cell stays at the position it was predicted for.  Warmup fills
  are unchanged.
"""
from __future__ import annotations


def pinned_suffix_length(N) -> int:
    """S = R = N - 1, admitted only for integer N >= 3 (0x01A).

    N = 2 would leave a single trajectory level, but both the first warmup
    fill and the steady advance read a second level, so it is refused before
    any state exists.
    """
    admitted = isinstance(N, int) and not isinstance(N, bool) and N >= 3
    if not admitted:
        raise ValueError(f"depth N={N!r} not admitted: the pinned schedule needs an integer N >= 3")
    return N - 1


def init_window(prompt, W: int, N: int):
    R = pinned_suffix_length(N)
    if not isinstance(W, int) or W < 1:
        raise ValueError("window width must be a positive integer")
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


def advance_pinned_window(window, z, N, W):
    """Steady ALWAYS_FWD_ONE advance (one column per round, whatever was accepted).

    Time axis: the oldest level is dropped and every other level moves up one;
    sequence axis: the level that becomes level 0 loses its first column,
    because the live token now stands in for it; the new outputs z become the
    deepest level.  Shapes are checked first: R levels, ragged [W-1, W, ..., W],
    and W outputs.
    """
    R = pinned_suffix_length(N)
    if not isinstance(W, int) or W < 1:
        raise ValueError("window width must be a positive integer")
    expected = [W - 1] + [W] * (R - 1)
    if len(window) != R or level_sizes(window) != expected:
        raise ValueError(f"window sizes {level_sizes(window)} are not the warm layout {expected}")
    if len(z) != W:
        raise ValueError(f"{len(z)} new outputs, expected W={W}")
    promoted = [list(window[r]) for r in range(2, R)]
    return [list(window[1])[1:], *promoted, list(z)]


def advance_by_accepted(window, z, N, W, h: int, fill: int):
    """ALWAYS_FWD_ONE=False: the pinned advance, then every level drops its
    first h entries and its tail is refilled with `fill`."""
    out = []
    for lv in advance_pinned_window(window, z, N, W):
        k = min(int(h), len(lv))
        out.append(lv[k:] + [int(fill)] * k)
    return out


def next_window(window, z, N, W, h: int = 0, fill=None):
    """Warmup fill while levels are missing, otherwise the steady advance
    (by the accepted count h when `fill` is given, ALWAYS_FWD_ONE=False)."""
    if is_warm(window):
        if fill is not None:
            return advance_by_accepted(window, z, N, W, h, fill)
        return advance_pinned_window(window, z, N, W)
    return fill_window(window, z)
