"""Packed-row compiler: row records, logical positions, branch visibility, slices.

"M7.3 - Lookahead Decoding", 0x04 and 0x04A:

* one step packs [1 ordinary row] + [lookahead trajectory rows] + [C
  candidate suffixes x S rows]; the dense path orders lookahead rows level by
  level (level-major), candidates after them, candidate-major;
* the current row plus level 0 form the base stripe b_0..b_{W-1}; u_(r,j) is
  trajectory level r > 0 at column j; v_(c,s) is candidate c at offset s;
* visibility (besides the committed prefix, which every row sees):
      Vis(b_j)    = {b_k : k <= j}
      Vis(u_(r,j)) = {b_k : k <= j} U {u_(q,j) : 1 <= q <= r}
      Vis(v_(c,s)) = {b_0} U {v_(c,q) : q <= s}
  with no edges between branches or between candidates;
* one shared row record (packed index, role, level, column, candidate,
  offset, logical position, requested logit) feeds tokens, positions, mask
  and output slices alike;
* slices: out = the ordinary row, inp = the deepest trajectory level's rows,
  guess = all verification rows.

Logical positions (the pages describe them only in words: the ordinary row
takes the next committed position, a lookahead row the future position its
window column stands for, a verification row the prefix length plus its
offset): with p the ordinary row's position,
    pos(b_j) = p + j,   pos(u_(r,j)) = p + j + r,   pos(v_(c,s)) = p + 1 + s.
This is the only choice under which the n-gram extraction of 0x03B and the
window shift of 0x03C keep every cell at the position it was predicted for.

Level cells: level 0 holds b_1.. (columns 1..len); level r >= 1 holds columns
start_r .. start_r + len - 1.  The pinned steady layout has start_r = 0 for
r >= 1; the rectangular semantic window (every level at columns 1..W, the
current row as an extra base cell) has start_r = 1.
"""
from __future__ import annotations

import dataclasses

import numpy as np

ORDINARY, LOOKAHEAD, VERIFY = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Row:
    packed_index: int
    role: int              # ORDINARY | LOOKAHEAD | VERIFY
    level: int             # trajectory level (lookahead; base stripe cells are level 0), else -1
    column: int            # window column (ordinary row is column 0 of the base stripe), else -1
    candidate: int         # verify only, else -1
    offset: int            # verify only, else -1
    logical_position: int
    request_logit: bool
    token: int

    @property
    def identity(self):
        """Semantic identity, independent of physical packing order."""
        return (self.role, self.level, self.column, self.candidate, self.offset)


@dataclasses.dataclass
class CompiledRound:
    rows: list
    visible: np.ndarray        # [Q, Q] bool, among current rows (prefix always visible)
    out: int                   # packed index of the ordinary row
    inp: list                  # packed indices of the deepest level, column order
    guess: list                # packed indices of verification rows, (candidate, offset) order
    S: int
    C: int

    @property
    def Q(self):
        return len(self.rows)

    @property
    def tokens(self):
        return [r.token for r in self.rows]

    @property
    def positions(self):
        return [r.logical_position for r in self.rows]


def compile_round(x_t: int, p: int, levels, candidates, S: int, starts=None) -> CompiledRound:
    """Compile one round.

    levels: list of per-level token lists (None for a level not materialised
    yet); level 0 is the base stripe after the current token.  starts: start
    column of each level r >= 1 (default 0).  candidates: list of S-token
    suffixes retrieved for key x_t.
    """
    R = len(levels)
    if starts is None:
        starts = [1] + [0] * (R - 1)
    rows = []
    # ordinary row b_0
    rows.append(dict(role=ORDINARY, level=0, column=0, candidate=-1, offset=-1, pos=p, token=x_t))
    present = [lv is not None for lv in levels]
    deepest = max(r for r in range(R) if present[r]) if any(present) else -1
    # lookahead rows, level-major
    for r in range(R):
        if levels[r] is None:
            continue
        st = 1 if r == 0 else starts[r]
        for i, tok in enumerate(levels[r]):
            j = st + i
            rows.append(dict(role=LOOKAHEAD, level=r, column=j, candidate=-1, offset=-1,
                             pos=p + j + r, token=int(tok)))
    # verification rows, candidate-major
    for c, suf in enumerate(candidates):
        assert len(suf) == S
        for s in range(S):
            rows.append(dict(role=VERIFY, level=-1, column=-1, candidate=c, offset=s,
                             pos=p + 1 + s, token=int(suf[s])))
    Q = len(rows)
    # visibility from the Vis sets
    vis = np.zeros((Q, Q), bool)

    def is_base(rw, k=None):
        if rw["role"] == ORDINARY:
            return k is None or k == 0
        return rw["role"] == LOOKAHEAD and rw["level"] == 0 and (k is None or rw["column"] == k)

    for i, a in enumerate(rows):
        for jx, b in enumerate(rows):
            if a["role"] == VERIFY:
                ok = (b["role"] == ORDINARY) or (b["role"] == VERIFY and b["candidate"] == a["candidate"]
                                                 and b["offset"] <= a["offset"])
            elif is_base(a):                       # b_j
                ja = a["column"]
                ok = is_base(b) and b["column"] <= ja
            else:                                  # u_(r,j), r >= 1
                ja, ra = a["column"], a["level"]
                ok = (is_base(b) and b["column"] <= ja) or (
                    b["role"] == LOOKAHEAD and b["level"] >= 1 and b["level"] <= ra and b["column"] == ja)
            vis[i, jx] = ok
    out = 0
    inp = [i for i, rw in enumerate(rows) if rw["role"] == LOOKAHEAD and rw["level"] == deepest]
    guess = [i for i, rw in enumerate(rows) if rw["role"] == VERIFY]
    req = set([out] + inp + guess)
    recs = [Row(i, rw["role"], rw["level"] if rw["role"] != VERIFY else -1,
                rw["column"] if rw["role"] != VERIFY else -1, rw["candidate"], rw["offset"],
                rw["pos"], i in req, rw["token"]) for i, rw in enumerate(rows)]
    return CompiledRound(recs, vis, out, inp, guess, S, len(candidates))


def pinned_row_counts(W: int, N: int, C: int):
    """Steady pinned ledger ("M7.3", 0x01A and 0x05C): Q_LA = W(N-1)-1, Q_V = C(N-1), Q = (W+C)(N-1)."""
    q_la = W * (N - 1) - 1
    q_v = C * (N - 1)
    return q_la, q_v, 1 + q_la + q_v
