"""A NumPy model of the attention kernel's softmax bookkeeping, on the CPU.

The kernel does not track a running maximum: each row takes a fixed
reference (the maximum of the first 32 scores it visits, among the keys it
can see), sums p = 2^(s - reference) in fp32, and lists for an exact two-pass
recomputation the rows whose sum says the reference was off. Pieces of a row
that several work-groups share are merged afterwards. This model follows
those steps (visit order, reference choice, fp32 exponentials, the listing
test, the merge) so that the listing rule can be checked against the plain
softmax of the oracle on planted inputs, with no GPU.

Two rules are modelled side by side:
  * "overflow only": list a row when its sum exceeds 2^100; merge pieces by
    their reference and sum, an empty piece keeping its reference;
  * "both ways" (the kernel's rule): also list a row that sees keys but sums
    below 2^-100, and merge pieces by log2 of their total weight, a piece
    with no visible key weighing 0.
Under the frame-causal mask the first case fails: a row that sees none of its
first 32 keys takes its reference from keys it cannot see, and if those score
far above what it can see every visible probability underflows to 0.
"""
import numpy as np

from oracle import mla_oracle as O

SUM_LIMIT, SUM_MIN = 2.0 ** 100, 2.0 ** -100


def visit_order(n_keys, tile, t_begin, t_end):
    """Key indices in the order a segment over tiles [t_begin, t_end) visits
    them: the last (possibly ragged) tile first, then the others in order."""
    tiles = [t_end - 1] + list(range(t_begin, t_end - 1))
    return [k for t in tiles for k in range(t * tile, min((t + 1) * tile, n_keys))]


def piece(s, visible, order):
    """One segment of one row: s are scores in log2 units (fp32), visible the
    row's mask, order the visit order. Returns (reference, l, o_weights, sees)
    with o_weights the fp32 probabilities by key (0 where not visited)."""
    s = np.asarray(s, np.float32)
    first = order[:32]
    vis_first = [k for k in first if visible[k]]
    ref = np.float32(max(s[k] for k in (vis_first or first)))
    p = np.zeros_like(s)
    for k in order:
        if visible[k]:
            p[k] = np.exp2(np.float32(s[k] - ref), dtype=np.float32)
    sees = any(visible[k] for k in order)
    return ref, np.float32(p.sum(dtype=np.float32)), p, sees


def whole_row(s, visible, order, rule):
    """Output weights of a row one work-group covers alone; None = listed for
    the exact recomputation."""
    ref, l, p, sees = piece(s, visible, order)
    ok = l <= SUM_LIMIT if rule == "overflow only" else (l <= SUM_LIMIT and (l >= SUM_MIN or not sees))
    if not ok:
        return None
    return p / l if l > 0 else np.zeros_like(p)


def merged_row(s, visible, orders, rule):
    """Output weights of a row whose keys were split between work-groups
    (one visit order per piece); None = listed."""
    pieces = [piece(s, visible, o) for o in orders]
    if rule == "overflow only":
        if any(not (l <= SUM_LIMIT) for _, l, _, _ in pieces):
            return None
        # empty pieces keep their reference; weight of piece g: 2^(r_g - M) l_g
        M = max(r for r, _, _, _ in pieces)
        ws = [np.exp2(np.float32(r - M), dtype=np.float32) * l for r, l, _, _ in pieces]
    else:
        if any(not (l <= SUM_LIMIT and (l >= SUM_MIN or not sees)) for _, l, _, sees in pieces):
            return None
        lw = [r + np.log2(l) if l > 0 else -np.inf for r, l, _, _ in pieces]
        M = max(lw)
        if M == -np.inf:
            return np.zeros_like(pieces[0][2])
        ws = [np.exp2(np.float32(x - M), dtype=np.float32) for x in lw]
    L = sum(ws)
    out = sum(w * (p / l if l > 0 else 0 * p) for w, (_, l, p, _) in zip(ws, pieces))
    return out / L if L > 0 else np.zeros_like(pieces[0][2])


def exact_weights(s, visible):
    """The oracle's masked two-pass softmax (log2 units -> natural: x ln 2)."""
    return O._masked_softmax_rows(np.asarray(s, np.float64)[None] * np.log(2.0), np.asarray(visible)[None])[0]


def _planted_row():
    """96 keys in three frames of 32 (tiles of 32): the row belongs to frame 0,
    so it sees keys 0..31. A segment visits the last tile (frame 2) first, so
    none of its first 32 keys is visible; one of them scores 300 (log2 units)
    above everything the row sees."""
    rng = np.random.default_rng(0)
    s = rng.standard_normal(96).astype(np.float32)
    s[70] = 300.0
    frames = np.repeat([0, 1, 2], 32)
    return s, frames <= 0


def test_overflow_only_rule_writes_a_zero_row_unlisted():
    s, visible = _planted_row()
    order = visit_order(96, 32, 0, 3)
    assert not visible[order[:32]].any()
    got = whole_row(s, visible, order, "overflow only")
    assert got is not None and not got.any()          # zeros, and not listed
    assert exact_weights(s, visible)[:32].sum() > 0.999  # the row does see keys


def test_both_ways_rule_lists_the_row():
    s, visible = _planted_row()
    order = visit_order(96, 32, 0, 3)
    assert whole_row(s, visible, order, "both ways") is None  # listed: the exact pass recomputes it


def test_rule_keeps_ordinary_rows_unlisted_and_exact():
    """Rows whose first visited keys are invisible but within the fp32 range
    of the visible ones are not listed and match the oracle."""
    rng = np.random.default_rng(1)
    frames = np.repeat([0, 1, 2], 32)
    for qf in (0, 1, 2):
        for scale in (1.0, 8.0):
            s = (rng.standard_normal(96) * scale).astype(np.float32)
            vis = frames <= qf
            order = visit_order(96, 32, 0, 3)
            got = whole_row(s, vis, order, "both ways")
            assert got is not None
            np.testing.assert_allclose(got, exact_weights(s, vis), rtol=2e-6, atol=1e-7)


def test_merge_with_an_empty_piece():
    """Split in two pieces: one holds only keys the row cannot see, led by a
    key scoring 300 above the rest; the old merge keeps that piece's reference
    as the maximum and the visible piece underflows to weight 0."""
    s, visible = _planted_row()
    orders = [visit_order(96, 32, 0, 1), visit_order(96, 32, 1, 3)]
    old = merged_row(s, visible, orders, "overflow only")
    assert old is not None and not old.any()
    new = merged_row(s, visible, orders, "both ways")
    np.testing.assert_allclose(new, exact_weights(s, visible), rtol=2e-6, atol=1e-7)


def test_merge_lists_a_piece_that_underflowed():
    """A piece whose visible keys sit far below its invisible reference is
    listed (the whole row goes to the exact pass)."""
    s, visible = _planted_row()
    # piece 0: tiles 0 and 2 of the row's keys in visit order 2, 0 (the
    # planted key leads, the visible frame-0 keys follow); piece 1: tile 1
    orders = [[k for k in range(64, 96)] + list(range(0, 32)), list(range(32, 64))]
    assert merged_row(s, visible, orders, "overflow only") is not None
    assert merged_row(s, visible, orders, "both ways") is None


def test_merge_matches_oracle_on_random_splits():
    rng = np.random.default_rng(2)
    frames = np.repeat([0, 1, 2, 3], 40)
    for trial in range(20):
        s = (rng.standard_normal(160) * 10).astype(np.float32)
        vis = frames <= rng.integers(0, 4)
        cut = sorted(rng.choice(np.arange(1, 5), 2, replace=False))
        bounds = [0] + list(cut) + [5]
        orders = [visit_order(160, 32, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
        got = merged_row(s, vis, orders, "both ways")
        assert got is not None
        np.testing.assert_allclose(got, exact_weights(s, vis), rtol=1e-5, atol=1e-7)
