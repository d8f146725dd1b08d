"""Pins for the oracle's top-8, gate and dedup table: brute force written
differently from the oracle (a full sort, a set scan), on random and on
tie-heavy inputs, plus the ordering rules the pages state (ties to the lower
expert ID; owner = first job, lowest row on a tie)."""
import numpy as np
import pytest

from oracle import oracle as O


def _brute_top8(z):
    """Full sort by (NaN last, value descending, id ascending)."""
    z = np.asarray(z, np.float64)
    ids = np.arange(z.size)
    isn = np.isnan(z)
    zz = np.where(isn, 0.0, z) + 0.0       # +0.0 folds -0 into +0
    order = np.lexsort((ids, -zz, isn))    # last key is primary
    return order[:8].astype(np.int32)


@pytest.mark.parametrize("E", [8, 9, 32, 256])
def test_top8_random(E):
    rng = np.random.default_rng(E)
    for _ in range(200):
        z = rng.standard_normal(E)
        assert np.array_equal(O.top8(z), _brute_top8(z))


def test_top8_heavy_ties():
    rng = np.random.default_rng(7)
    for E in (8, 16, 256):
        for _ in range(200):
            z = rng.integers(-3, 4, size=E).astype(np.float64)  # many exact ties
            assert np.array_equal(O.top8(z), _brute_top8(z))


def test_top8_signed_zero_ties_go_to_lower_id():
    z = np.full(16, -1.0)
    z[3], z[9], z[12] = -0.0, 0.0, -0.0
    got = O.top8(z)
    assert list(got[:3]) == [3, 9, 12]
    assert list(got[3:]) == [0, 1, 2, 4, 5]


def test_top8_nan_ranks_last():
    z = np.full(12, np.nan)
    z[5], z[7] = -1e30, -np.inf
    got = O.top8(z)
    assert list(got) == [5, 7, 0, 1, 2, 3, 4, 6]
    rng = np.random.default_rng(3)
    for _ in range(100):
        z = rng.standard_normal(32)
        z[rng.integers(0, 32, 6)] = np.nan
        assert np.array_equal(O.top8(z), _brute_top8(z))


def test_top8_duplicate_router_rows_tie_exactly():
    # two experts with identical router rows produce identical logits: the
    # lower ID must come first (#85 Mod. row 9: ID reduction only on ties)
    z = np.array([0.1, 0.5, 0.3, 0.5, 0.2, 0.5, 0.0, -0.1, 0.4])
    assert list(O.top8(z)) == [1, 3, 5, 8, 2, 4, 0, 6]


def test_softmax8_matches_numpy_and_sums_to_one():
    rng = np.random.default_rng(11)
    for _ in range(100):
        z = rng.standard_normal(8) * 5
        g = O.softmax8(z)
        ref = np.exp(z) / np.exp(z).sum()
        assert np.allclose(g, ref, rtol=1e-14, atol=0)
        assert abs(g.sum() - 1.0) < 1e-15 * 8
    g = O.softmax8(np.array([1000.0] + [0.0] * 7))   # no overflow
    assert g[0] == 1.0 and np.all(g[1:] == 0.0)


def _brute_dedup(ids):
    """Set-based: the distinct experts, each placed at its first pick in
    slot-major order (slot, row); mask and per-row slots from a full scan."""
    ids = np.asarray(ids)
    R = ids.shape[0]
    first = {}
    for e in set(ids.ravel().tolist()):
        pos = [(j, r) for r in range(R) for j in range(8) if ids[r, j] == e]
        first[e] = min(pos)
    experts = sorted(first, key=lambda e: first[e])
    mask = [sum(1 << r for r in range(R) if e in ids[r]) for e in experts]
    slot = np.full((len(experts), 8), 0xFF, np.uint8)
    for g, e in enumerate(experts):
        for r in range(R):
            hit = np.where(ids[r] == e)[0]
            if hit.size:
                slot[g, r] = hit[0]
    return experts, [first[e] for e in experts], mask, slot


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_dedup_against_brute_force(R):
    rng = np.random.default_rng(100 + R)
    for E in (8, 12, 32, 256):
        for _ in range(50):
            ids = np.stack([rng.permutation(E)[:8] for _ in range(R)]).astype(np.int32)
            t = O.dedup(ids)
            experts, firsts, mask, slot = _brute_dedup(ids)
            assert t["n"] == len(experts) <= min(8 * R, E)
            assert list(t["expert"]) == experts
            assert [(int(a), int(b)) for a, b in zip(t["owner_slot"], t["owner_row"])] == firsts
            assert list(t["mask"]) == mask
            assert np.array_equal(t["slot"], slot)


def test_dedup_owner_rule_example():
    # row 1 picks expert 7 in slot 0, row 0 picks it in slot 2: the owner is
    # the earliest job (slot 0, row 1).  Expert 3 is slot 1 for both rows: the
    # owner is the lowest row (row 0).
    ids = np.array([[1, 3, 7, 4, 5, 6, 8, 9], [7, 3, 2, 10, 11, 12, 13, 14]], np.int32)
    t = O.dedup(ids)
    g7 = list(t["expert"]).index(7)
    g3 = list(t["expert"]).index(3)
    assert (t["owner_slot"][g7], t["owner_row"][g7]) == (0, 1)
    assert (t["owner_slot"][g3], t["owner_row"][g3]) == (1, 0)
    assert t["mask"][g7] == 3 and list(t["slot"][g7][:2]) == [2, 0]
    assert t["n"] == 14


def test_dedup_identical_rows_collapse():
    ids = np.tile(np.arange(8, dtype=np.int32)[::-1], (8, 1))
    t = O.dedup(ids)
    assert t["n"] == 8 and all(m == 0xFF for m in t["mask"])
    assert list(t["expert"]) == list(range(8))[::-1]
