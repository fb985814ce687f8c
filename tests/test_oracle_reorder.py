"""Pins of the bitmap-aware row-reordering oracle ("UnionSparse", section on
bitmap-aware row reordering): brute force over every row permutation of
tiny LTs, the union mask the IE-BME encoder builds from the reordered LT,
closed forms and a hand-worked case.  A planted greedy solver and a planted
cost that ignores column partitions must fail."""
import numpy as np
import pytest

from oracle import ie_bme as ou
from oracle import row_reorder as rr
from oracle import tca_bme as ob


def random_lt(H, KL, density, seed):
    rng = np.random.default_rng(seed)
    return rng.random((H, KL)) < density


@pytest.mark.parametrize("H,r_a,c_a", [(4, 2, 1), (6, 2, 2), (6, 3, 1), (8, 2, 2), (8, 4, 1), (8, 2, 1)])
@pytest.mark.parametrize("seed", range(4))
def test_dp_minimum_equals_brute_force(H, r_a, c_a, seed):
    density = [0.1, 0.25, 0.4, 0.6][seed]
    B = random_lt(H, 16 if c_a == 1 else 32, density, 100 * H + 10 * r_a + c_a + seed)
    total, groups = rr.solve_lt(B, r_a, c_a)
    assert total == rr.brute_force_min(B, r_a, c_a)


@pytest.mark.parametrize("H,KL,r_a,c_a", [(8, 64, 2, 2), (16, 64, 2, 2), (12, 32, 3, 2), (16, 64, 4, 1)])
def test_permutation_realises_the_minimum_in_the_ie_bme_encoder(H, KL, r_a, c_a):
    """The permuted LT, encoded by the IE-BME oracle, stores exactly Q x
    (minimum) payload elements; the permutation is a bijection laid out
    partition-wise from sorted groups."""
    B = random_lt(H, KL, 0.3, H + KL + r_a)
    perm, total = rr.reorder_lt(B, r_a, c_a)
    assert sorted(perm) == list(range(H))
    _, groups = rr.solve_lt(B, r_a, c_a)
    assert groups == sorted(groups) and all(list(g) == sorted(g) for g in groups)
    G = H // r_a
    assert [perm[i + p * G] for i in range(G) for p in range(r_a)] == [r for g in groups for r in g]
    W = np.where(B, np.float16(1.0), np.float16(0.0)).astype(np.float16)
    Q = r_a * c_a
    enc_after = ou.encode_union(W[perm], B[perm], H, KL, r_a, c_a, ob.VAL_I4)
    assert enc_after.payload == Q * total
    enc_before = ou.encode_union(W, B, H, KL, r_a, c_a, ob.VAL_I4)
    assert enc_before.payload == Q * rr.union_actives(B, r_a, c_a) >= enc_after.payload


def test_hand_worked_case():
    """Rows 0, 1 share columns 0-1 and rows 2, 3 share columns 2-3.  The
    natural grouping (0, 2), (1, 3) activates 4 + 4 entries; grouping (0, 1),
    (2, 3) activates 2 + 2, laid out as rows [0, 2, 1, 3]."""
    B = np.array([[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]], bool)
    assert rr.union_actives(B, 2, 1) == 8
    perm, total = rr.reorder_lt(B, 2, 1)
    assert total == 4
    assert perm == [0, 2, 1, 3]
    assert rr.union_actives(B[perm], 2, 1) == 4


def test_single_row_groups_keep_the_identity():
    """R_A = 1: every row is its own group, nothing to gain; the canonical
    permutation is the identity and the cost is the sum of folded rows."""
    B = random_lt(10, 32, 0.3, 5)
    perm, total = rr.reorder_lt(B, 1, 2)
    assert perm == list(range(10))
    folded = B[:, :16] | B[:, 16:]
    assert total == int(folded.sum())


def test_empty_and_full_lts():
    B = np.zeros((8, 32), bool)
    assert rr.reorder_lt(B, 2, 2)[1] == 0
    B = np.ones((8, 32), bool)
    assert rr.reorder_lt(B, 2, 2)[1] == 4 * 16
    assert rr.reorder_lt(B, 2, 2)[0] == [0, 2, 4, 6, 1, 3, 5, 7]


def test_reorder_matrix_is_per_lt():
    mask = random_lt(32, 128, 0.3, 9)
    perms, before, after = rr.reorder_matrix(mask, 16, 64, 2, 2)
    assert perms.shape == (4, 16)
    for t in range(4):
        ti, tj = divmod(t, 2)
        B = mask[ti * 16:(ti + 1) * 16, tj * 64:(tj + 1) * 64]
        assert after[t] == rr.union_actives(B[perms[t]], 2, 2) <= before[t] == rr.union_actives(B, 2, 2)


def _greedy(B, r_a, c_a):
    """Planted mistake: pair each smallest remaining row with its cheapest
    partner, no look-ahead (R_A = 2)."""
    u = rr.folded_rows(B, c_a)
    left = list(range(B.shape[0]))
    total = 0
    while left:
        r = left.pop(0)
        best = min(left, key=lambda s: bin(u[r] | u[s]).count("1"))
        left.remove(best)
        total += bin(u[r] | u[best]).count("1")
    return total


def test_planted_greedy_fails_brute_force():
    bad = 0
    for seed in range(40):
        B = random_lt(8, 16, 0.3, 1000 + seed)
        if _greedy(B, 2, 1) != rr.brute_force_min(B, 2, 1):
            bad += 1
    assert bad > 0


def test_planted_unfolded_cost_fails_the_encoder_check():
    """Planted mistake: a cost that looks at the first column partition only."""
    B = random_lt(8, 64, 0.3, 77)
    unfolded = rr.folded_rows(B[:, :32], 1)
    G = 4
    wrong = sum(bin(unfolded[i] | unfolded[i + G]).count("1") for i in range(G))
    W = np.where(B, np.float16(1.0), np.float16(0.0)).astype(np.float16)
    enc = ou.encode_union(W, B, 8, 64, 2, 2, ob.VAL_I4)
    assert enc.payload == 4 * rr.union_actives(B, 2, 2) != 4 * wrong
