"""Oracle: bitmap-aware row reordering of IE-BME local tiles.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the library.

Source: "UnionSparse" page, section on bitmap-aware row reordering (the
objective, the grouped cost formulation, the grouped subset dynamic
programming and the canonicalisation of its result).

What is computed, per local tile (LT) W_t of H_L x K_L with an R_A x C_A area
grid (areas of H_L/R_A x K_L/C_A):
  * a row group is a set of R_A rows of the LT; its grouped cost is the number
    of grouped columns j in [0, K_L/C_A) at which any of its rows is nonzero
    in any of the C_A column partitions (the union-mask entries the group
    activates);
  * F(S) over sets S of ungrouped rows (|S| a multiple of R_A): F({}) = 0,
    F(S) = min over groups g of R_A rows of S that contain the smallest row of
    S of cost(g) + F(S minus g); F(all rows) is the least number of active
    union-mask entries any row arrangement gives;
  * the optimal groups, each sorted ascending and the groups sorted
    lexicographically, are laid out partition-wise: partition p (rows
    p*G .. p*G + G - 1, G = H_L/R_A) holds the p-th row of every group in
    group order.  Logical row i of the union mask then groups the rows
    i, i + G, ..., exactly the rows of group i.
Ties between groups of equal total cost are broken by the enumeration order:
groups containing the smallest row are tried with their other rows in
lexicographic order, and the first minimum is kept (the pages leave ties
open; any minimum is valid).
"""
from __future__ import annotations

from functools import lru_cache
from itertools import combinations, permutations
from typing import List, Tuple

import numpy as np


def folded_rows(B: np.ndarray, c_a: int) -> List[int]:
    """Per row, the OR over the C_A column partitions as an integer bit set
    over the grouped columns (bit j = grouped column j)."""
    H, KL = B.shape
    ak = KL // c_a
    out = []
    for r in range(H):
        bits = 0
        for j in range(ak):
            if any(B[r, a * ak + j] for a in range(c_a)):
                bits |= 1 << j
        out.append(bits)
    return out


def grouped_cost(B: np.ndarray, rows, c_a: int) -> int:
    """Active union-mask entries of the group ``rows`` (the grouped cost)."""
    u = folded_rows(B, c_a)
    acc = 0
    for r in rows:
        acc |= u[r]
    return bin(acc).count("1")


def solve_lt(B: np.ndarray, r_a: int, c_a: int) -> Tuple[int, List[Tuple[int, ...]]]:
    """Subset DP of one LT: (minimum grouped cost, canonical groups)."""
    H = B.shape[0]
    if H % r_a or B.shape[1] % c_a:
        raise ValueError("LT shape must be divisible by the area grid")
    u = folded_rows(B, c_a)

    def cost(g):
        acc = 0
        for r in g:
            acc |= u[r]
        return bin(acc).count("1")

    @lru_cache(maxsize=None)
    def F(S: int) -> Tuple[int, Tuple[Tuple[int, ...], ...]]:
        if S == 0:
            return 0, ()
        rows = [r for r in range(H) if (S >> r) & 1]
        r0, rest = rows[0], rows[1:]
        best = None
        for others in combinations(rest, r_a - 1):
            g = (r0,) + others
            mask = 0
            for r in g:
                mask |= 1 << r
            sub_cost, sub_groups = F(S & ~mask)
            c = cost(g) + sub_cost
            if best is None or c < best[0]:
                best = (c, (g,) + sub_groups)
        return best

    total, groups = F((1 << H) - 1)
    canon = sorted(tuple(sorted(g)) for g in groups)
    return total, canon


def permutation_from_groups(groups: List[Tuple[int, ...]], r_a: int) -> List[int]:
    """perm[i] = the LT row placed at row i: partition p lists the p-th row
    of every group, groups in order."""
    return [g[p] for p in range(r_a) for g in groups]


def union_actives(B: np.ndarray, r_a: int, c_a: int) -> int:
    """Active union-mask entries of an LT as it stands: logical row i groups
    rows i, i + G, ... (G = H_L / R_A), as the IE-BME encoder does."""
    H = B.shape[0]
    G = H // r_a
    return sum(grouped_cost(B, [i + p * G for p in range(r_a)], c_a) for i in range(G))


def reorder_lt(B: np.ndarray, r_a: int, c_a: int) -> Tuple[List[int], int]:
    """(row permutation, active entries after it) for one LT."""
    total, groups = solve_lt(B, r_a, c_a)
    return permutation_from_groups(groups, r_a), total


def reorder_matrix(mask: np.ndarray, lt_m: int, lt_k: int, r_a: int, c_a: int):
    """Every LT independently (row-major LT order): perms [NLT][lt_m] of
    LT-local rows, active entries before and after, per LT."""
    M, K = mask.shape
    perms, before, after = [], [], []
    for ti in range(M // lt_m):
        for tj in range(K // lt_k):
            B = mask[ti * lt_m:(ti + 1) * lt_m, tj * lt_k:(tj + 1) * lt_k]
            p, a = reorder_lt(B, r_a, c_a)
            perms.append(p)
            before.append(union_actives(B, r_a, c_a))
            after.append(a)
    return np.array(perms, dtype=np.int32), np.array(before, dtype=np.int32), np.array(after, dtype=np.int32)


def brute_force_min(B: np.ndarray, r_a: int, c_a: int) -> int:
    """Least active count over every row permutation (tiny LTs only): each
    permutation is applied and the union mask of the result counted."""
    H = B.shape[0]
    G = H // r_a
    u = folded_rows(B, c_a)
    best = None
    for perm in permutations(range(H)):
        total = 0
        for i in range(G):
            acc = 0
            for p in range(r_a):
                acc |= u[perm[i + p * G]]
            total += bin(acc).count("1")
        best = total if best is None else min(best, total)
    return best
