"""Brute-force top-k by enumeration, for tiny E.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[Appendix C, Core MoE symbols] T_k(x) is the set of the k top-scoring experts.
Enumerates every k-subset, keeps those of maximal total score (exact rational
sums of the float64 scores, so no rounding can fake or hide a tie) and among
them picks the lexicographically smallest sorted index tuple, which is the
lowest-index tie-break.  Returned in (score desc, index asc) order.
"""
from __future__ import annotations

import itertools
from fractions import Fraction
from typing import Sequence, Tuple


def brute_topk(scores: Sequence[float], k: int) -> Tuple[int, ...]:
    s = [Fraction(float(v)) for v in scores]
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(s)), k):   # lexicographic order
        tot = sum((s[i] for i in comb), Fraction(0))
        if best_sum is None or tot > best_sum:
            best, best_sum = comb, tot
    return tuple(sorted(best, key=lambda i: (-s[i], i)))
