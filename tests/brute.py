"""Brute-force node-limited top-k selection, exact arithmetic, pure Python.

A checker for the oracle's selection (tiny inputs only).  It follows the
definition by enumeration instead of sorting:
  * a group's score is the largest sum over all gk-subsets of its experts'
    biased affinities (exact rational sums of the fp32 values);
  * among all M-subsets of groups, keep the one with the largest total score,
    ties to the lexicographically smallest sorted tuple of group indices;
  * among all k-subsets of experts inside the kept groups, keep the one with
    the largest total biased affinity, ties to the lexicographically smallest
    sorted index tuple;
  * list the chosen experts by biased affinity descending, index ascending;
  * weights w_j = s_j / sum(s), exact, for comparison within rounding.
With values on a dyadic grid every fp32 sum the oracle forms is exact, so the
two must agree exactly, ties included.
"""
from fractions import Fraction
from itertools import combinations


def _best_subset(items, size, value):
    best, best_key = None, None
    for sub in combinations(items, size):
        tot = sum((value[i] for i in sub), Fraction(0))
        key = (-tot, tuple(sorted(sub)))
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return tuple(sorted(best))


def select_token(s_row, b_row, G, M, k, gk):
    E = len(b_row)
    gsz = E // G
    b = [Fraction(float(v)) for v in b_row]
    s = [Fraction(float(v)) for v in s_row]
    gscore = []
    for g in range(G):
        members = range(g * gsz, (g + 1) * gsz)
        best = max(sum((b[i] for i in sub), Fraction(0)) for sub in combinations(members, gk))
        gscore.append(best)
    groups = _best_subset(range(G), M, gscore)
    eligible = [e for g in groups for e in range(g * gsz, (g + 1) * gsz)]
    chosen = _best_subset(eligible, k, b)
    ordered = sorted(chosen, key=lambda e: (-b[e], e))
    S = sum((s[e] for e in ordered), Fraction(0))
    w = [s[e] / S for e in ordered]
    return ordered, w, groups
