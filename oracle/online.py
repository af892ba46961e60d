"""Mergeable online-normalizer reference, standard library only.
TEST INFRASTRUCTURE ONLY.

This is the second, independent reference. It imports nothing but ``math``
(it runs under ``python -S``, as the CPU workshop on "Intermediate and advanced
workshop validation", "Correctness and review", does) and shares no code with
``oracle.dense`` or the HIP path.

A state is a tuple (m, l, acc): the running maximum of the scaled scores seen
so far, the exp-sum of those scores rescaled to that maximum, and the matching
rescaled numerator (a tuple of Dv floats). The pages fix the rules this
follows:

* "Intermediate and advanced extension", workshop table, online-normalization
  row: the (maximum, exponential sum) state is mergeable and its result does
  not depend on how the row is partitioned or in which order parts merge.
* "Intermediate and advanced extension", "Logic review before implementation":
  a state that has seen no key starts from a maximum of -inf, which must be
  handled as a special case; when the maximum moves, both the running output
  sum and the running exponential sum are scaled by the same factor.
* "Intermediate and advanced workshop validation", review table: empty + empty
  is handled explicitly, so no NaN can appear.
* "Attention algorithms and data movement", lesson 01: partials are combined
  with their rescaled denominators, not averaged; the empty row has an
  explicit result (the reading taken here: output 0, logsumexp -inf).
"""
import math

NEG_INF = -math.inf


def empty(dv):
    """The empty state: maximum -inf, zero exp-sum, zero numerator."""
    return (NEG_INF, 0.0, tuple(0.0 for _ in range(dv)))


def is_empty(state):
    return state[0] == NEG_INF


def block(scores, values, dv):
    """State of one block of keys.

    scores: list of scaled scores (floats; -inf marks an ineligible key);
    values: list of value rows (each a sequence of dv floats).
    """
    m = NEG_INF
    for s in scores:
        if s > m:
            m = s
    if m == NEG_INF:
        return empty(dv)
    l = 0.0
    acc = [0.0] * dv
    for s, row in zip(scores, values):
        if s == NEG_INF:
            continue
        p = math.exp(s - m)
        l += p
        for d in range(dv):
            acc[d] += p * row[d]
    return (m, l, tuple(acc))


def merge(a, b):
    """Merge two states. The empty state is an explicit two-sided identity."""
    if is_empty(a):
        return b
    if is_empty(b):
        return a
    m = a[0] if a[0] >= b[0] else b[0]
    fa = math.exp(a[0] - m)
    fb = math.exp(b[0] - m)
    l = a[1] * fa + b[1] * fb
    acc = tuple(x * fa + y * fb for x, y in zip(a[2], b[2]))
    return (m, l, acc)


def finalize(state):
    """Normalized output and natural-log logsumexp of a state.

    Empty state -> (zeros, -inf)."""
    m, l, acc = state
    if m == NEG_INF:
        return tuple(0.0 for _ in acc), NEG_INF
    return tuple(x / l for x in acc), m + math.log(l)


def fold(states, dv):
    """Left fold of ``merge`` over a sequence of states, starting from empty."""
    out = empty(dv)
    for st in states:
        out = merge(out, st)
    return out


def row_scores(q_row, keys, scale):
    """Scaled scores scale * <q, k_j> of one query row (plain Python sums)."""
    return [scale * sum(a * b for a, b in zip(q_row, kr)) for kr in keys]
