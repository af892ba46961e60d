"""Pins of the standard-library online-merge reference (CPU only).

The (m, l, acc) state must be invariant to how a row is partitioned and to the
order and tree shape of merges, the empty state must be an exact two-sided
identity (including empty + empty, with no NaN), and the result must agree
with the independent dense float64 oracle and with torch's logsumexp.
"""
import math
import random
import subprocess
import sys
import os

import numpy as np
import torch

from oracle import dense, online

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _row(seed, n, d, scale=0.4):
    rng = random.Random(seed)
    q = [rng.gauss(0, 1) for _ in range(d)]
    keys = [[rng.gauss(0, 1) for _ in range(d)] for _ in range(n)]
    vals = [[rng.gauss(0, 1) for _ in range(d)] for _ in range(n)]
    return q, keys, vals, online.row_scores(q, keys, scale)


def _random_partition(rng, n):
    cuts = sorted(rng.sample(range(1, n), rng.randint(0, min(n - 1, 12)))) if n > 1 else []
    bounds = [0] + cuts + [n]
    return list(zip(bounds[:-1], bounds[1:]))


def test_matches_dense_oracle_and_logsumexp():
    n, d = 57, 6
    q, keys, vals, s = _row(1, n, d)
    o, lse = online.finalize(online.block(s, vals, d))
    o_ref, lse_ref = dense.attention(np.array([q]), np.array(keys), np.array(vals), 0.4)
    np.testing.assert_allclose(o, o_ref[0], rtol=1e-12, atol=1e-13)
    assert abs(lse - lse_ref[0]) < 1e-12
    assert abs(lse - float(torch.logsumexp(torch.tensor(s, dtype=torch.float64), 0))) < 1e-12


def test_partition_invariance():
    n, d = 41, 5
    q, keys, vals, s = _row(2, n, d)
    ref = online.finalize(online.block(s, vals, d))
    rng = random.Random(20)
    for _ in range(25):
        parts = _random_partition(rng, n)
        st = online.fold([online.block(s[a:b], vals[a:b], d) for a, b in parts], d)
        o, lse = online.finalize(st)
        np.testing.assert_allclose(o, ref[0], rtol=1e-12, atol=1e-13)
        assert abs(lse - ref[1]) < 1e-12


def test_merge_order_and_tree_invariance():
    n, d = 48, 4
    q, keys, vals, s = _row(3, n, d)
    parts = [online.block(s[a:a + 6], vals[a:a + 6], d) for a in range(0, n, 6)]
    ref = online.finalize(online.fold(parts, d))
    rng = random.Random(30)
    for _ in range(25):
        pool = parts[:]
        rng.shuffle(pool)
        while len(pool) > 1:                    # random merge tree
            i = rng.randrange(len(pool) - 1)
            a, b = pool[i], pool[i + 1]
            merged = online.merge(a, b) if rng.random() < 0.5 else online.merge(b, a)
            pool[i:i + 2] = [merged]
        o, lse = online.finalize(pool[0])
        np.testing.assert_allclose(o, ref[0], rtol=1e-12, atol=1e-13)
        assert abs(lse - ref[1]) < 1e-12


def test_empty_identity_bitwise():
    d = 3
    _, _, vals, s = _row(4, 9, d)
    x = online.block(s, vals, d)
    e = online.empty(d)
    assert online.merge(e, x) == x
    assert online.merge(x, e) == x
    ee = online.merge(e, e)
    assert ee == e
    o, lse = online.finalize(ee)
    assert lse == -math.inf and all(v == 0.0 for v in o)
    assert not any(math.isnan(v) for v in o)
    # a block whose keys are all ineligible is the empty state
    assert online.block([-math.inf, -math.inf], [[1.0] * d, [2.0] * d], d) == e


def test_rescales_numerator_and_denominator():
    """Two single-key blocks with scores 0 and ln 2: merged weights 1/3, 2/3
    (a merge that rescaled only l, or only acc, would not give 5)."""
    a = online.block([0.0], [[3.0]], 1)
    b = online.block([math.log(2.0)], [[6.0]], 1)
    o, lse = online.finalize(online.merge(a, b))
    assert abs(o[0] - 5.0) < 1e-15
    assert abs(lse - math.log(3.0)) < 1e-15


def test_chunked_decode_row_width_131072():
    """A 131072-key row folded from 4096-key chunks (the split-KV decode
    structure) equals the dense oracle."""
    n, d, chunk = 131072, 4, 4096
    rng = np.random.default_rng(5)
    q = rng.standard_normal(d)
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    s = (0.5 * (k @ q)).tolist()           # scores computed once, fed to both
    vals = v.tolist()
    st = online.fold([online.block(s[a:a + chunk], vals[a:a + chunk], d)
                      for a in range(0, n, chunk)], d)
    o, lse = online.finalize(st)
    o_ref, lse_ref = dense.attention(q[None], k, v, 0.5)
    np.testing.assert_allclose(o, o_ref[0], rtol=1e-10, atol=1e-12)
    assert abs(lse - lse_ref[0]) < 1e-10


def test_runs_under_python_dash_S():
    """The reference needs only the standard library (no site packages)."""
    code = ("import sys; sys.path.insert(0, %r); import oracle.online as o; "
            "st = o.merge(o.block([0.0], [[3.0]], 1), o.block([0.6931471805599453], [[6.0]], 1)); "
            "print(o.finalize(st)[0][0])") % ROOT
    out = subprocess.run([sys.executable, "-S", "-c", code], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert abs(float(out.stdout.strip()) - 5.0) < 1e-12
