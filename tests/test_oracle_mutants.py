"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of an oracle module's source with one plausible slip
(an excluded diagonal, a reversed mask, log2 instead of ln, a flipped sign, a
dropped scale, a missing normalization, a wrong GQA head map, an unrescaled
denominator, an averaged merge, a dropped empty identity). The mutant runs in
a private module object; the real oracle is never modified. A battery of pin
checks -- hand-derived cases, closed forms and independent library routines --
must reject every mutant.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.dense
import oracle.online

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "hand_derived_cases.json")))


def _mutant(module, old, new, count=1):
    src = open(module.__file__).read()
    assert src.count(old) >= count, "mutation anchor not found: %r" % old
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__file__ = module.__file__
    exec(compile(src.replace(old, new), module.__file__, "exec"), mod.__dict__)
    return mod


# ---------------------------------------------------------- dense battery
def _dense_checks(d):
    """Yield (name, passed) for each pin applied to dense-oracle module d."""
    def golden():
        for case in GOLDEN["attention"]:
            q, k, v = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
            for mode in ("noncausal", "causal"):
                if mode in case:
                    o, lse = d.attention(q, k, v, case["scale"], causal=(mode == "causal"))
                    if not (np.allclose(o, case[mode]["o"], rtol=1e-12, atol=1e-12)
                            and np.allclose(lse, case[mode]["lse"], rtol=1e-13, atol=1e-12)):
                        return False
        for case in GOLDEN["merge"]:
            m = np.array([float(x) for x in case["m"]])
            o, lse = d.merge_partials(m[None], np.array(case["l"])[None], np.array(case["acc"])[None])
            want = float(case["lse"])
            if np.isnan(o).any() or not np.allclose(o[0], case["o"], atol=1e-13):
                return False
            if (math.isinf(want) and lse[0] != want) or (not math.isinf(want) and abs(lse[0] - want) > 1e-13):
                return False
        return True

    def sdpa():
        rng = np.random.default_rng(1)
        for causal in (False, True):
            q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
            o, lse = d.attention(q, k, v, 0.5, causal)
            qt, kt, vt = (torch.from_numpy(x)[None] for x in (q, k, v))
            o_ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.5)[0].numpy()
            if not np.allclose(o, o_ref, rtol=1e-12, atol=1e-12):
                return False
        return True

    def gqa():
        rng = np.random.default_rng(2)
        t, hq, hkv, dd = 7, 4, 2, 3
        q = rng.standard_normal((t, hq, dd))
        k = rng.standard_normal((t, hkv, dd))
        v = rng.standard_normal((t, hkv, dd))
        o, _ = d.varlen_gqa(q, k, v, np.array([0, t]), 0.5, causal=True)
        qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v))
        o_ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.5,
                                               enable_gqa=True)[0].permute(1, 0, 2).numpy()
        return np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)

    def split():
        rng = np.random.default_rng(3)
        q = rng.standard_normal((2, 4)) * 3
        k = rng.standard_normal((21, 4))
        v = rng.standard_normal((21, 4))
        o, lse = d.merge_partials(*d.split_partials(q, k, v, 0.5, 8))
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        o_ref = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=0.5)[0].numpy()
        lse_ref = torch.logsumexp(0.5 * qt @ kt.T, dim=-1).numpy()
        return np.allclose(o, o_ref, rtol=1e-12, atol=1e-12) and np.allclose(lse, lse_ref, rtol=1e-12)

    def cache():
        # bottom-right causal alignment with grouped KV heads and Nq < Nk,
        # against torch SDPA with an explicit mask j <= i + (Nk - Nq)
        rng = np.random.default_rng(5)
        q = rng.standard_normal((1, 4, 5, 3))
        k = rng.standard_normal((1, 2, 9, 3))
        v = rng.standard_normal((1, 2, 9, 3))
        o, lse = d.attention_cache(q, k, v, 0.5, True)
        mask = torch.arange(9)[None, :] <= (torch.arange(5) + 4)[:, None]
        kt = torch.from_numpy(k).repeat_interleave(2, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(2, dim=1)
        o_ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=mask, scale=0.5).numpy()
        return np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)

    def causal_split():
        # merged causal partials, with rows and chunks that hold no eligible
        # key (Nq > Nk), against the explicit-mask library result
        rng = np.random.default_rng(6)
        q = rng.standard_normal((9, 4))
        k = rng.standard_normal((7, 4))
        v = rng.standard_normal((7, 4))
        o, lse = d.merge_partials(*d.split_partials(q, k, v, 0.5, 3, causal=True))
        if not (np.all(o[:2] == 0.0) and np.all(lse[:2] == -np.inf)) or np.isnan(o).any():
            return False
        mask = torch.arange(7)[None, :] <= (torch.arange(9) - 2)[:, None]
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        o_ref = F.scaled_dot_product_attention(qt[2:], kt, vt, attn_mask=mask[2:], scale=0.5).numpy()
        return np.allclose(o[2:], o_ref, rtol=1e-12, atol=1e-12)

    def sparse():
        # causal window of 3 keys united with 2 global tokens: closed-form
        # pair count and one-key-window closed form, then a block mask that
        # is not symmetric against torch SDPA with the brute-force mask
        n = 20
        m = d.sparse_eligibility(n, n, causal=True, left=2, n_global=2)
        want = sum(i + 1 if i < 2 else min(i + 1, 3) + 2 - max(0, 2 - max(0, i - 2)) for i in range(n))
        if int(m.sum()) != want:
            return False
        # non-causal band of +-1 with 2 global tokens: the global queries see
        # all n keys; any other row sees its band plus the globals outside it
        m = d.sparse_eligibility(n, n, left=1, right=1, n_global=2)
        band = lambda i: set(range(max(0, i - 1), min(n, i + 2)))  # noqa: E731
        want = sum(n if i < 2 else len(band(i) | {0, 1}) for i in range(n))
        if int(m.sum()) != want:
            return False
        rng = np.random.default_rng(7)
        q, k, v = (rng.standard_normal((1, 1, 12, 3)) for _ in range(3))
        o, _ = d.attention_sparse(q, k, v, 0.5, causal=True, left=0)
        if not np.allclose(o[0, 0], v[0, 0], rtol=1e-13, atol=1e-14):
            return False
        bm = np.array([[1, 0, 0], [1, 1, 0], [0, 0, 1]], dtype=np.uint8)   # rows of 4 queries, 4 keys
        o, _ = d.attention_sparse(q, k, v, 0.5, block_mask=bm, block_q=4, block_k=4)
        allowed = torch.tensor([[bool(bm[i // 4][j // 4]) for j in range(12)] for i in range(12)])
        qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
        o_ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed, scale=0.5).numpy()
        return np.allclose(o, o_ref, rtol=1e-12, atol=1e-12)

    for name, fn in (("golden", golden), ("sdpa", sdpa), ("gqa", gqa), ("split", split), ("cache", cache),
                     ("causal_split", causal_split), ("sparse", sparse)):
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        yield name, ok


DENSE_MUTANTS = [
    ("diagonal excluded", "key_idx[None, :] <= q_pos", "key_idx[None, :] < q_pos"),
    ("mask reversed", "key_idx[None, :] <= q_pos", "key_idx[None, :] >= q_pos"),
    ("log2 lse", "lse_blk = m_safe + np.log(", "lse_blk = m_safe + np.log2("),
    ("max shift sign", "p = np.exp(s - m_safe[:, None])", "p = np.exp(s + m_safe[:, None])"),
    ("scale dropped", "s = scale * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)"),
    ("no normalization", "o_blk = num / np.where", "o_blk = num * 0 + num / 1 + 0 * np.where"),
    ("gqa head map h % hkv", "g = h // group", "g = h % hkv", ),
    ("merge weight sign", "np.exp(m - m0[..., None])", "np.exp(m0[..., None] - m)"),
    ("merge denominator unrescaled", "big_l = (w * l).sum(axis=-1)", "big_l = l.sum(axis=-1)"),
    ("merge averages outputs", "o = num / np.where(nonempty, big_l, 1.0)[..., None]",
     "o = (acc / np.where(l > 0, l, 1.0)[..., None]).mean(axis=-2)"),
    ("partial unshifted", "p = np.exp(s - np.where(nonempty, mc, 0.0)[:, None])", "p = np.exp(s)"),
    ("empty partial shifted by -inf", "p = np.exp(s - np.where(nonempty, mc, 0.0)[:, None])",
     "p = np.exp(s - mc[:, None])"),
    ("causal partial excludes position", "<= q_pos[:, None], s, NEG_INF)", "< q_pos[:, None], s, NEG_INF)"),
    ("top-left alignment", "return np.arange(nq, dtype=np.int64) + (nk - nq)", "return np.arange(nq, dtype=np.int64)"),
    ("alignment off by one", "return np.arange(nq, dtype=np.int64) + (nk - nq)",
     "return np.arange(nq, dtype=np.int64) + (nk - nq - 1)"),
    ("global tokens intersected, not united", "ok = win | (j < n_global) | (p < n_global)",
     "ok = win & ((j < n_global) | (p < n_global))"),
    ("globals counted only as keys", "ok = win | (j < n_global) | (p < n_global)", "ok = win | (j < n_global)"),
    ("window left bound off by one", "win &= j >= p - left", "win &= j > p - left"),
    ("block mask transposed", "ok &= bm[np.arange(nq)[:, None] // block_q, j // block_k]",
     "ok &= bm[j // block_k, np.arange(nq)[:, None] // block_q]"),
    ("sparse causal dropped", "    if causal:\n        ok &= j <= p\n", ""),
    ("partial numerator without weights", "acc[:, c, :] = p @ v[j0:j1]", "acc[:, c, :] = v[j0:j1].sum(axis=0)"),
]


def test_real_dense_oracle_passes_battery():
    assert all(ok for _, ok in _dense_checks(oracle.dense))


@pytest.mark.parametrize("name,old,new", DENSE_MUTANTS, ids=[m[0] for m in DENSE_MUTANTS])
def test_dense_mutant_is_caught(name, old, new):
    mod = _mutant(oracle.dense, old, new)
    results = dict(_dense_checks(mod))
    assert not all(results.values()), "mutant '%s' survived every pin: %s" % (name, results)


# --------------------------------------------------------- online battery
def _online_checks(o):
    def closed():
        st = o.merge(o.block([0.0], [[3.0]], 1), o.block([math.log(2.0)], [[6.0]], 1))
        out, lse = o.finalize(st)
        return abs(out[0] - 5.0) < 1e-14 and abs(lse - math.log(3.0)) < 1e-14

    def empties():
        e = o.empty(2)
        ee = o.merge(e, e)
        out, lse = o.finalize(ee)
        return lse == -math.inf and all(x == 0.0 for x in out) and not any(math.isnan(x) for x in ee[2]) \
            and not math.isnan(ee[1])

    def vs_logsumexp():
        rng = np.random.default_rng(4)
        s = (rng.standard_normal(30) * 4).tolist()
        vals = rng.standard_normal((30, 2)).tolist()
        st = o.fold([o.block(s[a:a + 7], vals[a:a + 7], 2) for a in range(0, 30, 7)], 2)
        _, lse = o.finalize(st)
        return abs(lse - float(torch.logsumexp(torch.tensor(s, dtype=torch.float64), 0))) < 1e-12

    def large_logits():
        st = o.merge(o.block([0.0], [[1.0]], 1), o.block([1000.0], [[2.0]], 1))
        out, lse = o.finalize(st)
        return abs(out[0] - 2.0) < 1e-12 and abs(lse - 1000.0) < 1e-12

    for name, fn in (("closed", closed), ("empties", empties), ("logsumexp", vs_logsumexp),
                     ("large", large_logits)):
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        yield name, ok


ONLINE_MUTANTS = [
    ("denominator not rescaled", "l = a[1] * fa + b[1] * fb", "l = a[1] + b[1]"),
    ("numerator not rescaled", "acc = tuple(x * fa + y * fb for", "acc = tuple(x + y for"),
    ("no explicit empty identity", "    if is_empty(a):\n        return b\n    if is_empty(b):\n        return a\n", ""),
    ("log2 lse", "return tuple(x / l for x in acc), m + math.log(l)",
     "return tuple(x / l for x in acc), m + math.log2(l)"),
    ("max kept from first operand", "m = a[0] if a[0] >= b[0] else b[0]", "m = a[0]"),
]


def test_real_online_passes_battery():
    assert all(ok for _, ok in _online_checks(oracle.online))


@pytest.mark.parametrize("name,old,new", ONLINE_MUTANTS, ids=[m[0] for m in ONLINE_MUTANTS])
def test_online_mutant_is_caught(name, old, new):
    mod = _mutant(oracle.online, old, new)
    results = dict(_online_checks(mod))
    assert not all(results.values()), "mutant '%s' survived every pin: %s" % (name, results)


# -------------------------------------------------------- backward battery
def _backward_checks(bmod):
    def autograd():
        rng = np.random.default_rng(9)
        for causal in (False, True):
            q, k, v, do = (rng.standard_normal((7, 3)) for _ in range(4))
            dq, dk, dv = bmod.attention_backward(q * 2, k, v, do, 0.6, causal)
            qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q * 2, k, v))
            o = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=causal, scale=0.6)[0]
            o.backward(torch.from_numpy(do))
            for a, t in ((dq, qt), (dk, kt), (dv, vt)):
                if not np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-11):
                    return False
        return True

    def grouped():
        rng = np.random.default_rng(10)
        q, do = (rng.standard_normal((1, 4, 5, 3)) for _ in range(2))
        k, v = (rng.standard_normal((1, 2, 5, 3)) for _ in range(2))
        _, dk, _ = bmod.attention_backward_bhnd(q, k, v, do, 0.5, True)
        want = np.zeros_like(k)
        for h in range(4):
            want[0, h // 2] += bmod.attention_backward(q[0, h], k[0, h // 2], v[0, h // 2], do[0, h], 0.5, True)[1]
        return np.allclose(dk, want, rtol=1e-13, atol=1e-14)

    def varlen():
        rng = np.random.default_rng(11)
        lengths = [3, 0, 4]
        cu = np.concatenate([[0], np.cumsum(lengths)])
        q, do = (rng.standard_normal((7, 4, 3)) for _ in range(2))
        k, v = (rng.standard_normal((7, 2, 3)) for _ in range(2))
        dq, dk, dv = bmod.attention_backward_varlen(q, k, v, do, cu, 0.7, True)
        seq = np.repeat(np.arange(3), lengths)
        pos = np.arange(7) - cu[seq]
        allowed = (seq[:, None] == seq[None, :]) & (pos[None, :] <= pos[:, None])
        qt, kt, vt = (torch.from_numpy(x.transpose(1, 0, 2).copy()).requires_grad_(True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(qt[None], kt.repeat_interleave(2, 0)[None], vt.repeat_interleave(2, 0)[None],
                                           attn_mask=torch.from_numpy(allowed), scale=0.7)[0]
        o.backward(torch.from_numpy(do.transpose(1, 0, 2).copy()))
        return all(np.allclose(a, t.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-11)
                   for a, t in ((dq, qt), (dk, kt), (dv, vt)))

    def sparse():
        from oracle import dense as dn
        rng = np.random.default_rng(12)
        n = 24
        q, do = (rng.standard_normal((1, 2, n, 3)) for _ in range(2))
        k, v = (rng.standard_normal((1, 1, n, 3)) for _ in range(2))
        bm = np.array([[[1, 0, 1], [1, 1, 0], [0, 1, 1]], [[1, 1, 0], [0, 1, 0], [1, 0, 1]]], dtype=np.uint8)
        dq, dk, dv = bmod.attention_backward_sparse_bhnd(q, k, v, do, 0.6, True, 5, -1, 1, bm, 8, 8)
        mask = torch.from_numpy(np.stack([dn.sparse_eligibility(n, n, True, 5, -1, 1, bm[h], 8, 8) for h in range(2)]))
        qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(qt, kt.repeat_interleave(2, 1), vt.repeat_interleave(2, 1),
                                           attn_mask=mask[None], scale=0.6)
        o.backward(torch.from_numpy(do))
        return all(np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-11) for a, t in ((dq, qt), (dk, kt), (dv, vt)))

    def cache():
        rng = np.random.default_rng(13)
        q, do = (rng.standard_normal((1, 2, 4, 3)) for _ in range(2))
        k, v = (rng.standard_normal((1, 2, 9, 3)) for _ in range(2))
        dq, dk, dv = bmod.attention_backward_cache_bhnd(q, k, v, do, 0.5, True)
        mask = torch.from_numpy(np.arange(9)[None, :] <= (np.arange(4) + 5)[:, None])
        qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
        F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.5).backward(torch.from_numpy(do))
        return all(np.allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-11) for a, t in ((dq, qt), (dk, kt), (dv, vt)))

    for name, fn in (("autograd", autograd), ("grouped", grouped), ("varlen", varlen), ("sparse", sparse),
                     ("cache", cache)):
        try:
            ok = bool(fn())
        except Exception:
            ok = False
        yield name, ok


BACKWARD_MUTANTS = [
    ("softmax row term dropped", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    ("dK without transpose", "dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    ("dQ scale dropped", "dq = scale * (ds @ k)", "dq = (ds @ k)"),
    ("dV without transpose", "dv = p.T @ do", "dv = p @ do"),
    ("causal mask dropped in backward", "    if causal:\n        # query i sits", "    if False:\n        # query i sits"),
    ("cache positions top-left in backward", "pos = np.arange(n) + (k.shape[0] - n)", "pos = np.arange(n)"),
    ("grouped gradients overwritten, not summed", "dk[b, g] += bk", "dk[b, g] = bk"),
    ("varlen KV gradients overwritten, not summed", "dk[a:b, g] += y", "dk[a:b, g] = y"),
    ("varlen KV head taken as h % Hkv", "            g = h // group\n            x, y, z = attention_backward(q[a:b, h]",
     "            g = h % hkv\n            x, y, z = attention_backward(q[a:b, h]"),
    ("sparse eligibility ignored in backward", "        s = np.where(np.asarray(allowed, dtype=bool), s, NEG_INF)",
     "        s = s"),
    ("sparse block mask of head 0 for every head", "            bm = bm[h] if bm.ndim == 3 else bm",
     "            bm = bm[0] if bm.ndim == 3 else bm"),
    ("varlen keys from the whole pack", "attention_backward(q[a:b, h], k[a:b, g], v[a:b, g], do[a:b, h]",
     "attention_backward(q[a:b, h], k[:, g][:b - a], v[:, g][:b - a], do[a:b, h]"),
]


def test_real_backward_oracle_passes_battery():
    import oracle.backward
    assert all(ok for _, ok in _backward_checks(oracle.backward))


@pytest.mark.parametrize("name,old,new", BACKWARD_MUTANTS, ids=[m[0] for m in BACKWARD_MUTANTS])
def test_backward_mutant_is_caught(name, old, new):
    import oracle.backward
    mod = _mutant(oracle.backward, old, new)
    results = dict(_backward_checks(mod))
    assert not all(results.values()), "mutant '%s' survived every pin: %s" % (name, results)
