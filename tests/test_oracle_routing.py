"""Pins of the oracle's routing: biased top-k, unbiased gates, counts and the
stable permutation, against brute force on small inputs and the invariants the
layer must keep (k distinct experts per token, gates >= 0 summing to 1, the
bias changes the selection only, loads sum to T*k)."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as o

F32 = np.float32


def _brute_topk(v, k):
    """Rank counting: expert e is taken iff fewer than k experts beat it under
    (v descending, index ascending); the taken ones are listed in that order."""
    out = []
    for row in v:
        E = len(row)
        beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)  # noqa: E731
        chosen = [e for e in range(E) if sum(beats(f, e) for f in range(E)) < k]
        chosen.sort(key=lambda e: sum(beats(f, e) for f in range(E)))
        out.append(chosen)
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("E,k", [(6, 3), (16, 2), (9, 9), (5, 1)])
def test_topk_bruteforce(E, k):
    rng = np.random.default_rng(E * 100 + k)
    s = rng.uniform(0, 1, (40, E)).astype(F32)
    s[:10] = np.round(s[:10] * 4) / 4          # many exact ties
    b = (rng.standard_normal(E) * 0.1).astype(F32)
    b[: E // 2] = 0
    v = (s + b).astype(F32)
    np.testing.assert_array_equal(o.topk_select(s, b, k), _brute_topk(v, k))


def test_topk_all_pairs_tiny_workload_shape():
    """E=16, k=2 (the tiny workload): the chosen pair is the best of all 120
    pairs under the (v desc, e asc) order of its sorted members."""
    rng = np.random.default_rng(7)
    s = rng.uniform(0, 1, (64, 16)).astype(F32)
    b = (rng.standard_normal(16) * 0.05).astype(F32)
    v = (s + b).astype(F32)
    idx = o.topk_select(s, b, 2)
    for t in range(64):
        key = lambda p: sorted(((-v[t, e], e) for e in p))  # noqa: E731
        best = min(itertools.combinations(range(16), 2), key=key)
        assert sorted(best) == sorted(idx[t].tolist())
        assert key(best)[0][1] == idx[t, 0]


def test_topk_negative_zero_ties_plus_zero():
    s = np.array([[0.25, 0.5, 0.25]], F32)
    b = np.array([-0.25, -0.5, -0.25], F32)    # v = +0, +0, +0 (some as -0 after rounding?)
    v = (s + b).astype(F32)
    assert np.all(v == 0)
    np.testing.assert_array_equal(o.topk_select(s, b, 2), [[0, 1]])


def test_gates_invariants_and_bias_independence():
    rng = np.random.default_rng(4)
    T, E, k = 500, 32, 6
    s = o.sigmoid_r(rng.standard_normal((T, E)).astype(F32))
    b = (rng.standard_normal(E) * 0.3).astype(F32)
    idx_b = o.topk_select(s, b, k)
    idx_0 = o.topk_select(s, np.zeros(E, F32), k)
    assert np.any(idx_b != idx_0)               # the bias reroutes
    for idx in (idx_b, idx_0):
        assert all(len(set(r)) == k for r in idx.tolist())
        g = o.gates_from(s, idx)
        assert np.all(g >= 0)
        assert np.max(np.abs(g.astype(np.float64).sum(1) - 1)) <= k * 2.0 ** -23
        # the gate values are the chosen scores renormalised, whatever chose them
        for t in range(0, T, 37):
            ssum = F32(0)
            for j in range(k):
                ssum = F32(ssum + s[t, idx[t, j]]) if j else s[t, idx[t, 0]]
            for j in range(k):
                assert g[t, j] == F32(s[t, idx[t, j]] / ssum)
    # a bias equal on all experts changes nothing
    idx_c = o.topk_select(s, np.full(E, 0.125, F32), k)
    np.testing.assert_array_equal(idx_c, idx_0)
    np.testing.assert_array_equal(o.gates_from(s, idx_c), o.gates_from(s, idx_0))


def _brute_perm(idx, E):
    T, k = idx.shape
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            counts[idx[t, j]] += 1
    off = [0] * (E + 1)
    for e in range(E):
        off[e + 1] = off[e] + counts[e]
    run = [0] * E
    perm = [None] * (T * k)
    inv = np.zeros((T, k), np.int32)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            row = off[e] + run[e]
            run[e] += 1
            perm[row] = t
            inv[t, j] = row
    return np.array(counts), np.array(off), np.array(perm), inv


@pytest.mark.parametrize("T,E,k", [(37, 5, 2), (64, 16, 2), (10, 3, 3), (1, 8, 4), (0, 4, 2)])
def test_permutation_bruteforce(T, E, k):
    rng = np.random.default_rng(T * 31 + E)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    counts, off, perm, inv = o.permutation(idx, E)
    bc, boff, bperm, binv = _brute_perm(idx, E)
    np.testing.assert_array_equal(counts, bc)
    np.testing.assert_array_equal(off, boff)
    np.testing.assert_array_equal(perm, bperm.reshape(-1) if T else perm)
    np.testing.assert_array_equal(inv, binv)


def test_permutation_invariants_large():
    rng = np.random.default_rng(9)
    T, E, k = 4096, 64, 6
    s = o.sigmoid_r(rng.standard_normal((T, E)).astype(F32))
    idx = o.topk_select(s, np.zeros(E, F32), k)
    counts, off, perm, inv = o.permutation(idx, E)
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    rows = inv.ravel()
    assert np.array_equal(np.sort(rows), np.arange(T * k))           # bijection
    np.testing.assert_array_equal(perm[inv], np.repeat(np.arange(T), k).reshape(T, k))
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                                # stable
        assert np.all(np.any(idx[seg] == e, axis=1))
