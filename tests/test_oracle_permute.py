"""Pins of the oracle's grouping (stable counting sort) and combine.

Pinned against: the permutation invariants (counts sum to N, offsets an
exclusive scan ending at N, bijection, stability, each token placed exactly k
times), numpy's stable argsort (library), and combine(permute(x)) == x
when the expert is replaced by the identity and gates are 1.
"""
import numpy as np
import pytest


@pytest.mark.parametrize("N,E", [(0, 5), (1, 1), (37, 4), (4096, 352), (1000, 1)])
def test_permute_invariants_and_library_sort(orc, N, E):
    rng = np.random.default_rng(N + E)
    keys = rng.integers(0, E, size=N).astype(np.int32)
    off, src, pos, dropped = orc.permute(keys, E)
    assert dropped == 0
    counts = np.bincount(keys, minlength=E)
    assert off[0] == 0 and off[E] == N and np.all(np.diff(off) == counts)
    assert np.array_equal(src[pos], np.arange(N))               # bijection
    assert np.array_equal(np.sort(src), np.arange(N))
    assert np.array_equal(src, np.argsort(keys, kind="stable"))  # library stable sort
    for e in range(E):
        seg = src[off[e]:off[e + 1]]
        assert np.all(keys[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_each_token_k_times(orc):
    rng = np.random.default_rng(3)
    T, E, k = 50, 12, 4
    ids = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(T)]).astype(np.int32)
    off, src, pos, _ = orc.permute(ids.ravel(), E)
    tokens = src // k
    assert np.array_equal(np.bincount(tokens, minlength=T), np.full(T, k))
    assert off[E] == T * k


def test_permute_drops_out_of_range(orc):
    keys = np.array([2, -1, 0, 5, 2, 1, 7], dtype=np.int32)
    off, src, pos, dropped = orc.permute(keys, 5)
    assert dropped == 3                          # -1, 5 and 7 are outside [0, 5)
    assert off.tolist() == [0, 1, 2, 4, 4, 4]
    assert pos[1] == -1 and pos[3] == -1 and pos[6] == -1
    assert src.tolist()[:4] == [2, 5, 0, 4]


def _gathered(x, src, k):
    return x[src // k]


def test_combine_of_permute_is_identity(orc):
    rng = np.random.default_rng(4)
    T, E, H = 33, 7, 48
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    # k = 1, gate 1 => y == x exactly
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    off, src, pos, _ = orc.permute(ids.ravel(), E)
    y = orc.combine(_gathered(x, src, 1), pos, np.ones(T, np.float32), T, k=1)
    assert np.array_equal(y, x)
    # k = 4, all gates 1 => y == 4 x exactly
    k = 4
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    off, src, pos, _ = orc.permute(ids.ravel(), E)
    y = orc.combine(_gathered(x, src, k), pos, np.ones(T * k, np.float32), T, k=k)
    assert np.array_equal(y, 4 * x)
    # renormalised gates => y == x to rounding
    g = rng.random((T, k)).astype(np.float32)
    g = (g / g.sum(1, keepdims=True)).astype(np.float32)
    y = orc.combine(_gathered(x, src, k), pos, g.ravel(), T, k=k)
    np.testing.assert_allclose(y, x * g.astype(np.float64).sum(1, keepdims=True), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y, x, rtol=1e-6, atol=1e-6)


def test_combine_with_tokens_and_shared(orc):
    rng = np.random.default_rng(5)
    T, H, N = 6, 8, 9
    tok = np.array([3, 0, 3, 5, 1, 3, 0, 2, 5], dtype=np.int32)
    yp = rng.standard_normal((N, H))
    pos = rng.permutation(N).astype(np.int32)
    g = rng.random(N).astype(np.float32)
    sh = rng.standard_normal((T, H))
    y = orc.combine(yp, pos, g, T, tok=tok, shared=sh)
    for t in range(T):
        ref = sh[t].copy()
        for i in range(N):
            if tok[i] == t:
                ref = ref + float(g[i]) * yp[pos[i]]
        assert np.array_equal(y[t], ref)
    assert np.array_equal(y[4], sh[4])     # token with no assignment: shared only
