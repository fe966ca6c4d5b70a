"""Pins of the oracle's router: logits, top-k selection, gates, gap.

Pinned against: numpy's fp64 matmul of the decoded operands (library), an
all-pairs brute-force check of the selection, injected exact ties, the
closed-form softmax (scipy) for k = E, and the identities k = 1 => g = 1 and
softmax-then-renormalise == softmax over the chosen logits.
"""
import numpy as np
import pytest
import torch
from scipy.special import softmax

from router_gemm_amd import workloads as W


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dec(b):
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).double().numpy()


def _tiny_layer(orc, E, k, H=64, seed=0, bias=None, wr=None):
    rng = np.random.default_rng(seed)
    wr = _bf16(rng.standard_normal((E, H)) / np.sqrt(H)) if wr is None else wr
    I = 8
    wgu = _bf16(rng.standard_normal((E, 2 * I, H)) * 0.1)
    wd = _bf16(rng.standard_normal((E, H, I)) * 0.1)
    return orc.Layer(H, I, E, k, False, wr, wgu, wd, router_bias=bias)


def test_logits_match_library_matmul(orc):
    rng = np.random.default_rng(10)
    L = _tiny_layer(orc, E=20, k=4, H=96, bias=rng.standard_normal(20).astype(np.float32))
    x = _bf16(rng.standard_normal((7, 96)))
    ids, gates, gap, logits = orc.route(L, x, want_logits=True)
    ref = _dec(x) @ _dec(L.w_router).T + L.router_bias.astype(np.float64)
    np.testing.assert_allclose(logits, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("E,k", [(12, 3), (32, 4), (9, 1), (16, 8)])
def test_topk_brute_force(orc, E, k):
    rng = np.random.default_rng(E * 100 + k)
    L = _tiny_layer(orc, E=E, k=k, seed=E + k)
    x = _bf16(rng.standard_normal((40, 64)))
    ids, gates, gap, logits = orc.route(L, x, want_logits=True)
    for t in range(40):
        chosen = set(ids[t].tolist())
        assert len(chosen) == k and list(ids[t]) == sorted(ids[t])       # ascending slots
        for c in chosen:
            for u in set(range(E)) - chosen:
                lc, lu = logits[t, c], logits[t, u]
                assert lc > lu or (lc == lu and c < u)
        srt = np.sort(logits[t])[::-1]
        expect_gap = srt[k - 1] - srt[k] if k < E else np.inf
        assert gap[t] == expect_gap


def test_exact_ties_pick_lowest_index(orc):
    # x = e_0 so that every logit equals W_r[e, 0] exactly (bf16 values, exact sums).
    E, k, H = 10, 3, 64
    col = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.5, 3.0, 2.0, -1.0])
    wr = np.zeros((E, H), dtype=np.float32)
    wr[:, 0] = col
    x = np.zeros((1, H), dtype=np.float32)
    x[0, 0] = 1.0
    L = _tiny_layer(orc, E, k, H=H, wr=_bf16(wr))
    ids, _, gap, _ = orc.route(L, _bf16(x))
    assert ids[0].tolist() == [1, 3, 7]        # the three 3.0s
    L2 = _tiny_layer(orc, E, 5, H=H, wr=_bf16(wr))
    ids2, _, gap2, _ = orc.route(L2, _bf16(x))
    assert ids2[0].tolist() == [1, 2, 3, 4, 7]  # 2.0 tie at indices 2,4,5,8 -> 2 and 4
    assert gap2[0] == 0.0


def test_gates_closed_forms(orc):
    rng = np.random.default_rng(11)
    E, k = 24, 6
    L = _tiny_layer(orc, E=E, k=k)
    x = _bf16(rng.standard_normal((30, 64)) * 3)
    ids, gates, _, logits = orc.route(L, x, want_logits=True)
    np.testing.assert_allclose(gates.sum(1), 1.0, rtol=0, atol=1e-15)
    full = softmax(logits, axis=1)
    renorm = np.take_along_axis(full, ids.astype(np.int64), 1)
    renorm /= renorm.sum(1, keepdims=True)
    np.testing.assert_allclose(gates, renorm, rtol=1e-13, atol=1e-16)
    # k = 1: the single gate is exactly 1
    L1 = _tiny_layer(orc, E=E, k=1)
    _, g1, _, _ = orc.route(L1, x)
    assert np.all(g1 == 1.0)
    # k = E: every expert is chosen, gates are the textbook softmax, gap = +inf
    LE = _tiny_layer(orc, E=E, k=E)
    idsE, gE, gapE, lE = orc.route(LE, x, want_logits=True)
    assert np.all(idsE == np.arange(E))
    np.testing.assert_allclose(gE, softmax(lE, axis=1), rtol=1e-13, atol=1e-17)
    assert np.all(np.isinf(gapE))


def test_bias_forces_selection(orc):
    rng = np.random.default_rng(12)
    E, k = 16, 2
    bias = np.zeros(E, dtype=np.float32)
    bias[13] = 1e4
    L = _tiny_layer(orc, E=E, k=k, bias=bias)
    ids, gates, _, _ = orc.route(L, _bf16(rng.standard_normal((20, 64))))
    for t in range(20):
        j = list(ids[t]).index(13)
        assert gates[t, j] == 1.0 and gates[t, 1 - j] == 0.0


def test_gates_for_ids_consistent(orc):
    rng = np.random.default_rng(13)
    L = _tiny_layer(orc, E=20, k=4)
    x = _bf16(rng.standard_normal((9, 64)))
    ids, gates, _, _ = orc.route(L, x)
    np.testing.assert_array_equal(orc.gates_for_ids(L, x, ids), gates)
    tl = np.array([8, 2, 2])
    ids2, g2, _, _ = orc.route(L, x, token_list=tl)
    np.testing.assert_array_equal(ids2, ids[tl])
    np.testing.assert_array_equal(g2, gates[tl])


def test_prefill_zipf_bias_skews_loads(orc):
    """The prefill workload's router bias gives the hottest expert ~10x the mean load."""
    cfg = W.get_config("prefill_fp8")
    lt_r = W._bf16_bits(W._rng(cfg.seed, 2).standard_normal((cfg.E, cfg.H), dtype=np.float32)
                        * np.float32(cfg.router_std))
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    x = W.make_x(cfg)
    L = orc.Layer(cfg.H, 128, cfg.E, cfg.k, False, bits(lt_r),
                  np.zeros((cfg.E, 2, 1), np.uint16), np.zeros((cfg.E, 1, 1), np.uint16),
                  router_bias=W.zipf_bias(cfg))
    tl = np.arange(0, cfg.T, 4)                      # every 4th token keeps this test short
    ids, _, gap, _ = orc.route(L, bits(x), token_list=tl)
    cnt = np.bincount(ids.ravel(), minlength=cfg.E)
    ratio = cnt.max() / cnt.mean()
    assert 8.5 < ratio < 11.5, ratio
    assert (cnt > 0).sum() == cfg.E


def test_nan_logits_rank_below_every_number(orc):
    """A NaN logit ranks as -infinity: experts whose bias is NaN are chosen only
    when fewer than k others are left, lowest index first; a token whose
    logits are all NaN (a NaN in x) gets experts 0..k-1 with gates 1/k (the k
    chosen values are equal, so the softmax over them is uniform); a +inf
    logit takes gate 1.  The oracle's logits output keeps the NaN values."""
    rng = np.random.default_rng(31)
    E, k, H = 12, 4, 64
    bias = np.zeros(E, dtype=np.float32)
    bias[[0, 3, 7]] = np.nan
    L = _tiny_layer(orc, E=E, k=k, H=H, bias=bias)
    x = _bf16(rng.standard_normal((6, H)))
    x[5, 9] = 0x7FC0                                  # bf16 NaN: every logit of token 5 is NaN
    ids, gates, gap, logits = orc.route(L, x, want_logits=True)
    assert np.isnan(logits[:, [0, 3, 7]]).all() and np.isnan(logits[5]).all()
    finite = np.setdiff1d(np.arange(E), [0, 3, 7])
    for t in range(5):
        lt = logits[t, finite]
        want = np.sort(finite[np.argsort(-lt, kind="stable")[:k]])
        np.testing.assert_array_equal(ids[t], want)
        np.testing.assert_allclose(gates[t], softmax(logits[t, want]), rtol=1e-13)
    np.testing.assert_array_equal(ids[5], np.arange(k))
    np.testing.assert_array_equal(gates[5], np.full(k, 1.0 / k))
    assert gap[5] == 0.0                               # the k-th and (k+1)-th values are equal (-inf)
    # only 2 numbers left for k = 4: the two finite logits, then the two lowest NaN experts
    bias2 = np.full(E, np.nan, dtype=np.float32)
    bias2[[5, 10]] = 0.0
    L2 = _tiny_layer(orc, E=E, k=k, H=H, bias=bias2)
    ids2, gates2, _, lg2 = orc.route(L2, x[:5], want_logits=True)
    np.testing.assert_array_equal(ids2, np.tile([0, 1, 5, 10], (5, 1)))
    for t in range(5):   # the NaN experts weigh exp(-inf) = 0
        np.testing.assert_allclose(gates2[t], [0, 0, *softmax(lg2[t, [5, 10]])], rtol=1e-13)
    # a +inf logit: chosen, gate 1
    bias3 = np.zeros(E, dtype=np.float32)
    bias3[6] = np.inf
    L3 = _tiny_layer(orc, E=E, k=k, H=H, bias=bias3)
    ids3, gates3, _, _ = orc.route(L3, x[:5], want_logits=True)
    for t in range(5):
        assert 6 in ids3[t]
        np.testing.assert_array_equal(gates3[t], (ids3[t] == 6).astype(np.float64))
