"""Pins of the oracle's expert FFN (gate/up, SwiGLU, h storage, down).

Pinned against: dequant-then-matmul vs the factored block-scale form; exact
integer products on grid values with unit scales (numpy int64 matmul); a
dense SwiGLU MLP evaluated with torch fp64 ops (library); exact linearity in
W_d; the e4m3 rounding bound on the stored h; and the parameter count printed
on the Step-5-Preview page (three hidden x intermediate matrices per expert).
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dec(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def _e4m3_dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).double().numpy()


def _fp8_layer(orc, E=2, H=256, I=128, k=1, seed=0, shared=False):
    rng = np.random.default_rng(seed)
    wgu = rng.integers(0, 0x7E, size=(E, 2 * I, H)).astype(np.uint8) | (rng.integers(0, 2, (E, 2 * I, H)) << 7).astype(np.uint8)
    wd = rng.integers(0, 0x7E, size=(E, H, I)).astype(np.uint8) | (rng.integers(0, 2, (E, H, I)) << 7).astype(np.uint8)
    sgu = (rng.random((E, 2 * I // 128, H // 128)) * 1e-4 + 1e-5).astype(np.float32)
    sd = (rng.random((E, H // 128, I // 128)) * 1e-4 + 1e-5).astype(np.float32)
    wr = _bf16(rng.standard_normal((E, H)) / 16)
    kw = {}
    if shared:
        kw = dict(w_shared_gate_up=_bf16(rng.standard_normal((2 * I, H)) * 0.02),
                  w_shared_down=_bf16(rng.standard_normal((H, I)) * 0.02))
    return orc.Layer(H, I, E, k, True, wr, wgu, wd, s_gate_up=sgu, s_down=sd, **kw)


def test_dequant_then_matmul_equals_factored(orc):
    L = _fp8_layer(orc)
    rng = np.random.default_rng(1)
    v = rng.standard_normal(L.H).astype(np.float32)
    q, s = orc.quant_row(v)
    for e in range(L.E):
        zg1, zu1 = orc.expert_gate_up(L, e, q, s, factored=False)
        zg2, zu2 = orc.expert_gate_up(L, e, q, s, factored=True)
        scale = np.abs(np.concatenate([zg1, zu1])).max()
        assert np.max(np.abs(zg1 - zg2)) <= 1e-12 * scale
        assert np.max(np.abs(zu1 - zu2)) <= 1e-12 * scale


def test_grid_values_unit_scales_are_exact(orc):
    # codes of small integers, all scales 1 -> every product and sum is an exact integer
    E, H, I = 1, 256, 128
    rng = np.random.default_rng(2)
    ints = {1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, -1: 0xB8, -2: 0xC0, -3: 0xC4, -4: 0xC8, 0: 0x00}
    keys = np.array(list(ints.keys()))
    wv = rng.choice(keys, size=(E, 2 * I, H))
    av = rng.choice(keys, size=H)
    code = np.vectorize(ints.get)
    wgu = code(wv).astype(np.uint8)
    L = orc.Layer(H, I, E, 1, True, np.zeros((E, H), np.uint16), wgu, np.zeros((E, H, I), np.uint8),
                  s_gate_up=np.ones((E, 2, 2), np.float32), s_down=np.ones((E, 2, 1), np.float32))
    zg, zu = orc.expert_gate_up(L, 0, code(av).astype(np.uint8), np.ones(2, np.float32), factored=False)
    ref = wv[0].astype(np.int64) @ av.astype(np.int64)
    assert np.array_equal(zg, ref[:I].astype(np.float64))
    assert np.array_equal(zu, ref[I:].astype(np.float64))


def test_bf16_dense_swiglu_matches_torch(orc):
    """E = 1, k = 1, gate 1: the layer is a dense SwiGLU MLP plus the shared MLP."""
    rng = np.random.default_rng(3)
    H, I, Is, T = 64, 48, 40, 11
    wgu = _bf16(rng.standard_normal((1, 2 * I, H)) * 0.2)
    wd = _bf16(rng.standard_normal((1, H, I)) * 0.2)
    sgu = _bf16(rng.standard_normal((2 * Is, H)) * 0.2)
    sd = _bf16(rng.standard_normal((H, Is)) * 0.2)
    wr = _bf16(rng.standard_normal((1, H)))
    L = orc.Layer(H, I, 1, 1, False, wr, wgu, wd, w_shared_gate_up=sgu, w_shared_down=sd)
    x = _bf16(rng.standard_normal((T, H)))
    y, ids, gates, _ = orc.forward(L, x)
    assert np.all(ids == 0) and np.all(gates == 1.0)

    def mlp(xx, wgu_, wd_, inter):
        a = torch.from_numpy(xx)
        w = torch.from_numpy(wgu_)
        z = a @ w.T
        h = F.silu(z[:, :inter]) * z[:, inter:]
        h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)   # h stored as bf16
        return (h @ torch.from_numpy(wd_).T).numpy()

    xd = _dec(x)
    ref = mlp(xd, _dec(sgu), _dec(sd), Is) + mlp(xd, _dec(wgu[0]), _dec(wd[0]), I)
    np.testing.assert_allclose(y, ref, rtol=1e-9, atol=1e-12)


def test_routed_part_is_linear_in_w_down(orc):
    rng = np.random.default_rng(4)
    H, I, E, k, T = 64, 32, 6, 2, 9
    wgu = _bf16(rng.standard_normal((E, 2 * I, H)) * 0.2)
    wd = _bf16(rng.standard_normal((E, H, I)) * 0.2)
    wd2 = _bf16(_dec(wd) * 2.0)                       # exact: exponent + 1
    sh = dict(w_shared_gate_up=_bf16(rng.standard_normal((2 * I, H)) * 0.2),
              w_shared_down=_bf16(rng.standard_normal((H, I)) * 0.2))
    wr = _bf16(rng.standard_normal((E, H)) / 8)
    x = _bf16(rng.standard_normal((T, H)))
    # without the shared expert the routed sum doubles bit for bit
    L1 = orc.Layer(H, I, E, k, False, wr, wgu, wd)
    L2 = orc.Layer(H, I, E, k, False, wr, wgu, wd2)
    y1, _, _, _ = orc.forward(L1, x)
    y2, _, _, _ = orc.forward(L2, x)
    assert np.array_equal(y2, 2 * y1)
    # with it, the shared part is untouched and the routed part doubles to rounding
    L1s = orc.Layer(H, I, E, k, False, wr, wgu, wd, **sh)
    L2s = orc.Layer(H, I, E, k, False, wr, wgu, wd2, **sh)
    s = np.stack([orc.shared_row(L1s, x[t]) for t in range(T)])
    np.testing.assert_allclose(orc.forward(L1s, x)[0], s + y1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(orc.forward(L2s, x)[0], s + 2 * y1, rtol=0, atol=1e-14)


def test_fp8_stored_h_within_e4m3_bound(orc):
    L = _fp8_layer(orc, seed=5)
    rng = np.random.default_rng(5)
    q, s = orc.quant_row(rng.standard_normal(L.H).astype(np.float32))
    out, h = orc.expert_row(L, 1, q, s)
    zg, zu = orc.expert_gate_up(L, 1, q, s, factored=False)
    hv = (zg / (1 + np.exp(-zg)) * zu).astype(np.float32).astype(np.float64)
    for g in range(L.I // 128):
        blk = slice(g * 128, (g + 1) * 128)
        sc = np.float32(np.float32(np.abs(hv[blk]).max()) / np.float32(448))
        bound = np.maximum(np.abs(hv[blk]) * 2.0 ** -4, float(sc) * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(np.abs(h[blk] - hv[blk]) <= bound)
        assert np.allclose(np.abs(h[blk]).max(), 448 * float(sc), rtol=1e-12)
    # down projection with library matmul on the dequantised weights
    wd = _e4m3_dec(L.w_down[1]) * np.repeat(np.repeat(L.s_down[1].astype(np.float64), 128, 0), 128, 1)
    np.testing.assert_allclose(out, wd @ h, rtol=1e-12, atol=1e-15)


def test_expert_ffn_rows_equal_expert_row(orc):
    L = _fp8_layer(orc, E=3, seed=6)
    rng = np.random.default_rng(6)
    off = np.array([0, 2, 2, 5], dtype=np.int32)
    v = rng.standard_normal((5, L.H)).astype(np.float32)
    qs = [orc.quant_row(r) for r in v]
    a = np.stack([q for q, _ in qs])
    sc = np.stack([s for _, s in qs])
    out = orc.expert_ffn(L, off, a, sc)
    experts = [0, 0, 2, 2, 2]
    for p in range(5):
        o, _ = orc.expert_row(L, experts[p], a[p], sc[p])
        assert np.array_equal(out[p], o)


def test_step5_parameter_count_implies_three_matrices(orc):
    """The page's total and activated counts fix the size of one routed expert."""
    g = json.load(open(os.path.join(GOLD, "step5_moe_shape.json")))
    H, I = g["hidden"], g["expert_intermediate"]
    per_expert = (g["total_params"] - g["activated_params"]) / (g["moe_layers"] * (g["routed_experts"] - g["top_k"]))
    matrices = per_expert / (H * I)
    assert abs(matrices - 3.0) < 0.01
    # the oracle's layer layout holds exactly three H x I matrices per expert
    L = orc.Layer(H, I, 1, 1, False, np.zeros((1, H), np.uint16),
                  np.zeros((1, 2 * I, H), np.uint16), np.zeros((1, H, I), np.uint16))
    assert (L.w_gate_up[0].size + L.w_down[0].size) == round(matrices) * H * I
