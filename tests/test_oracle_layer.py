"""Whole-layer pins of the oracle on the small bf16 workload and small fp8 layers.

Pinned against: re-assembly from separately pinned pieces (router, shared and
expert rows), forced-routing and pre-routed-triple entry points agreeing with
the routed forward, token-order equivariance, and the fp8 E = 1 case evaluated
with torch fp64 ops on dequantised weights (library decode of e4m3).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from router_gemm_amd import workloads as W


@pytest.fixture(scope="module")
def small(orc):
    cfg = W.get_config("small_bf16")
    lt = W.make_layer(cfg)
    h = W.host_layer_arrays(lt)
    L = orc.Layer(cfg.H, cfg.I, cfg.E, cfg.k, False, h["w_router"], h["w_gate_up"], h["w_down"],
                  router_bias=h["router_bias"], w_shared_gate_up=h["w_shared_gate_up"],
                  w_shared_down=h["w_shared_down"])
    x = W.bf16_bits(W.make_x(cfg))
    return cfg, L, x


def test_forward_reassembles_from_pieces(orc, small):
    cfg, L, x = small
    y, ids, gates, gap = orc.forward(L, x)
    ids2, g2, gap2, _ = orc.route(L, x)
    assert np.array_equal(ids, ids2) and np.array_equal(gates, g2)
    for t in range(0, cfg.T, 17):
        ref = orc.shared_row(L, x[t])
        for j in range(cfg.k):
            o, _ = orc.expert_row(L, ids[t, j], x[t])
            ref = ref + gates[t, j] * o
        assert np.array_equal(y[t], ref)


def test_forced_ids_and_triples_agree(orc, small):
    cfg, L, x = small
    y, ids, gates, _ = orc.forward(L, x)
    assert np.array_equal(orc.forward_with_ids(L, x, ids), y)
    tok = np.repeat(np.arange(cfg.T), cfg.k).astype(np.int32)
    yt = orc.forward_triples(L, x, tok, ids.ravel(), gates.ravel().astype(np.float32))
    rel = np.abs(yt - y).max(1) / np.abs(y).max(1)
    assert rel.max() < 1e-6          # gates rounded to fp32 in the triple form
    # shuffled triple order changes only the summation order
    perm = np.random.default_rng(0).permutation(tok.size)
    ys = orc.forward_triples(L, x, tok[perm], ids.ravel()[perm], gates.ravel()[perm].astype(np.float32))
    np.testing.assert_allclose(ys, yt, rtol=1e-12, atol=1e-14)


def test_token_order_equivariance(orc, small):
    cfg, L, x = small
    y, _, _, _ = orc.forward(L, x)
    perm = np.random.default_rng(1).permutation(cfg.T)
    yp, _, _, _ = orc.forward(L, x[perm])
    assert np.array_equal(yp, y[perm])
    tl = np.array([5, 77, 5, 0])
    ys, _, _, _ = orc.forward(L, x, token_list=tl)
    assert np.array_equal(ys, y[tl])


def test_fp8_single_expert_matches_torch(orc):
    rng = np.random.default_rng(7)
    H, I, T = 256, 128, 5
    w = torch.from_numpy(rng.standard_normal((2 * I, H)).astype(np.float32) * 0.05)
    wdn = torch.from_numpy(rng.standard_normal((H, I)).astype(np.float32) * 0.05)
    q1, s1 = W.quantize_blocks_e4m3(w)
    q2, s2 = W.quantize_blocks_e4m3(wdn)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    L = orc.Layer(H, I, 1, 1, True, np.zeros((1, H), np.uint16), q1.numpy()[None], q2.numpy()[None],
                  s_gate_up=s1.numpy()[None], s_down=s2.numpy()[None])
    y, _, _, _ = orc.forward(L, bits(x))
    deq = lambda q, s: q.view(torch.float8_e4m3fn).double() * s.double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    Wg, Wd = deq(q1, s1), deq(q2, s2)
    for t in range(T):
        qa, sa = orc.quant_row(x[t].float().numpy())
        a = torch.from_numpy(qa).view(torch.float8_e4m3fn).double() * torch.from_numpy(sa).double().repeat_interleave(128)
        z = Wg @ a
        h = (F.silu(z[:I]) * z[I:]).float()
        qh, sh = orc.quant_row(h.numpy())
        hd = torch.from_numpy(qh).view(torch.float8_e4m3fn).double() * torch.from_numpy(sh).double().repeat_interleave(128)
        ref = (Wd @ hd).numpy()
        np.testing.assert_allclose(y[t], ref, rtol=1e-9, atol=1e-12)
