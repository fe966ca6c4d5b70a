"""Pins of the oracle's backward (bf16 experts, routed experts fixed to the
forward's choice).

Pinned against torch autograd in fp64 (library): the test states the layer's
forward with torch ops -- softmax over the chosen logits, SwiGLU experts, the
unweighted shared expert -- and lets autograd derive every gradient (input,
router weights and bias, routed and shared expert weights), which the
oracle's hand-derived backward must reproduce; the same on a token subset;
and exact doubling when the output gradient is doubled.
"""
import numpy as np
import pytest
import torch


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _dec(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double()


def _layer(orc, E=6, H=64, I=32, k=2, Is=16, seed=0, bias=True):
    rng = np.random.default_rng(seed)
    p = dict(
        wr=_bf16(rng.standard_normal((E, H)) / 8),
        bias=(rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None,
        wgu=_bf16(rng.standard_normal((E, 2 * I, H)) * 0.2),
        wd=_bf16(rng.standard_normal((E, H, I)) * 0.2),
        wsgu=_bf16(rng.standard_normal((2 * Is, H)) * 0.2) if Is else None,
        wsd=_bf16(rng.standard_normal((H, Is)) * 0.2) if Is else None,
    )
    L = orc.Layer(H, I, E, k, "bf16", p["wr"], p["wgu"], p["wd"], router_bias=p["bias"],
                  w_shared_gate_up=p["wsgu"], w_shared_down=p["wsd"])
    return L, p


def _autograd(L, p, x, ids, dy, tokens):
    """Gradients of sum_t <y_t, dy_t> over `tokens`, the forward written with torch ops."""
    E, H, I, Is, k = L.E, L.H, L.I, L.Is, L.k
    P = {n: (_dec(v).clone().requires_grad_(True) if v is not None and v.dtype == np.uint16 else
             (torch.from_numpy(v).double().requires_grad_(True) if v is not None else None)) for n, v in p.items()}
    X = _dec(x).clone().requires_grad_(True)
    DY = _dec(dy)
    ids_t = torch.from_numpy(np.asarray(ids, dtype=np.int64))

    def ffn(a, wgu, wd, inter):
        z = a @ wgu.T
        return (torch.nn.functional.silu(z[..., :inter]) * z[..., inter:]) @ wd.T

    loss = 0.0
    for t in tokens:
        logits = X[t] @ P["wr"].T + (P["bias"] if P["bias"] is not None else 0.0)
        g = torch.softmax(logits[ids_t[t]], dim=0)
        y = torch.zeros(H, dtype=torch.float64)
        if Is:
            y = y + ffn(X[t], P["wsgu"], P["wsd"], Is)
        for j in range(k):
            e = int(ids_t[t, j])
            y = y + g[j] * ffn(X[t], P["wgu"][e], P["wd"][e], I)
        loss = loss + (y * DY[t]).sum()
    loss.backward()
    return X.grad.numpy(), {n: (v.grad.numpy() if v is not None else None) for n, v in P.items()}


def _close(a, b, tol=1e-10):
    scale = max(np.abs(b).max(), 1e-300)
    assert np.abs(a - b).max() <= tol * scale, (np.abs(a - b).max(), scale)


@pytest.mark.parametrize("Is,bias", [(16, True), (0, False)])
def test_backward_matches_autograd(orc, Is, bias):
    L, p = _layer(orc, Is=Is, bias=bias)
    rng = np.random.default_rng(1)
    T = 5
    x = _bf16(rng.standard_normal((T, L.H)))
    dy = _bf16(rng.standard_normal((T, L.H)))
    ids, _, _, _ = orc.route(L, x)
    got = orc.backward(L, x, ids, dy)
    dX, dP = _autograd(L, p, x, ids, dy, range(T))
    _close(got["dx"], dX)
    _close(got["dw_gate_up"], dP["wgu"])
    _close(got["dw_down"], dP["wd"])
    _close(got["dw_router"], dP["wr"])
    if bias:
        _close(got["dbias"], dP["bias"])
    if Is:
        _close(got["dw_shared_gate_up"], dP["wsgu"])
        _close(got["dw_shared_down"], dP["wsd"])


def test_backward_token_subset_and_linearity(orc):
    L, p = _layer(orc, seed=3)
    rng = np.random.default_rng(4)
    T = 7
    x = _bf16(rng.standard_normal((T, L.H)))
    dy = _bf16(rng.standard_normal((T, L.H)))
    ids = np.stack([rng.choice(L.E, L.k, replace=False) for _ in range(T)]).astype(np.int32)
    ids.sort(axis=1)
    sub = np.array([1, 4, 6])
    got = orc.backward(L, x, ids, dy, token_list=sub)
    dX, dP = _autograd(L, p, x, ids, dy, sub)
    _close(got["dx"], dX[sub])
    _close(got["dw_gate_up"], dP["wgu"])
    _close(got["dw_down"], dP["wd"])
    _close(got["dw_router"], dP["wr"])
    # doubling dy (exact in bf16) doubles every gradient exactly
    dy2 = _bf16(_dec(dy).numpy() * 2)
    got2 = orc.backward(L, x, ids, dy2, token_list=sub)
    for n in ("dx", "dw_gate_up", "dw_down", "dw_router", "dbias", "dw_shared_gate_up", "dw_shared_down"):
        assert np.array_equal(got2[n], 2 * got[n]), n


def test_bias_gradient_is_sum_of_logit_gradients_that_cancel_per_token(orc):
    """Softmax over the chosen logits: each token's logit gradients sum to zero,
    so the bias gradient summed over experts is zero; with k = 1 every logit
    gradient is zero (the gate is 1)."""
    L, p = _layer(orc, seed=5)
    rng = np.random.default_rng(6)
    x = _bf16(rng.standard_normal((6, L.H)))
    dy = _bf16(rng.standard_normal((6, L.H)))
    ids, _, _, _ = orc.route(L, x)
    got = orc.backward(L, x, ids, dy)
    assert abs(got["dbias"].sum()) <= 1e-12 * np.abs(got["dbias"]).max()
    L1, _ = _layer(orc, k=1, seed=5)
    ids1, _, _, _ = orc.route(L1, x)
    got1 = orc.backward(L1, x, ids1, dy)
    assert np.all(got1["dbias"] == 0) and np.all(got1["dw_router"] == 0)


def test_expert_weight_grads_matches_full_backward(orc):
    """The per-expert weight gradients (numpy products over the expert's
    tokens) agree with the full backward (pinned to autograd above) for every
    expert, including one that receives no token; dx-only mode gives the same
    dx as the full call."""
    L, p = _layer(orc, E=8, k=2, seed=7)
    rng = np.random.default_rng(8)
    T = 9
    x = _bf16(rng.standard_normal((T, L.H)))
    dy = _bf16(rng.standard_normal((T, L.H)))
    ids = np.stack([rng.choice(7, L.k, replace=False) for _ in range(T)]).astype(np.int32)  # expert 7 unused
    ids.sort(axis=1)
    full = orc.backward(L, x, ids, dy)
    for e in range(L.E):
        dgu, dd = orc.expert_weight_grads(L, x, ids, dy, e)
        _close(dgu, full["dw_gate_up"][e]) if np.abs(full["dw_gate_up"][e]).max() > 0 else None
        _close(dd, full["dw_down"][e]) if np.abs(full["dw_down"][e]).max() > 0 else None
        if e == 7:
            assert not dgu.any() and not dd.any()
            assert not full["dw_gate_up"][7].any()
    dx_only = orc.backward(L, x, ids, dy, weights=False)
    assert dx_only["dw_gate_up"] is None and np.array_equal(dx_only["dx"], full["dx"])


def test_vectorised_bf16_decode_matches_codec(orc):
    rng = np.random.default_rng(9)
    b = rng.integers(0, 1 << 16, 4000, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]          # finite values
    assert np.array_equal(orc._bf16_f64(b), orc.bf16_decode(b))
