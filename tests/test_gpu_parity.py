"""GPU parity: every primitive and the fused forward through the C ABI against
the fp64 oracle on the same seeded inputs.

Bars: expert ids, offsets and permutation indices and the fp8 x_perm bytes and
scales bit-exact (ids up to the near-tie exemption); gates within 2e-6;
outputs within the per-token max relative error 2e-2 (bf16) / 4e-2 (fp8).
"""
import numpy as np
import pytest
import torch

import oracle
from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import REG, TOL, check_forward, check_ids, dev, oracle_layer, rel_err_rows, run_forward, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name", ["small_bf16", "small_fp8"])
def test_route_matches_oracle(name):
    cfg = W.get_config(name)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev())
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev())
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev())
    B.moe_route(layer, x, cfg.T, ids, gates, logits, ws=B.workspace(layer, cfg.T, cfg.N, dev()))
    torch.cuda.synchronize()
    OL = oracle_layer(lt)
    ids_ref, g_ref, gap, l_ref = oracle.route(OL, W.bf16_bits(x), want_logits=True)
    same = check_ids(ids.cpu().numpy(), ids_ref, gap)
    np.testing.assert_allclose(logits.cpu().numpy(), l_ref, rtol=0, atol=2e-5)
    assert np.abs(gates.cpu().numpy()[same] - g_ref[same]).max() < 2e-6


def test_route_many_tokens_tiled_path():
    """T >= 2048 takes the LDS-tiled logits kernel: ragged T (not a multiple of
    the 128-token tile) and E = 352 (not a multiple of the 192-expert tile),
    one K split at this hidden size; every token's ids, gates and logits
    against the oracle."""
    cfg = W.get_config("small_bf16", T=2085, E=352, k=8, I=64, Is=0)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev())
    gates = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev())
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev())
    B.moe_route(layer, x, cfg.T, ids, gates, logits, ws=B.workspace(layer, cfg.T, cfg.N, dev()))
    torch.cuda.synchronize()
    OL = oracle_layer(lt)
    ids_ref, g_ref, gap, l_ref = oracle.route(OL, W.bf16_bits(x), want_logits=True)
    same = check_ids(ids.cpu().numpy(), ids_ref, gap)
    np.testing.assert_allclose(logits.cpu().numpy(), l_ref, rtol=0, atol=2e-5)
    assert np.abs(gates.cpu().numpy()[same] - g_ref[same]).max() < 2e-6


@pytest.mark.parametrize("T,H,E,k", [
    (50, 640, 100, 6),      # 2-way K split, 320-wide chunks: a batch of 8 K-steps, then one of 2
    (33, 384, 77, 3),       # no split, a 384-wide chunk: 8 K-steps, then 4
    (16, 4096, 1000, 32),   # 16 experts per lane, k = 32, a 16-way split (four batches of split loads)
    (70, 4096, 1024, 8),    # the largest expert count, an 8-way split
])
def test_route_split_chunk_tails_and_wide_experts(T, H, E, k):
    """The split-K logits kernel on chunks that are not a multiple of its
    8-step batches, and the top-k kernel with 16 experts per lane: ids, gates
    and logits of every token against the oracle."""
    g = torch.Generator(device="cpu").manual_seed(7)
    wr = (torch.randn(E, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    I = 64   # the expert weights are never read by the router
    layer = B.Layer(H, I, E, k, B.MOE_BF16, torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=dev()),
                    torch.zeros((E, H, I), dtype=torch.bfloat16, device=dev()), w_router=wr.to(dev()))
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    gates = torch.empty((T, k), dtype=torch.float32, device=dev())
    logits = torch.empty((T, E), dtype=torch.float32, device=dev())
    B.moe_route(layer, x.to(dev()), T, ids, gates, logits, ws=B.workspace(layer, T, T * k, dev()))
    torch.cuda.synchronize()
    OL = oracle.Layer(H, I, E, k, "bf16", W.bf16_bits(wr), np.zeros((E, 2 * I, H), np.uint16),
                      np.zeros((E, H, I), np.uint16))
    ids_ref, g_ref, gap, l_ref = oracle.route(OL, W.bf16_bits(x), want_logits=True)
    same = check_ids(ids.cpu().numpy(), ids_ref, gap)
    np.testing.assert_allclose(logits.cpu().numpy(), l_ref, rtol=0, atol=2e-5)
    assert np.abs(gates.cpu().numpy()[same] - g_ref[same]).max() < 2e-6
    # slots in ascending expert id, no repeats
    ids_np = ids.cpu().numpy()
    assert (np.diff(ids_np, axis=1) > 0).all()


def _route_with(wr, x, k, bias=None):
    E, H = wr.shape
    I = 64
    wgu = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=dev())
    wd = torch.zeros((E, H, I), dtype=torch.bfloat16, device=dev())
    layer = B.Layer(H, I, E, k, B.MOE_BF16, wgu, wd, w_router=wr, router_bias=bias)
    T = x.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    gates = torch.empty((T, k), dtype=torch.float32, device=dev())
    B.moe_route(layer, x, T, ids, gates, ws=B.workspace(layer, T, T * k, dev()))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy()


@pytest.mark.parametrize("T,H,E", [(4096, 4096, 352), (2500, 8192, 200)])
def test_route_tiled_split_k(T, H, E):
    """Many tokens at a long hidden size: the LDS-tiled logits kernel with its
    K split into partials (4 and 8 ways here; ragged T and E), summed in order
    by the top-k kernel: ids, gates and logits of every token."""
    k = 8
    g = torch.Generator(device="cpu").manual_seed(8)
    wr = (torch.randn(E, H, generator=g) / H ** 0.5).to(torch.bfloat16)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    I = 64   # the expert weights are never read by the router
    layer = B.Layer(H, I, E, k, B.MOE_BF16, torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=dev()),
                    torch.zeros((E, H, I), dtype=torch.bfloat16, device=dev()), w_router=wr.to(dev()))
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    gates = torch.empty((T, k), dtype=torch.float32, device=dev())
    logits = torch.empty((T, E), dtype=torch.float32, device=dev())
    B.moe_route(layer, x.to(dev()), T, ids, gates, logits, ws=B.workspace(layer, T, T * k, dev()))
    torch.cuda.synchronize()
    OL = oracle.Layer(H, I, E, k, "bf16", W.bf16_bits(wr), np.zeros((E, 2 * I, H), np.uint16),
                      np.zeros((E, H, I), np.uint16))
    ids_ref, g_ref, gap, l_ref = oracle.route(OL, W.bf16_bits(x), want_logits=True)
    same = check_ids(ids.cpu().numpy(), ids_ref, gap)
    np.testing.assert_allclose(logits.cpu().numpy(), l_ref, rtol=0, atol=2e-5)
    assert np.abs(gates.cpu().numpy()[same] - g_ref[same]).max() < 2e-6


def test_route_exact_ties_lowest_index():
    # duplicated router rows give bit-identical logits in any arithmetic
    E, H, T, k = 40, 256, 70, 4
    g = torch.Generator(device="cpu").manual_seed(5)
    wr = (torch.randn(E, H, generator=g) / 16).to(torch.bfloat16)
    for a, b in [(3, 17), (5, 6), (20, 39), (0, 1)]:
        wr[b] = wr[a]
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    ids, gates = _route_with(wr.to(dev()), x.to(dev()), k)
    for t in range(T):
        s = set(ids[t].tolist())
        for a, b in [(3, 17), (5, 6), (20, 39), (0, 1)]:
            assert not (b in s and a not in s), (t, a, b, ids[t])
        if 3 in s and 17 in s:
            j3, j17 = list(ids[t]).index(3), list(ids[t]).index(17)
            assert gates[t, j3] == gates[t, j17]
    # all-equal logits: x = 0 -> every logit 0 -> experts 0..k-1, gates 1/k
    ids0, g0 = _route_with(wr.to(dev()), torch.zeros((3, H), dtype=torch.bfloat16, device=dev()), k)
    assert (ids0 == np.arange(k)).all() and np.allclose(g0, 1.0 / k, atol=1e-7)


@pytest.mark.parametrize("T", [40, 2100])     # split-K logits kernel; LDS-tiled logits kernel
def test_route_nan_logits_rank_lowest(T):
    """NaN logits rank as -infinity, as in the oracle: experts with a NaN bias
    are never chosen while k others are left; a token with a NaN in x (every
    logit NaN) gets experts 0..k-1 with gates 1/k; the same with only two
    finite logits (the two, then the lowest NaN experts, gate 0); the logits
    output keeps the NaN values."""
    E, H, k = 40, 256, 4
    g = torch.Generator(device="cpu").manual_seed(6)
    wr = (torch.randn(E, H, generator=g) / 16).to(torch.bfloat16)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    x[3, 17] = float("nan")
    for nan_experts in ([1, 8, 33], [e for e in range(E) if e not in (12, 30)]):
        bias = np.zeros(E, dtype=np.float32)
        bias[nan_experts] = np.nan
        ids, gates = _route_with(wr.to(dev()), x.to(dev()), k, bias=torch.from_numpy(bias).to(dev()))
        OL = oracle.Layer(H, 64, E, k, "bf16", W.bf16_bits(wr), np.zeros((E, 128, H), np.uint16),
                          np.zeros((E, H, 64), np.uint16), router_bias=bias)
        ids_ref, g_ref, gap, l_ref = oracle.route(OL, W.bf16_bits(x), want_logits=True)
        same = check_ids(ids, ids_ref, gap)
        assert np.abs(gates[same] - g_ref[same]).max() < 2e-6
        np.testing.assert_array_equal(ids[3], np.arange(k))
        np.testing.assert_array_equal(gates[3], np.full(k, 0.25, dtype=np.float32))
        assert not np.isin(ids[np.arange(T) != 3], nan_experts).any() if len(nan_experts) < E - k else True


def test_route_k_equals_E_and_k1():
    cfg = W.get_config("small_bf16", k=32, T=37)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    OL = oracle_layer(lt)
    ids, gates = _route_with(lt.w_router, x, 32)
    assert (ids == np.arange(32)).all()
    _, g_ref, _, _ = oracle.route(OL, W.bf16_bits(x))
    assert np.abs(gates - g_ref).max() < 2e-6
    ids1, g1 = _route_with(lt.w_router, x, 1)
    OL1 = oracle_layer(W.make_layer(W.get_config("small_bf16", k=1), "cpu"))
    ids1_ref, _, gap1, _ = oracle.route(OL1, W.bf16_bits(x))
    check_ids(ids1, ids1_ref, gap1)
    assert (g1 == 1.0).all()


# ------------------------------------------------------------------ permute

def _permute(cfg_name, N, T, k, E, with_tokens, invalid, fp8, seed=0):
    rng = np.random.default_rng(seed)
    H = 512
    keys = rng.integers(0, E, size=N).astype(np.int32)
    tok = rng.integers(0, T, size=N).astype(np.int32) if with_tokens else None
    if invalid:
        keys[rng.choice(N, size=max(1, N // 50), replace=False)] = rng.choice([-1, E, E + 7])
        if with_tokens:
            tok[rng.choice(N, size=max(1, N // 60), replace=False)] = T + 3
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32) * 3).to(torch.bfloat16)
    lt_dtype = B.MOE_FP8_E4M3FN if fp8 else B.MOE_BF16
    layer = B.Layer(H, 128, E, k if not with_tokens else 0, lt_dtype, None, None)
    d = dev()
    xg = x.to(d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    src = torch.full((N,), -7, dtype=torch.int32, device=d)
    pos = torch.empty(N, dtype=torch.int32, device=d)
    xp = torch.zeros((N, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=d)
    xs = torch.zeros((N, H // 128), dtype=torch.float32, device=d) if fp8 else None
    kg = torch.from_numpy(keys).to(d)
    tg = torch.from_numpy(tok).to(d) if with_tokens else None
    B.moe_permute(layer, xg, T, kg, tg, N, off, src, pos, xp, xs, ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    okeys = keys.copy()
    if with_tokens:
        okeys[(tok < 0) | (tok >= T)] = -1
    off_r, src_r, pos_r, dropped = oracle.permute(okeys, E)
    assert np.array_equal(off.cpu().numpy(), off_r)
    nv = off_r[E]
    assert np.array_equal(src.cpu().numpy()[:nv], src_r[:nv])
    assert np.array_equal(pos.cpu().numpy(), pos_r)
    # gathered rows
    toks = (tok[src_r[:nv]] if with_tokens else src_r[:nv] // k)
    xb = W.bf16_bits(x)
    if fp8:
        q_r, s_r = oracle.quant_bf16_rows(xb[toks])
        assert np.array_equal(xp.cpu().numpy()[:nv], q_r)
        assert np.array_equal(xs.cpu().numpy()[:nv], s_r)
    else:
        assert np.array_equal(W.bf16_bits(xp)[:nv], xb[toks])
    return dropped


@pytest.mark.parametrize("N,T,k,E,tokens,invalid,fp8", [
    (1000, 250, 4, 32, False, False, False),
    (1000, 250, 4, 32, False, False, True),
    (513, 400, 0, 44, True, True, True),        # ragged, pre-routed, dropped entries
    (512, 300, 0, 44, True, True, True),        # one chunk exactly (one-workgroup sort), dropped entries
    (65536, 8192, 8, 352, False, False, True),  # prefill size
    (1, 1, 1, 5, False, False, True),
    (7, 9, 0, 1000, True, False, False),
])
def test_permute_bit_exact(N, T, k, E, tokens, invalid, fp8):
    if not tokens:
        N = T * k
    _permute("p", N, T, k, E, tokens, invalid, fp8)


def test_permute_empty():
    d = dev()
    layer = B.Layer(512, 128, 8, 2, B.MOE_BF16, None, None)
    off = torch.full((9,), 5, dtype=torch.int32, device=d)
    z = torch.empty(0, dtype=torch.int32, device=d)
    B.moe_permute(layer, torch.empty((0, 512), dtype=torch.bfloat16, device=d), 0, z, None, 0, off, z, z,
                  torch.empty((0, 512), dtype=torch.bfloat16, device=d), ws=B.workspace(layer, 1, 1, d))
    torch.cuda.synchronize()
    assert (off.cpu().numpy() == 0).all()


# ------------------------------------------------------------------ expert FFN

def _grouped_rows(E, N, H, fp8, rng, empty_frac=0.3):
    counts = rng.multinomial(N, rng.dirichlet(np.ones(E) * 0.5))
    counts[rng.random(E) < empty_frac] = 0
    counts[0] += N - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    if fp8:
        codes = rng.integers(0, 0x7E, size=(N, H)).astype(np.uint8) | (rng.integers(0, 2, (N, H)) << 7).astype(np.uint8)
        scales = (rng.random((N, H // 128)) * 0.01 + 1e-3).astype(np.float32)
        return off, codes, scales
    xb = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(torch.bfloat16)
    return off, W.bf16_bits(xb), None


@pytest.mark.parametrize("fp8,E,N,H,I,ydt", [
    (False, 32, 300, 512, 192, torch.float32),
    (False, 5, 1000, 512, 128, torch.bfloat16),
    (True, 16, 777, 512, 256, torch.float32),
    (True, 3, 2000, 1024, 384, torch.bfloat16),
    # many rows per expert but H % 256 != 0: the streaming kernels (64-row token tiles)
    (True, 3, 600, 384, 256, torch.float32),
    # the dense FF layers' width (intermediate 13824) as one expert holding every row
    (False, 1, 300, 512, 13824, torch.float32),
    (True, 1, 300, 512, 13824, torch.bfloat16),
])
def test_expert_ffn_matches_oracle(fp8, E, N, H, I, ydt):
    rng = np.random.default_rng(E * N)
    cfg = W.MoEConfig("t", T=N, H=H, E=E, k=1, I=I, Is=0, expert_dtype="fp8" if fp8 else "bf16",
                      router_std=0.05, seed=3)
    lt = W.make_layer(cfg, dev())
    off, a, s = _grouped_rows(E, N, H, fp8, rng)
    d = dev()
    layer = B.Layer.from_tensors(lt)
    a_t = torch.from_numpy(a).to(d) if fp8 else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(d)
    s_t = torch.from_numpy(s).to(d) if fp8 else None
    y = torch.full((N, H), float("nan"), dtype=ydt, device=d)
    B.moe_expert_ffn(layer, torch.from_numpy(off).to(d), a_t, s_t, N, y, ws=B.workspace(layer, N, N, d))
    torch.cuda.synchronize()
    y_ref = oracle.expert_ffn(oracle_layer(lt), off, a, s)
    err = rel_err_rows(to_np(y), y_ref)
    _print(f"expert_ffn fp8={fp8} E={E} N={N}: max rel err {err.max():.3e}")
    assert err.max() < TOL["fp8" if fp8 else "bf16"]


def test_shared_expert_view_matches_oracle():
    cfg = W.get_config("small_bf16")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.shared_view(lt)
    off = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev())
    y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev())
    B.moe_expert_ffn(layer, off, x, None, cfg.T, y, ws=B.workspace(layer, cfg.T, cfg.T, dev()))
    torch.cuda.synchronize()
    OL = oracle_layer(lt)
    xb = W.bf16_bits(x)
    y_ref = np.stack([oracle.shared_row(OL, xb[t]) for t in range(cfg.T)])
    assert rel_err_rows(to_np(y), y_ref).max() < TOL["bf16"]


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("tokens,ydt,sdt,odt", [
    (False, torch.float32, torch.float32, torch.float32),
    (False, torch.bfloat16, torch.bfloat16, torch.bfloat16),
    (True, torch.bfloat16, torch.float32, torch.float32),
    (True, torch.float32, None, torch.bfloat16),
])
def test_combine_matches_oracle(tokens, ydt, sdt, odt):
    rng = np.random.default_rng(11)
    T, H, k = 300, 512, 4
    N = 777 if tokens else T * k
    d = dev()
    yp = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(ydt)
    pos = rng.permutation(N).astype(np.int32)
    pos[rng.choice(N, 5, replace=False)] = -1
    tok = rng.integers(0, T, size=N).astype(np.int32) if tokens else None
    if tokens:
        tok[:3] = [T + 5, -2, T]           # out of range: skipped
    gates = rng.random(N).astype(np.float32)
    sh = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(sdt) if sdt else None
    layer = B.Layer(H, 128, 8, 0 if tokens else k, B.MOE_BF16, None, None)
    y = torch.empty((T, H), dtype=odt, device=d)
    B.moe_combine(layer, yp.to(d), B.dtype_code(yp), torch.from_numpy(pos).to(d),
                  torch.from_numpy(tok).to(d) if tokens else None, torch.from_numpy(gates).to(d), N,
                  sh.to(d) if sh is not None else None, B.dtype_code(sh) if sh is not None else 0, T, y,
                  B.dtype_code(y), ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    y_ref = oracle.combine(to_np(yp), pos, gates, T, k=k, tok=tok, shared=None if sh is None else to_np(sh))
    err = rel_err_rows(to_np(y), y_ref)       # rows with nothing to add are exactly zero
    assert err.max() < (1e-6 if odt == torch.float32 else 2 ** -8)


@pytest.mark.parametrize("k,ydt,odt", [(1, torch.float32, torch.float32), (3, torch.bfloat16, torch.bfloat16),
                                       (8, torch.bfloat16, torch.float32), (8, torch.float32, torch.bfloat16)])
def test_combine_router_layout_edges(k, ydt, odt):
    """The router's layout (slot u of token t at t*k + u) at k = 1, 3 and 8:
    a second 2048-column block only partly covered (H = 2176), skipped slots
    (perm_pos -1 and positions at or past the N rows), a shared expert, every
    combination of fp32 / bf16 rows and outputs."""
    rng = np.random.default_rng(17 + k)
    T, H = 37, 2176
    N = T * k
    d = dev()
    yp = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32)).to(ydt)
    pos = rng.permutation(N).astype(np.int32)
    skip = rng.choice(N, min(6, N), replace=False)
    pos[skip[:3]] = -1
    pos[skip[3:]] = N + np.arange(len(skip) - 3, dtype=np.int32)   # past the last row
    gates = rng.random(N).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    layer = B.Layer(H, 128, 8, k, B.MOE_BF16, None, None)
    y = torch.empty((T, H), dtype=odt, device=d)
    B.moe_combine(layer, yp.to(d), B.dtype_code(yp), torch.from_numpy(pos).to(d), None,
                  torch.from_numpy(gates).to(d), N, torch.from_numpy(sh).to(d), B.MOE_F32, T, y,
                  B.dtype_code(y), ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    pos_ref = np.where(pos >= N, -1, pos).astype(np.int32)
    y_ref = oracle.combine(to_np(yp), pos_ref, gates, T, k=k, tok=None, shared=sh)
    err = rel_err_rows(to_np(y), y_ref)
    assert err.max() < (1e-6 if odt == torch.float32 else 2 ** -8)


@pytest.mark.parametrize("tokens", [True, False])
def test_combine_long_assignment_lists_and_partial_column_block(tokens):
    """Tokens with 70, 33, 32, 9 and 0 assignments (several 32-slot batches,
    8-row load groups cut short), k = 32 slots per token, and H = 2176: a
    second 2048-column block only partly covered."""
    rng = np.random.default_rng(13)
    H = 2176
    d = dev()
    if tokens:
        T, k = 5, 0
        counts = [70, 33, 32, 9, 0]
        tok = np.repeat(np.arange(T), counts).astype(np.int32)
        rng.shuffle(tok)
        N = tok.size
    else:
        T, k = 7, 32
        N, tok = T * k, None
    yp = rng.standard_normal((N, H)).astype(np.float32)
    pos = rng.permutation(N).astype(np.int32)
    pos[rng.choice(N, 6, replace=False)] = -1
    gates = rng.random(N).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    layer = B.Layer(H, 128, 8, k, B.MOE_BF16, None, None)
    y = torch.empty((T, H), dtype=torch.float32, device=d)
    B.moe_combine(layer, torch.from_numpy(yp).to(d), B.MOE_F32, torch.from_numpy(pos).to(d),
                  torch.from_numpy(tok).to(d) if tokens else None, torch.from_numpy(gates).to(d), N,
                  torch.from_numpy(sh).to(d), B.MOE_F32, T, y, B.MOE_F32, ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    y_ref = oracle.combine(yp.astype(np.float64), pos, gates, T, k=max(k, 1), tok=tok, shared=sh.astype(np.float64))
    assert rel_err_rows(to_np(y), y_ref).max() < 1e-6


def test_combine_of_permute_is_identity():
    """y_perm := x_perm (identity expert, bf16): k = 1 with gate 1 gives y == x
    bit for bit; k = 4 with all gates 1 gives y == 4x bit for bit."""
    rng = np.random.default_rng(12)
    T, H, E = 333, 512, 24
    d = dev()
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16).to(d)
    for k in (1, 4):
        N = T * k
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        layer = B.Layer(H, 128, E, k, B.MOE_BF16, None, None)
        ws = B.workspace(layer, T, N, d)
        off = torch.empty(E + 1, dtype=torch.int32, device=d)
        src = torch.empty(N, dtype=torch.int32, device=d)
        pos = torch.empty(N, dtype=torch.int32, device=d)
        xp = torch.empty((N, H), dtype=torch.bfloat16, device=d)
        B.moe_permute(layer, x, T, torch.from_numpy(ids).to(d), None, N, off, src, pos, xp, ws=ws)
        y = torch.empty((T, H), dtype=torch.bfloat16, device=d)
        B.moe_combine(layer, xp, B.MOE_BF16, pos, None, torch.ones(N, device=d), N, None, 0, T, y, B.MOE_BF16,
                      ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.float(), x.float() * k)


def test_combine_rounds_to_bf16_nearest_even():
    """One assignment per token with gate 1 and no shared expert: y = bf16(y_perm)
    (the single rounding of the combine).  Every bf16 store of the layer uses the
    same conversion; here it meets exact midpoints (ties to even both ways),
    values just either side of them, zeros, the largest finite values,
    overflow to infinity and fp32 subnormals, checked bit for bit against torch's
    round-to-nearest-even conversion on the CPU."""
    rng = np.random.default_rng(21)
    H = 512
    hi = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]                       # finite bf16 upper halves
    lo = np.concatenate([np.full(hi.size // 4, 0x8000), np.full(hi.size // 4, 0x7FFF),
                         np.full(hi.size // 4, 0x8001), rng.integers(0, 1 << 16, size=hi.size - 3 * (hi.size // 4))])
    bits = (hi << 16) | lo.astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
                        0x00000001, 0x80008000, 0x00018000, 0x007FFFFF, 0x00800000], dtype=np.uint32)
    bits = np.concatenate([special, bits])
    T = -(-bits.size // H)
    bits = np.resize(bits, T * H)
    vals = bits.view(np.float32).reshape(T, H)
    d = dev()
    layer = B.Layer(H, 128, 8, 1, B.MOE_BF16, None, None)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=d)
    pos = torch.arange(T, dtype=torch.int32, device=d)
    B.moe_combine(layer, torch.from_numpy(vals).to(d), B.MOE_F32, pos, None, torch.ones(T, device=d), T,
                  None, 0, T, y, B.MOE_BF16, ws=B.workspace(layer, T, T, d))
    torch.cuda.synchronize()
    # the sum starts from +0 (no shared expert), so -0 comes out as +0
    want = torch.from_numpy(vals + np.float32(0)).to(torch.bfloat16).view(torch.int16).numpy()
    got = y.cpu().view(torch.int16).numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, e.g. fp32 {bits.reshape(T, H)[bad][:4]} -> " \
                             f"{got[bad][:4].view(np.uint16)} (want {want[bad][:4].view(np.uint16)})"


# ------------------------------------------------------------------ whole layer

@pytest.mark.parametrize("name", ["small_bf16", "small_fp8"])
def test_forward_small_full_parity(name):
    cfg = W.get_config(name)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x, reg=REG[cfg.name])
    _print(f"forward {name}: {st}")


@pytest.mark.parametrize("name,over", [
    ("small_bf16", dict(T=517, I=128, Is=128)),                     # 128-row token tiles (mean 65 rows)
    ("small_fp8", dict(T=389)),                             # 128-row token tiles (mean 97 rows)
    ("small_bf16", dict(T=1500, I=256, Is=128)),                    # 256-row token tiles (mean 188 rows)
    ("small_fp8", dict(T=777)),                             # 256-row token tiles (mean 194 rows)
    ("small_fp8", dict(T=1100, zipf_s=1.1, zipf_beta=0.6)),  # 256-row tiles, skewed: 1..4 tiles per expert
])
def test_forward_tiled_path_reads_rows_through_permutation(name, over):
    """Enough rows per expert (mean >= 48) for the LDS-tiled kernels, which read
    the routed rows through the sort permutation (bf16 x directly, fp8 x
    quantised once per token) instead of a gathered copy; ragged T.  From a
    mean of 128 rows per expert the token tiles are 256 rows (eight-wave
    workgroups); the skewed case has experts with a few rows (waves whose
    token slices are all past the end) next to experts spanning several
    tiles."""
    cfg = W.get_config(name, **over)
    assert cfg.N / cfg.E >= 48 and cfg.I % 128 == 0 and cfg.Is % 128 == 0
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x)
    _print(f"forward tiled {name} {over}: {st}")


@pytest.mark.parametrize("name,over", [
    ("small_fp8", dict(Is=192)),                            # fp8 routed experts, streaming kernels
    ("small_fp8", dict(T=777, Is=192)),                     # fp8 routed experts, 256-row tiles
    ("small_bf16", dict(T=1500, I=256, Is=192)),                    # bf16 routed experts, 256-row tiles
])
def test_forward_shared_width_not_multiple_of_128(name, over):
    """A shared expert whose width is a multiple of 64 but not of 128 next to
    routed experts whose width is: the shared expert gets a launch of its own
    (streaming kernels, 64-column tiles) and the routed experts keep theirs
    (fp8 needs 128-column tiles; bf16 keeps the LDS-tiled kernels)."""
    cfg = W.get_config(name, **over)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x)
    _print(f"forward shared width {cfg.Is} {name} {over}: {st}")


@pytest.mark.parametrize("name,over", [
    ("small_fp8", dict(H=384, T=100)),              # mean 25 rows per expert: 32-row token tiles
    ("small_fp8", dict(H=384, T=180)),              # mean 45: 64-row token tiles
    ("small_bf16", dict(H=384, I=256, T=200)),      # mean 25, two weight tiles per workgroup
    ("small_bf16", dict(H=384, I=256, T=360)),      # mean 45
    ("small_mxfp4", dict(H=384, T=100)),            # mean 25, MX weights (odd chunk count)
    ("small_mxfp4", dict(H=384, T=180)),            # mean 45
])
def test_forward_streaming_many_rows_when_not_tileable(name, over):
    """H % 256 != 0 keeps the layer on the streaming kernels at any T, so their
    multi-slice token tiles (32 and 64 rows) still run once the tiled kernels
    take the tileable shapes from 10 rows per expert on.  Every token against
    the oracle, and the worst token plus three seeded ones run alone (T = 1,
    16-row tiles) must give the batched rows bit for bit: a token's output
    depends on no other token (at this H the router's K is never split, so
    its logits do not depend on T either)."""
    cfg = W.get_config(name, **over)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    # fp8 at H = 384: one token of seed 0 reaches 1.14e-2 (p99 5.8e-3, mean
    # 1.5e-3), the same bits when it runs alone; the other shapes stay < 3.2e-3
    reg = 1.5e-2 if name == "small_fp8" else REG.get(name, 1e-2)
    st = check_forward(lt, x, reg=reg)
    print(f"[{name} {over}] {st}", flush=True)
    OL = oracle_layer(lt)
    y, _, _ = run_forward(lt, x)
    y_ref, _, _, _ = oracle.forward(OL, W.bf16_bits(x))
    worst = int(rel_err_rows(to_np(y), y_ref).argmax())
    for t in sorted({worst, *np.random.default_rng(2).choice(cfg.T, 3, replace=False).tolist()}):
        y1, _, _ = run_forward(lt, x[t:t + 1].contiguous())
        assert torch.equal(y1[0], y[t]), f"token {t} alone differs from the batched run"


def test_forward_ragged_and_single_token():
    cfg = W.get_config("small_fp8")
    lt = W.make_layer(cfg, dev())
    OL = oracle_layer(lt)
    for T in (1, 17, 63):
        x = W.make_x(cfg, dev(), T=T)
        check_forward(lt, x, OL=OL)


@pytest.mark.parametrize("name,T", [("small_fp8", 40), ("small_fp8", 100), ("small_bf16", 43)])
def test_forward_top_k_above_8(name, T):
    """k = 12 of 32 experts: the combine's batched path (more than 8 slots a
    token); 480 assignments (the one-launch grouping), 516 and 1200 (the
    chunk-table sort, which also writes the tile list, then the gather);
    ragged T, fp8 and bf16 experts."""
    cfg = W.get_config(name, E=32, k=12, T=T)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x)
    _print(f"forward k=12 {name} T={T}: {st}")


def test_forward_bf16_output_and_k1_E1():
    cfg = W.get_config("small_bf16", E=1, k=1)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    check_forward(lt, x, out_dtype=torch.bfloat16)


def test_forward_zero_tokens():
    cfg = W.get_config("small_bf16")
    lt = W.make_layer(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    y = torch.empty((0, cfg.H), dtype=torch.float32, device=dev())
    B.moe_forward(layer, torch.empty((0, cfg.H), dtype=torch.bfloat16, device=dev()), 0, y)


def test_forward_deterministic_and_workspace_independent():
    cfg = W.get_config("small_fp8")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    ws = B.workspace(layer, cfg.T, cfg.N, dev())
    ws.fill_(0xFF)                              # NaN patterns everywhere
    y1, i1, g1 = run_forward(lt, x, ws=ws)
    ws.fill_(0x7F)
    y2, i2, g2 = run_forward(lt, x, ws=ws)
    for _ in range(20):
        y3, _, _ = run_forward(lt, x)
        assert torch.equal(y1, y3)
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(g1, g2)


def test_forward_token_order_equivariance():
    cfg = W.get_config("small_fp8")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    perm = torch.randperm(cfg.T, generator=torch.Generator().manual_seed(3)).to(dev())
    y, ids, _ = run_forward(lt, x)
    yp, idsp, _ = run_forward(lt, x[perm].contiguous())
    assert torch.equal(yp, y[perm]) and torch.equal(idsp, ids[perm])


def test_combine_many_tokens_uses_multiblock_scan():
    """More token bins than one workgroup scans (T > 4096): per-token order and sums."""
    rng = np.random.default_rng(21)
    T, H, N = 6000, 128, 9001
    d = dev()
    yp = rng.standard_normal((N, H)).astype(np.float32)
    pos = rng.permutation(N).astype(np.int32)
    tok = rng.integers(0, T, size=N).astype(np.int32)
    tok[rng.choice(N, 7, replace=False)] = T + 1
    gates = rng.random(N).astype(np.float32)
    layer = B.Layer(H, 128, 8, 0, B.MOE_BF16, None, None)
    y = torch.empty((T, H), dtype=torch.float32, device=d)
    B.moe_combine(layer, torch.from_numpy(yp).to(d), B.MOE_F32, torch.from_numpy(pos).to(d),
                  torch.from_numpy(tok).to(d), torch.from_numpy(gates).to(d), N, None, 0, T, y, B.MOE_F32,
                  ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    y_ref = oracle.combine(yp.astype(np.float64), pos, gates, T, tok=tok)
    assert rel_err_rows(to_np(y), y_ref).max() < 1e-6


def test_combine_per_token_grouping_without_chunk_table():
    """Many tokens and assignments (T = 40000, N = 60000: the stable sort's
    chunk table would pass 4M words), so the per-token grouping takes the
    O(N + T) path (atomic counts and placement, then a per-token rank pass):
    sums against the oracle, bit-identical repeats, and the summation order
    (increasing assignment index) on triples whose fp32 sum depends on it."""
    rng = np.random.default_rng(23)
    T, H, N = 40000, 128, 60000
    d = dev()
    yp = rng.standard_normal((N, H)).astype(np.float32)
    pos = rng.permutation(N).astype(np.int32)
    tok = rng.integers(0, T, size=N).astype(np.int32)
    tok[rng.choice(N, 9, replace=False)] = -3          # dropped
    gates = rng.random(N).astype(np.float32)
    # order probes: token t0 has exactly three assignments, i0 < i1 < i2 with
    # rows +2^25, 1, -2^25 and gates 1: in index order (2^25 + 1) - 2^25 = 0,
    # while -2^25 or 1 placed before 2^25 leaves 1
    probes = rng.choice(T, 50, replace=False)
    tok[np.isin(tok, probes)] = rng.choice(np.setdiff1d(np.arange(T), probes), int(np.isin(tok, probes).sum()))
    for t0 in probes:
        idx = np.sort(rng.choice(np.nonzero(~np.isin(tok, probes))[0], 3, replace=False))
        tok[idx] = t0
        for v, i in zip((2.0 ** 25, 1.0, -(2.0 ** 25)), idx):
            yp[pos[i]] = v
            gates[i] = 1.0
    layer = B.Layer(H, 128, 8, 0, B.MOE_BF16, None, None)
    args = (torch.from_numpy(yp).to(d), B.MOE_F32, torch.from_numpy(pos).to(d), torch.from_numpy(tok).to(d),
            torch.from_numpy(gates).to(d), N, None, 0, T)
    outs = []
    for _ in range(2):
        y = torch.empty((T, H), dtype=torch.float32, device=d)
        B.moe_combine(layer, *args, y, B.MOE_F32, ws=B.workspace(layer, T, N, d))
        torch.cuda.synchronize()
        outs.append(y)
    assert torch.equal(outs[0], outs[1])
    y = outs[0].cpu().numpy()
    assert (y[probes] == 0).all(), "assignments of a token were not summed in increasing index order"
    keep = ~np.isin(np.arange(T), probes)
    y_ref = oracle.combine(yp.astype(np.float64), pos, gates, T, tok=tok)
    assert rel_err_rows(y[keep], y_ref[keep]).max() < 1e-6


@pytest.mark.parametrize("name,over,N", [("small_fp8", dict(T=300), 700), ("small_fp8", dict(T=300, Is=192), 700),
                                         ("small_bf16", dict(T=150), 333), ("small_fp8", dict(T=2000), 6000)])
def test_forward_routed_matches_oracle(name, over, N):
    """moe_forward_routed on seeded pre-routed triples (some dropped: expert or
    token out of range; some tokens without an assignment) against the oracle
    on every token; small (streaming kernels) and large (LDS-tiled) shares,
    and a shared expert of a width that gets its own launch."""
    cfg = W.get_config(name, **over)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    rng = np.random.default_rng(N)
    T, E = cfg.T, cfg.E
    tok = rng.integers(0, T, size=N).astype(np.int32)
    exp = rng.integers(0, E, size=N).astype(np.int32)
    gate = rng.random(N).astype(np.float32)
    exp[rng.choice(N, 5, replace=False)] = E + 2
    tok[rng.choice(N, 5, replace=False)] = -1
    tok[np.isin(tok, [3, 7])] = 0               # tokens 3 and 7 get only the shared expert
    d = dev()
    layer = B.Layer.from_tensors(lt, top_k=0)
    y = torch.empty((T, cfg.H), dtype=torch.float32, device=d)
    B.moe_forward_routed(layer, x, T, torch.from_numpy(exp).to(d), torch.from_numpy(tok).to(d),
                         torch.from_numpy(gate).to(d), N, y, ws=B.workspace(layer, T, N, d))
    torch.cuda.synchronize()
    OL = oracle_layer(lt)
    y_ref = oracle.forward_triples(OL, W.bf16_bits(x), tok, exp, gate)
    err = rel_err_rows(to_np(y), y_ref)
    _print(f"forward_routed {name} {over} N={N}: max rel err {err.max():.3e}")
    assert err.max() < TOL[cfg.expert_dtype]
