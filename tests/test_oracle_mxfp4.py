"""Pins of the oracle's MX FP4 expert-weight format (E2M1 codes two to a byte,
one E8M0 scale per 32 inputs of a row).

Pinned against: torch's float8_e8m0fnu decoder (library) for every scale
byte; the E4M3 decoder (itself pinned against torch) through the bit-level
embedding of E2M1 into E4M3; exact integer products on grid values with unit
scales (numpy int64 matmul); the fp8 block-scaled path of the same oracle on
weights that both formats hold exactly (bit-identical fp64 results, which
fixes nibble order, row stride, expert offsets and the per-32 scale index);
and the factored block form of the scaled MFMA against dequant-then-matmul.
The input-side quantiser of the synthetic workloads is checked against the
MX rules it states (round trip of representable values, ties to even,
saturation, zero blocks).
"""
import numpy as np
import pytest
import torch

from router_gemm_amd import workloads as W


def _e2m1_to_e4m3(code):
    """Bit-level embedding: E2M1 (S.EE.M, bias 1) -> the E4M3 code of the same value."""
    code = np.asarray(code, dtype=np.int64) & 15
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    # normal: exponent e - 1 -> E4M3 field e - 1 + 7; mantissa bit -> top mantissa bit
    normal = ((e + 6) << 3) | (m << 2)
    # subnormal: 0.5 * m -> zero, or 2^-1 (field 6, mantissa 0)
    sub = np.where(m == 1, 6 << 3, 0)
    mag = np.where(e == 0, sub, normal)
    return (mag | (s << 7)).astype(np.uint8)


def test_e2m1_values_through_e4m3_embedding(orc):
    codes = np.arange(16, dtype=np.uint8)
    got = orc.e2m1_decode(codes)
    want = orc.e4m3_decode(_e2m1_to_e4m3(codes))
    assert np.array_equal(got[[0, 8]], [0.0, 0.0])
    assert np.array_equal(got[1:8], want[1:8]) and np.array_equal(got[9:], want[9:])
    # the format's landmarks: largest 6, smallest normal 1, subnormal 0.5, sign bit 8
    assert got[7] == 6.0 and got[2] == 1.0 and got[1] == 0.5 and got[15] == -6.0
    # only the low nibble is read
    assert np.array_equal(orc.e2m1_decode(codes | 0xA0), got)


def test_e8m0_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def _mx_layer(orc, E, H, I, codes_gu, sc_gu, codes_d, sc_d, k=1):
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    return orc.Layer(H, I, E, k, "mxfp4", np.zeros((E, H), np.uint16), pack(codes_gu), pack(codes_d),
                     s_gate_up=sc_gu.astype(np.uint8), s_down=sc_d.astype(np.uint8))


def test_grid_values_unit_scales_are_exact(orc):
    # E2M1 codes of small integers, E4M3 codes of small integers, all scales 1
    E, H, I = 1, 256, 128
    rng = np.random.default_rng(11)
    w_ints = {1: 2, 2: 4, 3: 5, 4: 6, 6: 7, 0: 0, -1: 10, -2: 12, -3: 13, -4: 14, -6: 15}
    a_ints = {1: 0x38, 2: 0x40, 3: 0x44, -1: 0xB8, -2: 0xC0, 0: 0x00}
    wv = rng.choice(np.array(list(w_ints)), size=(E, 2 * I, H))
    av = rng.choice(np.array(list(a_ints)), size=H)
    wc = np.vectorize(w_ints.get)(wv).astype(np.int64)
    L = _mx_layer(orc, E, H, I, wc, np.full((E, 2 * I, H // 32), 127), np.zeros((E, H, I), np.int64),
                  np.full((E, H, I // 32), 127))
    a = np.vectorize(a_ints.get)(av).astype(np.uint8)
    ref = wv[0].astype(np.int64) @ av.astype(np.int64)
    for factored in (False, True):
        zg, zu = orc.expert_gate_up(L, 0, a, np.ones(2, np.float32), factored=factored)
        assert np.array_equal(zg, ref[:I].astype(np.float64))
        assert np.array_equal(zu, ref[I:].astype(np.float64))


def _pair(orc, seed, E=3, H=256, I=128, shared=False):
    """An MX layer with random codes and per-32 scales in 2^-3..2^3, and the fp8
    layer (unit block scales) that holds exactly the same weight values."""
    rng = np.random.default_rng(seed)
    cg = rng.integers(0, 16, size=(E, 2 * I, H))
    cd = rng.integers(0, 16, size=(E, H, I))
    sg = rng.integers(124, 131, size=(E, 2 * I, H // 32))
    sd = rng.integers(124, 131, size=(E, H, I // 32))

    def fp8_of(codes, sc):
        c = _e2m1_to_e4m3(codes).astype(np.int64)
        shift = np.repeat(sc - 127, 32, axis=-1)
        nz = (c & 0x7F) != 0
        mag = np.where(nz, (c & 0x7F) + (shift << 3), 0)   # exponent field + (scale - 127)
        assert mag.min() >= 0 and mag.max() <= 0x7E
        return (mag | (c & 0x80)).astype(np.uint8)

    wr = torch.randn(E, H, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    wr = wr.view(torch.int16).numpy().view(np.uint16)
    kw = {}
    if shared:
        g = torch.Generator().manual_seed(seed + 1)
        bits = lambda t: t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        kw = dict(w_shared_gate_up=bits(torch.randn(2 * 128, H, generator=g) * 0.05),
                  w_shared_down=bits(torch.randn(H, 128, generator=g) * 0.05))
    pack = lambda c: (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
    mx = orc.Layer(H, I, E, 2, "mxfp4", wr, pack(cg), pack(cd), s_gate_up=sg.astype(np.uint8),
                   s_down=sd.astype(np.uint8), **kw)
    f8 = orc.Layer(H, I, E, 2, "fp8", wr, fp8_of(cg, sg), fp8_of(cd, sd),
                   s_gate_up=np.ones((E, 2 * I // 128, H // 128), np.float32),
                   s_down=np.ones((E, H // 128, I // 128), np.float32), **kw)
    return mx, f8


def test_mx_equals_fp8_on_shared_values(orc):
    mx, f8 = _pair(orc, seed=5)
    rng = np.random.default_rng(6)
    for e in range(mx.E):
        q, s = orc.quant_row(rng.standard_normal(mx.H).astype(np.float32))
        o1, h1 = orc.expert_row(mx, e, q, s)
        o2, h2 = orc.expert_row(f8, e, q, s)
        assert np.array_equal(h1, h2) and np.array_equal(o1, o2)


def test_mx_forward_equals_fp8_forward(orc):
    mx, f8 = _pair(orc, seed=7, shared=True)
    x = torch.randn(9, mx.H, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    x = x.view(torch.int16).numpy().view(np.uint16)
    y1, ids1, g1, _ = orc.forward(mx, x)
    y2, ids2, g2, _ = orc.forward(f8, x)
    assert np.array_equal(ids1, ids2) and np.array_equal(g1, g2)
    assert np.array_equal(y1, y2)
    # the grouped-rows form on the same weights
    off = np.array([0, 4, 4, 9], np.int32)
    q, s = orc.quant_bf16_rows(x)
    assert np.array_equal(orc.expert_ffn(mx, off, q, s), orc.expert_ffn(f8, off, q, s))


def test_mx_factored_equals_dequant(orc):
    mx, _ = _pair(orc, seed=9)
    rng = np.random.default_rng(10)
    q, s = orc.quant_row(rng.standard_normal(mx.H).astype(np.float32))
    for e in range(mx.E):
        zg1, zu1 = orc.expert_gate_up(mx, e, q, s, factored=False)
        zg2, zu2 = orc.expert_gate_up(mx, e, q, s, factored=True)
        scale = np.abs(np.concatenate([zg1, zu1])).max()
        assert np.max(np.abs(zg1 - zg2)) <= 1e-12 * scale
        assert np.max(np.abs(zu1 - zu2)) <= 1e-12 * scale


def test_swapped_nibbles_change_the_result(orc):
    """A layer whose bytes have their nibbles swapped is a different layer
    (guards the equivalence tests against a symmetric mistake)."""
    mx, _ = _pair(orc, seed=12, E=1)
    sw = ((mx.w_gate_up >> 4) | (mx.w_gate_up << 4)).astype(np.uint8)
    mx2 = orc.Layer(mx.H, mx.I, 1, 1, "mxfp4", mx.w_router, sw, mx.w_down,
                    s_gate_up=mx.s_gate_up, s_down=mx.s_down)
    q, s = orc.quant_row(np.random.default_rng(13).standard_normal(mx.H).astype(np.float32))
    assert not np.array_equal(orc.expert_gate_up(mx, 0, q, s, False)[0],
                              orc.expert_gate_up(mx2, 0, q, s, False)[0])


# ---------------------------------------------------------------- input-side quantiser

def _mx_decode(orc, packed, sbytes):
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)
    return orc.e2m1_decode(codes) * np.repeat(orc.e8m0_decode(sbytes), 32, 1)


def test_quantiser_round_trips_representable_values(orc):
    # block b of row r: E2M1 grid values times 2^q, with one entry +-6 * 2^q so
    # that the block's scale is 2^q; every value is then held exactly
    rng = np.random.default_rng(20)
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6])
    qexp = rng.integers(-6, 3, size=(16, 4))
    w = rng.choice(vals, size=(16, 4, 32))
    w[:, :, 0] = rng.choice([-6.0, 6.0], size=(16, 4))
    w = (w * 2.0 ** qexp[:, :, None]).reshape(16, 128)
    q, s = W.quantize_mxfp4(torch.from_numpy(w.astype(np.float32)))
    assert np.array_equal(s.numpy().astype(np.int64), qexp + 127)
    assert np.array_equal(_mx_decode(orc, q.numpy(), s.numpy()), w)


def test_quantiser_ties_saturation_and_zero_blocks(orc):
    # one block of 32 with amax 4 -> scale 2^(2-2) = 1; midpoints go to the even code
    row = np.zeros(64, np.float32)
    row[:10] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -0.75, 0.3, 1.3]
    row[32:] = 0.0                                          # an all-zero block
    q, s = W.quantize_mxfp4(torch.from_numpy(row[None]))
    back = _mx_decode(orc, q.numpy(), s.numpy())[0]
    assert s.numpy()[0, 0] == 127 and s.numpy()[0, 1] == 127
    assert list(back[:10]) == [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, -1.0, 0.5, 1.5]
    assert np.all(back[32:] == 0) and np.all(q.numpy()[0, 16:] == 0)
    # amax 7.5 -> scale 2^(2-2) = 1, 7.5 saturates to 6; 5.0 is a tie between 4 and 6 -> 4
    row2 = np.zeros(32, np.float32)
    row2[:3] = [7.5, 5.0, -7.9]
    q2, s2 = W.quantize_mxfp4(torch.from_numpy(row2[None]))
    b2 = _mx_decode(orc, q2.numpy(), s2.numpy())[0]
    assert s2.numpy()[0, 0] == 127 and list(b2[:3]) == [6.0, 4.0, -6.0]


@pytest.mark.parametrize("std", [0.02, 3.0])
def test_quantiser_error_bound(orc, std):
    """Each value is within half a grid step of the E2M1 grid at its block's
    scale, except values saturated at 6 * scale."""
    w = torch.randn(32, 256, generator=torch.Generator().manual_seed(21)) * std
    q, s = W.quantize_mxfp4(w)
    back = _mx_decode(orc, q.numpy(), s.numpy())
    wn = w.double().numpy()
    scale = np.repeat(orc.e8m0_decode(s.numpy()), 32, 1)
    a = np.abs(wn) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(back - wn) / scale
    sat = a > 6
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.all(np.abs(back[sat]) == 6 * scale[sat])
