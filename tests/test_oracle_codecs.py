"""Pins of the oracle's number codecs and its 1x128 activation quantiser.

Pinned against: values fixed by the OCP 8-bit E4M3 definition (a handful of
codes with known values), torch's own float8_e4m3fn and bfloat16 conversions
(independent library routines), round trips, and closed-form error bounds.
"""
import numpy as np
import pytest
import torch


def test_e4m3_known_codes(orc):
    # OCP E4M3: bias 7, 3 mantissa bits, subnormal step 2^-9, max 448, NaN at S.1111.111
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x44: 3.0, 0x7E: 448.0, 0x7D: 416.0,
             0xB8: -1.0, 0xFE: -448.0}
    for code, val in known.items():
        assert orc.e4m3_decode(code) == val, hex(code)
    assert np.isnan(orc.e4m3_decode(0x7F)) and np.isnan(orc.e4m3_decode(0xFF))
    assert np.signbit(orc.e4m3_decode(0x80)) and orc.e4m3_decode(0x80) == 0.0


def test_e4m3_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(lib)
    assert np.all(both_nan | (ours == lib))
    assert both_nan.sum() == 2


def test_e4m3_roundtrip_all_finite_codes(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = orc.e4m3_decode(codes).astype(np.float32)
    back = orc.e4m3_encode(vals)
    # +0 and -0 keep their sign bit
    assert np.array_equal(back, codes)


def test_e4m3_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(1)
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (v[:-1] + v[1:]) / 2          # exact ties: must go to the even mantissa
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    cases = np.concatenate([
        mids32, np.nextafter(mids32, np.float32(0)), np.nextafter(mids32, np.float32(1e9)),
        rng.uniform(-448, 448, 20000).astype(np.float32),
        (rng.standard_normal(20000) * 0.01).astype(np.float32),    # subnormal-heavy
        np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6]),
    ]).astype(np.float32)
    cases = np.concatenate([cases, -cases])
    ours = orc.e4m3_encode(cases)
    lib = torch.from_numpy(cases).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != lib)[0]
    assert bad.size == 0, [(float(cases[i]), hex(ours[i]), hex(lib[i])) for i in bad[:5]]
    # ties-to-even spot checks: 1.0625 lies between 1.0 (m=0) and 1.125 (m=1) -> 1.0;
    # 1.1875 between 1.125 (m=1) and 1.25 (m=2) -> 1.25
    assert orc.e4m3_encode(np.float32([1.0625, 1.1875])).tolist() == [0x38, 0x3A]


def test_e4m3_encode_saturates_and_nan(orc):
    out = orc.e4m3_encode(np.float32([449.0, 463.9, 464.0, 1e6, np.inf, -1e6, -np.inf]))
    assert out.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.e4m3_encode(np.float32([np.nan]))[0] & 0x7F == 0x7F


def test_bf16_codec_matches_torch(orc):
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, 1e-40]])
    ours = orc.bf16_encode(v)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)
    dec = orc.bf16_decode(ours[:2000])
    ref = torch.from_numpy(ours[:2000].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(dec, ref)
    # ties to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1.0
    assert orc.bf16_encode([1.0 + 2.0 ** -8])[0] == 0x3F80


def test_quant_row_grid_values_are_lossless(orc):
    # A group whose values are e4m3 grid points times 2^j, with max |v| = 448 * 2^j,
    # quantises with scale exactly 2^j and reproduces every code.
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, size=256).astype(np.uint8)
    codes[rng.random(256) < 0.5] |= 0x80
    codes[0], codes[128] = 0x7E, 0xFE          # amax of each group is 448
    j = np.array([-20, 3])
    grid = orc.e4m3_decode(codes)
    v = (grid * np.repeat(2.0 ** j, 128)).astype(np.float32)
    q, s = orc.quant_row(v)
    assert np.array_equal(s, (2.0 ** j).astype(np.float32))
    assert np.array_equal(q, codes)


def test_quant_row_zero_group_and_bounds(orc):
    rng = np.random.default_rng(4)
    v = np.concatenate([np.zeros(128), rng.standard_normal(384) * 3]).astype(np.float32)
    q, s = orc.quant_row(v)
    assert s[0] == 1.0 and np.all(q[:128] == 0)
    deq = orc.e4m3_decode(q) * np.repeat(s.astype(np.float64), 128)
    for g in range(1, 4):
        blk = v[g * 128:(g + 1) * 128].astype(np.float64)
        amax = np.abs(blk).max()
        assert s[g] == np.float32(np.float32(amax) / np.float32(448.0))
        assert np.max(np.abs(q[g * 128:(g + 1) * 128] & 0x7F)) == 0x7E   # amax -> 448
        err = np.abs(deq[g * 128:(g + 1) * 128] - blk)
        # half an ulp: 2^-4 relative in the normal range, 2^-10 * s in the subnormal range
        bound = np.maximum(np.abs(blk) * 2.0 ** -4, float(s[g]) * 2.0 ** -10) * (1 + 1e-6)
        assert np.all(err <= bound)


def test_quant_bf16_rows_matches_row_quantiser(orc):
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((3, 256)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    q, s = orc.quant_bf16_rows(xb)
    for r in range(3):
        q1, s1 = orc.quant_row(x[r].float().numpy())
        assert np.array_equal(q[r], q1) and np.array_equal(s[r], s1)
