"""Pins for the oracle's MXFP4 codec, bf16 rounding and SwiGLU.

Each test checks the oracle against something other than itself: a library
routine (torch's UE8M0 and bf16 conversions), a literal table of the format,
a brute-force search that uses a different algorithm from the oracle's, or an
invariant the format fixes.
"""
import math

import numpy as np
import pytest
import torch

import oracle

# E2M1 magnitudes as the OCP Microscaling element table lists them for codes
# 0..7 (sign is bit 3).  The XFP blog (section "路线二：硬件格式（NVFP4 / MXFP4）")
# fixes the split 1 sign + 2 exponent + 1 mantissa bits and that the 16 codes form
# a fixed codebook; the layer's quantiser saturates at +-6, the largest entry.
E2M1_LITERAL = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_matches_literal_table_and_sign_symmetry():
    for c in range(8):
        assert oracle.e2m1_value(c) == E2M1_LITERAL[c]
        assert oracle.e2m1_value(c | 8) == -E2M1_LITERAL[c]
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0  # code 8 is -0


def test_e2m1_structure():
    mags = [oracle.e2m1_value(c) for c in range(8)]
    assert all(a < b for a, b in zip(mags, mags[1:]))       # monotone in the code
    assert max(mags) == 6.0                                   # saturation bound
    # 1 mantissa bit: every non-zero magnitude is 2^p or 1.5 * 2^p
    for m in mags[1:]:
        p = math.floor(math.log2(m))
        assert m in (2.0 ** p, 1.5 * 2.0 ** p)
    # 2 exponent bits with bias 1: normals span exponents 0..2, one subnormal 0.5
    assert sorted({math.floor(math.log2(m)) for m in mags[2:]}) == [0, 1, 2]
    assert mags[1] == 0.5


def test_ue8m0_matches_torch_e8m0():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.ue8m0_value(s) for s in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    np.testing.assert_array_equal(got[:255], ref[:255])


def test_dequant_every_byte_every_scale():
    # every (code pair, scale byte) combination: 256 rows, each holding the same 16
    # bytes (32 codes) so that every scale byte is paired with every code byte
    codes_bytes = np.arange(256, dtype=np.uint8)
    K = 32
    rows = []
    scales = []
    for s in range(256):
        for b0 in range(0, 256, 16):
            rows.append(codes_bytes[b0:b0 + 16])
            scales.append([s])
    codes = np.array(rows, dtype=np.uint8)
    sc = np.array(scales, dtype=np.uint8)
    got = oracle.dequant(codes, sc, K).astype(np.float64)
    e8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    lit = np.array(E2M1_LITERAL + [-v for v in E2M1_LITERAL])
    lo = lit[codes & 0x0F]
    hi = lit[codes >> 4]
    expect = np.empty_like(got)
    expect[:, 0::2] = lo       # element 2i: low nibble of byte i
    expect[:, 1::2] = hi
    expect = (expect * e8[sc[:, :1]]).astype(np.float32).astype(np.float64)
    nan_rows = sc[:, 0] == 255
    assert np.isnan(got[nan_rows]).all()
    np.testing.assert_array_equal(got[~nan_rows], expect[~nan_rows])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7F8001,
                        0x00008000, 0x00018000, 0x3F808000, 0x3F818000, 0x7F800000,
                        0xFF800000, 0x00000001, 0x807FFFFF], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    f = bits.view(np.float32)
    got = oracle.bf16_from_f32(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(f)
    np.testing.assert_array_equal(got[~isnan], ref[~isnan])
    # NaN: a quiet NaN with the input's sign
    g = got[isnan]
    assert ((g & 0x7FC0) == 0x7FC0).all()
    np.testing.assert_array_equal(g >> 15, (bits[isnan] >> 31).astype(np.uint16))


def _brute_force_codes(vals: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Argmin over the 16 grid points of |v / 2^(S-127) - grid|, in fp64; on a
    distance tie the even code wins; the sign bit is always the input's."""
    r = vals / np.ldexp(1.0, scale.astype(np.int64) - 127)
    mags = np.array(E2M1_LITERAL)
    d = np.abs(np.abs(r)[..., None] - mags)           # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among the nearest magnitudes pick the even index if there is one
    idx = np.where(cand[..., 0::2].any(-1), np.argmax(cand[..., 0::2], -1) * 2,
                   np.argmax(cand, -1))
    sign = np.signbit(vals).astype(np.int64) << 3
    return (sign | idx).astype(np.uint8)


@pytest.mark.parametrize("anchor_shift", [0, 1, 3, 7])
def test_quantiser_brute_force_every_bf16(anchor_shift):
    """Every finite bf16 value v, quantised in a block whose largest element is
    2^(floor(log2|v|) + anchor_shift) (shift 0: v itself sets the scale)."""
    allb = np.arange(1 << 16, dtype=np.uint32)
    f = (allb << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(f) & (f != 0)
    v = f[fin]
    if anchor_shift == 0:
        anchor = np.abs(v)
    else:
        e = np.floor(np.log2(np.abs(v)))
        anchor = np.ldexp(1.0, (e + anchor_shift).astype(np.int64))
        keep = np.isfinite(anchor) & (anchor < 3.0e38)
        v, anchor = v[keep], anchor[keep]
    blocks = np.empty((v.size, 32), dtype=np.float64)
    blocks[:, 0] = anchor
    blocks[:, 1:] = v[:, None]
    blocks[:, 2::2] *= -1.0
    codes, scales = oracle.quantize(blocks)
    # the scale puts the block maximum's magnitude in [4, 8) unless clamped
    s = scales[:, 0].astype(np.int64)
    scaled_max = anchor / np.ldexp(1.0, s - 127)
    unclamped = (s > 0) & (s < 254)
    assert ((scaled_max[unclamped] >= 4.0) & (scaled_max[unclamped] < 8.0)).all()
    nib = np.empty((v.size, 32), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    expect = _brute_force_codes(blocks, np.repeat(scales, 32, axis=1))
    np.testing.assert_array_equal(nib, expect)


def test_quantiser_ties_go_to_even_code():
    # a block with max 4 (scale byte 127), then the grid midpoints
    vals = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0, 0.2, 6.9] + [0.0] * 19
    codes, scales = oracle.quantize(np.array([vals], dtype=np.float64))
    assert scales[0, 0] == 127
    nib = np.empty(32, dtype=np.uint8)
    nib[0::2] = codes[0] & 0x0F
    nib[1::2] = codes[0] >> 4
    assert list(nib[:13]) == [6, 0, 2, 2, 4, 4, 6, 6, 7, 8, 14, 0, 7]


def test_quantiser_special_blocks():
    z = np.zeros((1, 32))
    z[0, 3] = -0.0
    c, s = oracle.quantize(z)
    assert s[0, 0] == 0
    assert c[0, 1] == 0x80 and (np.delete(c[0], 1) == 0).all()   # element 3 keeps its sign
    for bad in (np.nan, np.inf, -np.inf):
        b = np.ones((1, 32))
        b[0, 17] = bad
        c, s = oracle.quantize(b)
        assert s[0, 0] == 255 and (c == 0).all()
    # tiny block: exponent clamps at 0
    t = np.full((1, 32), 2.0 ** -140)
    c, s = oracle.quantize(t)
    assert s[0, 0] == 0
    # decoded value: nearest grid point of 2^-140 / 2^-127 = 2^-13 -> 0
    assert (oracle.dequant(c, s, 32) == 0).all()


def test_quantiser_idempotent_and_exact_round_trip():
    rng = np.random.default_rng(3)
    v = rng.standard_t(3, size=(2048, 64)) * 0.02
    c1, s1 = oracle.quantize(v)
    d1 = oracle.dequant(c1, s1, 64)
    c2, s2 = oracle.quantize(d1.astype(np.float64))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    # blocks built on the grid with a magnitude-4 or -6 element come back exactly
    idx = rng.integers(0, 16, size=(512, 32))
    idx[:256, 5] = 6
    idx[256:, 9] = 15
    p = rng.integers(-20, 20, size=(512, 1))
    lit = np.array(E2M1_LITERAL + [-x for x in E2M1_LITERAL])
    vals = lit[idx] * np.ldexp(1.0, p)
    c, s = oracle.quantize(vals)
    np.testing.assert_array_equal(oracle.dequant(c, s, 32).astype(np.float64), vals)
    np.testing.assert_array_equal(s[:, 0], (p[:, 0] + 127).astype(np.uint8))


def test_quantiser_input_types_agree():
    rng = np.random.default_rng(11)
    v32 = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    bits = v32.view(np.uint32) & np.uint32(0xFFFF0000)       # exact bf16 values
    vb = bits.view(np.float32)
    c_f32, s_f32 = oracle.quantize(vb)
    c_f64, s_f64 = oracle.quantize(vb.astype(np.float64))
    c_b, s_b = oracle.quantize((bits >> 16).astype(np.uint16))
    np.testing.assert_array_equal(c_f32, c_f64)
    np.testing.assert_array_equal(c_b, c_f64)
    np.testing.assert_array_equal(s_b, s_f64)


def test_swiglu_clamp_and_nan():
    L = 7.0
    # plain silu(g)*u in fp64, compared within fp32 rounding
    for g, u in [(0.3, -1.2), (-2.0, 0.5), (5.0, 3.0), (-6.5, -6.9)]:
        ref = g / (1.0 + math.exp(-g)) * u
        assert abs(oracle.swiglu(g, u, L) - ref) <= 4e-7 * max(1.0, abs(ref))
    assert oracle.swiglu(0.0, 5.0, L) == 0.0
    assert oracle.swiglu(100.0, 1.0, L) == oracle.swiglu(7.0, 1.0, L)      # gate <= L
    assert oracle.swiglu(-100.0, 1.0, L) != oracle.swiglu(-7.0, 1.0, L)    # no lower gate clamp
    assert oracle.swiglu(2.0, 50.0, L) == oracle.swiglu(2.0, 7.0, L)
    assert oracle.swiglu(2.0, -50.0, L) == oracle.swiglu(2.0, -7.0, L)
    assert math.isnan(oracle.swiglu(float("nan"), 1.0, L))
    assert math.isnan(oracle.swiglu(1.0, float("nan"), L))
    big = 1e6
    ref = big * 1.0 * 3.0
    assert oracle.swiglu(big, 3.0, float("inf")) == pytest.approx(ref, rel=1e-6)
