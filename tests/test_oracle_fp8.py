"""Pins of the oracle's fp8 (E4M3) latent cache reading, CPU only.

The pages name an 8-bit cache for inference ("MLA多头潜在注意力机制", 9.2
部署注意事项) without a format or scale; the reading is E4M3 with one float32
scale per cache tensor (see the oracle's fp8 section). What pins it here,
none of it computed by the oracle:

* every code's value against torch's float8_e4m3fn conversion, a library
  implementation of the same format, and a few values written out from the
  format's definition;
* the encoder against a brute-force search over the 254 finite values (ties
  to the even code), against torch inside the finite range, and against the
  saturation and special-value rules;
* the error bound of a round trip (half a spacing: 2^-4 relative for normal
  values, 2^-10 absolute below 2^-6);
* the scale folding that the library uses (scores and outputs computed on the
  codes' values with the scales moved into the query and the output) against
  the unabsorbed decode of the dequantised cache: linearity, up to rounding.
"""

import math

import numpy as np
import pytest
import torch

import oracle

CODES = np.arange(256, dtype=np.uint8)


def torch_values():
    return torch.from_numpy(CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_encode(x):
    """Nearest finite E4M3 value by exhaustive search (values from torch), ties
    to the even code; |x| > 448 saturates."""
    vals = torch_values()
    finite = ~np.isnan(vals)
    codes, v = CODES[finite], vals[finite]
    out = []
    for xi in np.asarray(x, dtype=np.float64).ravel():
        if abs(xi) > 448.0:
            out.append(0x7E | (0x80 if xi < 0 else 0))
            continue
        d = np.abs(v - xi)
        best = np.flatnonzero(d == d.min())
        # candidates at the same distance: two neighbours (take the even
        # code) and, where zero is one, both zeros (a result that rounds to
        # zero keeps the sign of x)
        cand = [int(codes[i]) for i in best]
        even = [c for c in cand if c % 2 == 0] or cand
        if len(even) > 1:
            neg = math.copysign(1.0, xi) < 0
            even = [c for c in even if bool(c & 0x80) == neg]
        out.append(even[0])
    return np.array(out, dtype=np.uint8).reshape(np.shape(x))


def test_decode_matches_torch_for_every_code():
    got, want = oracle.e4m3_decode(CODES), torch_values()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_closed_forms():
    v = oracle.e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x07, 0x08, 0x40, 0x00, 0x80, 0xFE, 0x7F,
                                     0xFF, 0x3C], np.uint8))
    assert v[0] == 1.0                   # exponent 7 = bias, mantissa 0
    assert v[1] == 448.0                 # 2^8 * 1.75, the largest finite value
    assert v[2] == 2.0 ** -9             # smallest subnormal
    assert v[3] == 7 * 2.0 ** -9         # largest subnormal
    assert v[4] == 2.0 ** -6             # smallest normal
    assert v[5] == 2.0
    assert v[6] == 0.0 and not np.signbit(v[6])
    assert v[7] == 0.0 and np.signbit(v[7])
    assert v[8] == -448.0
    assert np.isnan(v[9]) and np.isnan(v[10])
    assert v[11] == 1.5
    assert int(np.isfinite(oracle.e4m3_decode(CODES)).sum()) == 254


def test_every_finite_code_round_trips():
    vals = oracle.e4m3_decode(CODES)
    ok = ~np.isnan(vals)
    assert np.array_equal(oracle.e4m3_encode(vals[ok]), CODES[ok])


def _samples(seed, n):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * np.exp2(rng.uniform(-13.0, 9.5, n))
    # exact midpoints between neighbouring finite values, both signs
    vals = np.sort(np.unique(torch_values()[~np.isnan(torch_values())]))
    mids = 0.5 * (vals[1:] + vals[:-1])
    return np.concatenate([x, mids, -mids, [0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 470.0]])


def test_encode_matches_brute_force_search():
    x = _samples(1, 4000)
    assert np.array_equal(oracle.e4m3_encode(x), brute_encode(x))


def test_encode_matches_torch_inside_the_finite_range():
    # torch rounds to nearest even like the reading, but sends values past
    # 464 to NaN instead of saturating, so it is compared up to 464 only
    x = _samples(2, 20000).astype(np.float32)
    x = x[np.abs(x) <= 464.0]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), t)


def test_saturation_and_special_values():
    got = oracle.e4m3_encode([449.0, 480.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -0.0,
                              2.0 ** -10, 3 * 2.0 ** -11, 15 * 2.0 ** -10])
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80,
                            0x00,   # a tie between 0 and 2^-9: the even code 0
                            0x01,   # 1.5 * 2^-10 is nearer 2^-9
                            0x08]   # 7.5 * 2^-9: a tie, the even code is 2^-6


def test_round_trip_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000) * np.exp2(rng.uniform(-12.0, 8.5, 50000))
    x = x[np.abs(x) <= 448.0]
    y = oracle.e4m3_decode(oracle.e4m3_encode(x))
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(np.abs(y - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(y - x)[~normal] <= 2.0 ** -10)
    # monotone: a larger input never gets a smaller value
    order = np.argsort(x)
    assert np.all(np.diff(y[order]) >= 0)


def test_quantize_with_scale():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1000) * 3.0
    s = 0.0523  # 448 s = 23.4: every |x| / s in the finite range
    codes = oracle.fp8_quantize(x, s)
    assert np.array_equal(codes, oracle.e4m3_encode(x / s))
    y = oracle.fp8_dequantize(codes, s)
    assert np.allclose(y, s * oracle.e4m3_decode(codes), rtol=0, atol=0)
    assert np.all(np.abs(y - x) <= 2.0 ** -4 * np.abs(x) + s * 2.0 ** -10)
    # past 448 s the stored value saturates
    assert np.array_equal(oracle.fp8_dequantize(oracle.fp8_quantize([30.0, -1e9], s), s),
                          [448.0 * s, -448.0 * s])


@pytest.mark.parametrize("n", [1, 2, 4])
def test_scales_fold_into_query_and_output(n):
    # the library decodes an fp8 cache on the codes' values: q~ times
    # ckv_scale, rho times krope_scale, the output times ckv_scale. That is
    # the decode of the dequantised cache (both sides are linear in the
    # scales); the unabsorbed oracle on the dequantised cache is the reference.
    rng = np.random.default_rng(5 + n)
    B, H, d_c, d_r, d_n, d_v, L = 2, 3, 8 * n, 4, 5, 3, 9
    sc, sr = 0.031, 0.47
    ckv8 = oracle.fp8_quantize(rng.standard_normal((B, L, d_c)), sc)
    kr8 = oracle.fp8_quantize(rng.standard_normal((B, L, d_r)), sr)
    q_nope, q_rope = rng.standard_normal((B, H, d_n)), rng.standard_normal((B, H, d_r))
    w_uk = rng.standard_normal((H, d_c, d_n)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c)
    lens = np.array([L, 4], np.int32)
    tau, aq, akv = 0.3, 1.7, 0.6
    ref = oracle.mlra_decode_ref(q_nope, q_rope, w_uk, w_uv, oracle.fp8_dequantize(ckv8, sc),
                                 oracle.fp8_dequantize(kr8, sr), lens, n, tau=tau, alpha_q=aq,
                                 alpha_kv=akv)
    qa = oracle.absorb_q_ref(q_nope, q_rope, w_uk, lens - 1, tau, aq)
    qa[..., :d_c] *= sc
    qa[..., d_c:] *= sr
    lo = oracle.latent_attn_ref(qa, oracle.e4m3_decode(ckv8), oracle.e4m3_decode(kr8), lens, n)
    got = oracle.out_proj_ref(lo, w_uv, akv * sc)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
