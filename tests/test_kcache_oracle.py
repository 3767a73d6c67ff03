"""Pins for the oracle of the key-cache writer (per-token OCP E4M3
quantisation), checked against things other than the oracle itself: torch's
independent float8_e4m3fn cast, exact round trips of every code, ties at
every midpoint, closed forms of the scale, and the half-step error bound.
No GPU needed."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

E4M3_MAX = 448.0


def _code_values():
    return np.array([oracle.e4m3_decode(c) for c in range(256)])


def _torch_encode(v: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn cast of float32 values already clamped to +-448."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).clamp(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _encode_via_unit_scale(v: np.ndarray, D: int = 64) -> np.ndarray:
    """The oracle's codes for values v (|v| <= 448): each token carries 448 as
    its first element, so its scale is exactly 1 and the quotient is v itself."""
    v = np.asarray(v, dtype=np.float32).ravel()
    per = D - 1
    n = (len(v) + per - 1) // per
    k = np.zeros((n, D), np.float32)
    k[:, 0] = E4M3_MAX
    flat = np.zeros(n * per, np.float32)
    flat[: len(v)] = v
    k[:, 1:] = flat.reshape(n, per)
    codes, scale = oracle.quantize_k(k, 0)
    assert np.all(scale == 1.0)
    assert np.all(codes[:, 0] == 0x7E)
    return codes[:, 1:].ravel()[: len(v)]


def _midpoints_and_neighbours():
    vals = _code_values()[:127]  # 0 .. 448 ascending
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    assert np.all(m32.astype(np.float64) == mids)  # every midpoint is an fp32 value
    near = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(np.inf))])
    near = np.concatenate([near, vals.astype(np.float32)])
    return np.concatenate([near, -near])


def test_encode_anchors():
    # Codes fixed by the E4M3FN definition: 1.0 = 0x38, 448 = 0x7E, 2^-6 =
    # 0x08 (smallest normal), 2^-9 = 0x01 (smallest subnormal); saturation
    # above 448; ties to the even code; the sign of zero kept.
    cases = [(1.0, 0x38), (448.0, 0x7E), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01), (1e6, 0x7E),
             (-1e6, 0xFE), (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (7.5 * 2.0 ** -9, 0x08), (-0.0, 0x80), (0.0, 0x00), (-(2.0 ** -11), 0x80), (464.0, 0x7E)]
    for x, code in cases:
        assert oracle.e4m3_encode(x) == code, (x, hex(code))


def test_every_code_round_trips():
    vals = _code_values()
    for c in range(256):
        if math.isnan(vals[c]):
            continue
        assert oracle.e4m3_encode(vals[c]) == c, hex(c)


def test_encode_matches_torch_at_midpoints_and_neighbours():
    v = _midpoints_and_neighbours()
    np.testing.assert_array_equal(_encode_via_unit_scale(v), _torch_encode(v))
    # and the scalar entry point agrees with the unit-scale quantisation
    for x in v[::7]:
        assert oracle.e4m3_encode(float(x)) == _torch_encode(np.array([x]))[0]


def test_encode_matches_torch_on_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    v = np.clip(v, -E4M3_MAX, E4M3_MAX)
    np.testing.assert_array_equal(_encode_via_unit_scale(v), _torch_encode(v))


def test_encode_matches_torch_on_random_fp32():
    g = np.random.Generator(np.random.PCG64(21))
    parts = [g.uniform(-448, 448, 20000), g.standard_normal(20000) * 2.0 ** -7,
             g.standard_normal(20000) * 2.0 ** -12]
    bits = g.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    v = np.concatenate([p.astype(np.float32) for p in parts] + [bits.view(np.float32)])
    v = np.clip(v[np.isfinite(v)], -E4M3_MAX, E4M3_MAX)
    np.testing.assert_array_equal(_encode_via_unit_scale(v), _torch_encode(v))


def _token_mix(g, D):
    n = 12
    k = g.standard_normal((n, D)).astype(np.float32)
    k[1] *= 1e30
    k[2] *= 1e-30
    k[3] = 0.0
    k[4] = 0.0
    k[4, D // 2] = -3.0
    k[5] = np.float32(2.0 ** -130)  # subnormal fp32: below the scale floor
    k[6] = g.standard_t(2, D)  # heavy tails
    k[7] = -0.0
    k[8, :] = np.float32(1.0)
    k[9] = (g.integers(-4, 5, D)).astype(np.float32)
    k[10] *= 2.0 ** 120
    k[11] *= 2.0 ** -120
    return k


@pytest.mark.parametrize("D", [8, 64, 128, 136])
def test_quantize_matches_torch_quantiser_fp32(D):
    g = np.random.Generator(np.random.PCG64(100 + D))
    k = _token_mix(g, D)
    codes, scale = oracle.quantize_k(k, 0)
    ref_codes, ref_scale = W.quantize_e4m3_per_token(k)
    np.testing.assert_array_equal(scale.view(np.uint32), ref_scale.view(np.uint32))
    np.testing.assert_array_equal(codes, ref_codes)


def test_quantize_matches_torch_quantiser_bf16():
    g = np.random.Generator(np.random.PCG64(7))
    k = _token_mix(g, 128)
    bits = W.to_bf16_bits(k)
    codes, scale = oracle.quantize_k(bits, 1)
    ref_codes, ref_scale = W.quantize_e4m3_per_token(W.bf16_bits_to_f32(bits))
    np.testing.assert_array_equal(scale.view(np.uint32), ref_scale.view(np.uint32))
    np.testing.assert_array_equal(codes, ref_codes)


def test_scale_closed_forms():
    # amax = 448 * 2^j gives scale = 2^j exactly, and then every code is the
    # encoding of k / 2^j (an exact quotient).
    g = np.random.Generator(np.random.PCG64(3))
    for j in (-100, -20, -1, 0, 1, 7, 60):
        k = (g.uniform(-1, 1, (4, 32)) * 448 * 2.0 ** j).astype(np.float32)
        k[:, 5] = np.float32(448 * 2.0 ** j)
        codes, scale = oracle.quantize_k(k, 0)
        assert np.all(scale == np.float32(2.0 ** j))
        np.testing.assert_array_equal(codes, _torch_encode(k / np.float32(2.0 ** j)))
    # an all-zero token takes the floor scale and zero codes
    codes, scale = oracle.quantize_k(np.zeros((1, 16), np.float32), 0)
    assert scale[0] == np.float32(2.0 ** -126) / np.float32(448.0) and np.all(codes == 0)
    codes, _ = oracle.quantize_k(np.full((1, 16), -0.0, np.float32), 0)
    assert np.all(codes == 0x80)


def test_amax_maps_to_448_and_error_is_half_step():
    g = np.random.Generator(np.random.PCG64(5))
    k = (g.standard_normal((256, 128)) * np.exp(g.uniform(-30, 30, (256, 1)))).astype(np.float32)
    codes, scale = oracle.quantize_k(k, 0)
    vals = _code_values()
    arg = np.abs(k).argmax(1)
    assert np.all(codes[np.arange(256), arg] & 0x7F == 0x7E)
    deq = vals[codes] * scale[:, None].astype(np.float64)
    # normal codes: half a step is 2^-4 of the value's binade, i.e. <= 2^-4 |q|;
    # subnormal codes: half of 2^-9; both measured in units of the scale
    q = k.astype(np.float64) / scale[:, None]
    bound = np.maximum(np.abs(q) * 2.0 ** -4, 2.0 ** -10) * scale[:, None] * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - k) <= bound)
    # order preserving within a token
    for i in range(0, 256, 17):
        o = np.argsort(k[i], kind="stable")
        assert np.all(np.diff(deq[i, o]) >= 0)
