"""Pins of the oracle's E4M3 encoding and per-row FP8 weight quantization.

The E4M3 grid is checked against values the OCP 8-bit floating-point format fixes
(1.0, the largest finite value 448, the smallest normal and subnormal values, NaN
codes) and the encoder against an independent library conversion
(``torch.float8_e4m3fn`` on the CPU, round to nearest even) on the grid, on every
midpoint between neighbours (where ties to even decide) and on random values.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def lib_codes(x):
    """E4M3 codes by torch's CPU conversion (values within +-448; -0 taken as 0)."""
    c = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.where(c == 0x80, 0, c).astype(np.uint8)


def test_e4m3_grid():
    v = oracle.e4m3_values()
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v).sum() == 254
    assert (np.diff(v[:127]) > 0).all()
    # the grid against the library's own decoding of every code
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    fin = np.isfinite(v)
    np.testing.assert_array_equal(v[fin], lib[fin])


def test_e4m3_encode_matches_library():
    grid = oracle.e4m3_values()[:127]
    mids = (grid[:-1] + grid[1:]) / 2                       # exactly representable in float32
    r = np.random.default_rng(0)
    rnd = np.exp(r.uniform(np.log(1e-4), np.log(448.0), size=20000)) * r.choice([-1, 1], size=20000)
    for x in (grid, -grid, mids, -mids, rnd):
        x32 = np.asarray(x, dtype=np.float32)
        np.testing.assert_array_equal(oracle.e4m3_encode(x32), lib_codes(x32))
    # ties go to the even code: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39)
    assert oracle.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert oracle.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    # saturation instead of NaN above the largest finite value
    np.testing.assert_array_equal(oracle.e4m3_encode(np.array([449.0, 464.0, 1e6, -1e6])), [0x7E, 0x7E, 0x7E, 0xFE])
    assert (oracle.e4m3_decode(oracle.e4m3_encode(grid)) == grid).all()


def test_quantize_rows():
    r = np.random.default_rng(1)
    w = (r.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[5] = 0.0
    w[9, :] = 0.0
    w[9, 3] = -1e-3
    codes, scale = oracle.quantize_fp8_rows(w)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    amax = np.abs(w).max(axis=1)
    np.testing.assert_array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    assert scale[5] == 0 and (codes[5] == 0).all()
    # every nonzero row's largest magnitude lands on +-448
    for i in range(64):
        if amax[i] > 0:
            j = int(np.argmax(np.abs(w[i])))
            assert codes[i, j] in (0x7E, 0xFE)
    assert codes[9, 3] == 0xFE
    deq = oracle.dequantize_fp8_rows(codes, scale)
    # within half a grid step: 2^-4 relative on normal codes, scale * 2^-10 on subnormals
    err = np.abs(deq - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()
    # codes are the library's encoding of w / scale (float32 division)
    ok = scale > 0
    x = (w[ok] / scale[ok, None]).astype(np.float32)
    np.testing.assert_array_equal(codes[ok], lib_codes(x))


def test_fp8_model_weights():
    dims = synth.workload("t_small").dims
    W = synth.make_weights(dims, 3)
    m8, m16 = oracle.Model(dims, W, fp8=True), oracle.Model(dims, W)
    for name in ("embed", "ps_left", "l0.g_attn", "g_final"):
        np.testing.assert_array_equal(m8.w(name), m16.w(name))
    for name in ("lm_head", "w_fc", "l1.w_q", "l0.w_down"):
        a, b = m8.w(name), m16.w(name)
        assert not np.array_equal(a, b)
        assert np.abs(a - b).max() <= np.abs(b).max() * 2.0 ** -4
    with pytest.raises(ValueError):
        oracle.Model(synth.workload("t_f32").dims, {}, fp8=True)
