"""Pins of the oracle's E4M3 (8-bit float) codes and per-row E4M3 quantiser.

Each pin is something other than the oracle's own formula: torch's CPU
float8_e4m3fn conversions (a library routine), the format's closed-form
values, a brute-force nearest search over all finite codes, a row worked by
hand, and invariants of the per-row scale (the row maximum lands on 448,
power-of-two scaling, the relative error of a 3-bit mantissa).
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth


def _torch_values():
    import torch

    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _torch_round(y):
    import torch

    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_values_match_torch_and_closed_forms():
    v = O.e4m3_value(np.arange(256))
    assert np.array_equal(v, _torch_values(), equal_nan=True)
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # 1.75 * 2^8, the largest value
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6   # smallest subnormal, smallest normal
    assert v[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert v[0x38] == 1.0 and v[0x40] == 2.0 and v[0x3C] == 1.5
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isfinite(v).sum() == 254
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                          # bytes 0..126 increase


def test_round_matches_torch():
    v = O.e4m3_value(np.arange(256))
    fin = v[np.isfinite(v)]
    mags = np.unique(np.abs(fin))
    mids = (mags[:-1] + mags[1:]) / 2                        # exact ties: ties go to the even mantissa
    rng = synth.rng(960)
    logu = np.exp2(rng.uniform(-12, np.log2(448.0), 20000)) * rng.choice([-1.0, 1.0], 20000)
    ys = np.concatenate([fin, mids, -mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), logu,
                         [0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -11, 1e-30, 447.99, 448.0]])
    ys = ys.astype(np.float32).astype(np.float64)  # torch converts from float32
    assert np.array_equal(O.round_e4m3(ys), _torch_round(ys))
    # every finite byte rounds to itself
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F])
    assert np.array_equal(O.round_e4m3(O.e4m3_value(codes)), codes.astype(np.uint8))


def test_round_is_nearest_by_brute_force_and_saturates():
    v = O.e4m3_value(np.arange(256))
    finite = np.array([c for c in range(256) if np.isfinite(v[c])])
    rng = synth.rng(961)
    y = rng.uniform(-460.0, 460.0, 3000)
    y[:1000] *= 2.0 ** -8
    got = O.round_e4m3(y)
    err = np.abs(v[got] - np.clip(y, -448, 448))
    best = np.min(np.abs(v[finite][None, :] - np.clip(y, -448, 448)[:, None]), axis=1)
    assert np.array_equal(err, best)
    assert np.all(np.sign(v[got]) * np.sign(y) >= 0)
    assert np.array_equal(O.round_e4m3(np.array([500.0, 1e6, -600.0])), np.array([0x7E, 0x7E, 0xFE], np.uint8))


def test_quant_row_worked_by_hand():
    # amax 1: scale 1/448, y = x * 448 = [448, -224, 134.4, 0]; -224 = -1.75 * 2^7 (e 14, m 6);
    # 134.4 = 1.05 * 2^7 rounds to 128 (m 0); so the bytes are 7e, f6, 70, 00
    codes, scale = O.quant_fp8_rows(np.array([[1.0, -0.5, 0.3, 0.0]]))
    assert codes.tolist() == [[0x7E, 0xF6, 0x70, 0x00]]
    assert scale[0] == np.float32(1.0) / np.float32(448.0)
    np.testing.assert_allclose(O.dequant_fp8_rows(codes, scale)[0], [1.0, -0.5, 128 / 448, 0.0], rtol=1e-6)


def test_quant_rows_invariants_and_error_bound():
    x = synth.normal((400, 128), 962).astype(np.float64)
    x[:50] *= 1e-3
    x[50:60] *= 1e3
    codes, scale = O.quant_fp8_rows(x)
    v = O.e4m3_value(codes)
    assert np.all(np.max(np.abs(v), axis=1) == 448.0)      # each row's largest element lands on 448
    x32 = x.astype(np.float32).astype(np.float64)
    y = x32 / scale.astype(np.float64)[:, None]
    err = np.abs(v * scale[:, None].astype(np.float64) - x32)
    normal = np.abs(y) >= 2.0 ** -6
    # a 3-bit mantissa: half a step is 2^-4 relative in the normal range, 2^-10 scale units below it
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x32[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * scale[:, None].astype(np.float64).repeat(128, 1)[~normal] * (1 + 1e-6))
    # power-of-two scaling moves only the scale
    c2, s2 = O.quant_fp8_rows(x * 2.0 ** 7)
    assert np.array_equal(c2, codes) and np.array_equal(s2, (scale * np.float32(2.0 ** 7)).astype(np.float32))
    # an all-zero row: scale 0, value 0 everywhere
    cz, sz = O.quant_fp8_rows(np.zeros((2, 16)))
    assert np.all(sz == 0) and np.all(O.e4m3_value(cz) == 0)


@pytest.mark.parametrize("n", [16, 64])
def test_fp8_decode_close_to_the_unquantised_one(n):
    # attention over E4M3 rows stays near attention over the exact rows (a sanity bound, not parity)
    Hkv, d = 2, 64
    k = synth.normal((n, Hkv, d), 963).astype(np.float64)
    v = synth.normal((n, Hkv, d), 964).astype(np.float64)
    q = synth.normal((2 * Hkv, d), 965).astype(np.float64)
    kd = O.dequant_fp8_rows(*O.quant_fp8_rows(k))
    vd = O.dequant_fp8_rows(*O.quant_fp8_rows(v))
    exact = O.decode_attention(q, lambda j: k[j], lambda j: v[j], n, 0, 0, Hkv)
    coded = O.decode_attention(q, lambda j: kd[j], lambda j: vd[j], n, 0, 0, Hkv)
    assert np.max(np.abs(coded - exact)) <= 0.1
    assert np.max(np.abs(coded - exact)) > 0
