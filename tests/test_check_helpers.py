"""The GPU tests' comparison helpers, pinned on the CPU: each accepts what it must accept and
rejects a planted mistake one unit beyond its bound (no GPU, no kernel involved)."""
import numpy as np
import pytest
import torch

from oracle import ropekv_oracle as O
from tests.gpu_util import (assert_bf16_attention, assert_bf16_close, assert_bf16_rounded, assert_f16_rounded, assert_fp8_codes_valid,
                            assert_int8_codes_valid, assert_rounded_once, decode_e4m3, decode_int8, excess, oracle_written)


def _bf16(x):
    """round to nearest bf16 (torch's conversion), back to fp64"""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _bf16_step(x, away):
    """the bf16 neighbour of bf16 values x one step toward (away=False) or away from zero"""
    b = torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16)
    return (b + (1 if away else -1)).view(torch.bfloat16).double().numpy()


def test_bf16_rounded_accepts_round_to_nearest_and_rejects_one_step():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((6, 128)) * np.exp(rng.uniform(-6, 6, (6, 1)))
    got = _bf16(ref)
    assert_bf16_rounded(got, ref)
    # the fp32 result of a short computation, then one rounding: still within the bound
    assert_bf16_rounded(_bf16((ref * (1 + 3e-7)).astype(np.float32)), ref)
    _, ex = np.frexp(got)
    ulp = np.ldexp(1.0, ex - 8)
    # elements whose exact value is at most 0.4 ulp from the rounded one: either neighbour fails
    picks = np.argwhere((np.abs(got - ref) < 0.4 * ulp) & (np.abs(got) > 0))[:6]
    assert len(picks) == 6
    for i, j in picks:
        for away in (False, True):
            bad = got.copy()
            bad[i, j] = _bf16_step(got[i, j], away)
            with pytest.raises(AssertionError):
                assert_bf16_rounded(bad, ref)


def test_f16_rounded_accepts_round_to_nearest_and_rejects_one_step():
    rng = np.random.default_rng(8)
    # magnitudes from the subnormal range (below 2^-14) to 2^11
    ref = rng.standard_normal((6, 128)) * np.exp(rng.uniform(-12, 7, (6, 1)))
    ref[0, :4] = [3e-8, -2e-6, 5.9e-5, 0.0]
    got = ref.astype(np.float16).astype(np.float64)
    assert_f16_rounded(got, ref, rel_fp32=0.0)
    assert_f16_rounded((ref * (1 + 3e-7)).astype(np.float32).astype(np.float16).astype(np.float64), ref)
    bits = got.astype(np.float16).view(np.int16)
    ulp = np.abs((bits + 1).view(np.float16).astype(np.float64) - got)
    picks = np.argwhere((np.abs(got - ref) < 0.4 * ulp) & (np.abs(got) > 0))
    picks = np.concatenate([picks[:5], [[0, 1]]])  # one subnormal among them
    for i, j in picks:
        for step in (1, -1):
            bad = got.copy()
            bad[i, j] = (bits[i, j:j + 1] + step).view(np.float16).astype(np.float64)[0]
            with pytest.raises(AssertionError):
                assert_f16_rounded(bad, ref, rel_fp32=0.0)
    # fp32 results: the dtype switch holds them to rel_fp32 of the row's largest value
    assert_rounded_once(ref.astype(np.float32).astype(np.float64), ref, "f32")
    bad = ref.copy()
    bad[2, 5] += 2e-6 * np.max(np.abs(ref[2]))
    with pytest.raises(AssertionError):
        assert_rounded_once(bad, ref, "f32")


def test_bf16_close_bound_and_signed_excess():
    ref = np.array([[0.0, 1.0, -2.0, 10.0]])
    ok = ref + np.array([[0.0199, 0.0299, -0.0399, 0.1199]])  # just inside atol 2e-2 + rtol 1e-2 |ref|
    assert_bf16_close(ok, ref)
    assert -2e-4 < excess(ok, ref) < 0
    bad = ok.copy()
    bad[0, 3] += 1e-3
    with pytest.raises(AssertionError):
        assert_bf16_close(bad, ref)
    assert excess(bad, ref) > 0
    assert excess(ref, ref) < 0  # the margin is reported signed


def test_int8_validity_accepts_edge_flips_only():
    want = np.array([3, -7, 10, 0], dtype=np.int8)
    quot = np.array([3.4996, -6.5004, 10.2, 0.0])  # two quotients sit within 5e-4 of an edge
    got = want.copy()
    got[0] = 4  # 3.4996 is 4e-4 from the 3 / 4 edge
    got[1] = -6  # -6.5004 is 4e-4 from the -7 / -6 edge
    assert assert_int8_codes_valid(got, want, quot, 1e-3) == 2
    with pytest.raises(AssertionError):  # the same flips need more than a 1e-4 margin
        assert_int8_codes_valid(got, want, quot, 1e-4)
    far = want.copy()
    far[2] = 11  # 10.2 is 0.3 from the 10 / 11 edge
    with pytest.raises(AssertionError):
        assert_int8_codes_valid(far, want, quot, 1e-3)
    two = want.copy()
    two[3] = 2  # two steps
    with pytest.raises(AssertionError):
        assert_int8_codes_valid(two, want, quot, 1e-3)


def test_fp8_validity_accepts_neighbour_at_midpoint_only():
    # E4M3 values 1.0 and 1.125 are neighbours (bytes 0x38, 0x39); their midpoint is 1.0625
    want = np.array([0x38, 0x38], dtype=np.uint8).view(np.int8)
    got = np.array([0x39, 0x38], dtype=np.uint8).view(np.int8)
    assert O.e4m3_value(np.array([0x38], dtype=np.uint8).view(np.int8))[0] == 1.0
    assert assert_fp8_codes_valid(got, want, np.array([1.0624, 1.0]), 1e-3) == 1
    with pytest.raises(AssertionError):
        assert_fp8_codes_valid(got, want, np.array([1.05, 1.0]), 1e-3)
    skip = np.array([0x3A, 0x38], dtype=np.uint8).view(np.int8)  # two steps (1.25)
    with pytest.raises(AssertionError):
        assert_fp8_codes_valid(skip, want, np.array([1.0624, 1.0]), 1e-3)


def test_host_decoders_agree_with_the_oracle_storage():
    # decode_e4m3 (torch's float8_e4m3fn) and the oracle's E4M3 table agree on every byte but the two
    # NaNs; decode_int8 is codes x the row scale
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(decode_e4m3(codes), O.e4m3_value(codes))
    assert decode_e4m3(np.array([0x7E], dtype=np.uint8))[0] == 448.0
    c = np.array([[127, -3, 0], [1, 2, -127]], dtype=np.int8)
    assert np.array_equal(decode_int8(c, np.array([0.5, 0.25], dtype=np.float32)),
                          [[63.5, -1.5, 0.0], [0.25, 0.5, -31.75]])


def test_oracle_written_is_one_storage_rounding():
    rng = np.random.default_rng(11)
    key = rng.standard_normal((5, 4, 128))
    vals, unit = oracle_written("f16", key)
    assert np.all(np.abs(vals - key) <= unit / 2)  # one fp16 rounding, at most half the row max's ulp
    assert np.array_equal(vals, key.astype(np.float16).astype(np.float64))
    vals, unit = oracle_written("i8", key)
    assert np.all(np.abs(vals - key) <= unit / 2 * (1 + 1e-6)) and np.all(unit[..., 0] > 0)
    assert np.allclose(np.max(np.abs(vals), axis=-1), 127 * unit[..., 0])  # the row max takes code 127
    hv, hunit = oracle_written("i8_hadamard", key)  # H domain: within half a step of H key
    assert np.all(np.abs(hv - O.hadamard(key)) <= hunit / 2 * (1 + 1e-6))
    assert not np.allclose(hv, vals)


def _attention_with_rounded_weights(q, K, V, Hkv, sign=None):
    """q [Hq, d], K, V [n, Hkv, d]: softmax weights rounded to bf16 one by one (or, with sign, moved
    by a full 2^-8 each in the direction sign), fp64 sums, the result rounded to bf16: the roundings
    a bf16 attention kernel makes, written out for one small case."""
    Hq, d = q.shape
    out = np.empty((Hq, d))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = K[:, g, :] @ q[h] / np.sqrt(d)
        p = np.exp(s - s.max())
        if sign is None:
            pr = _bf16(p)
            out[h] = (pr @ V[:, g, :]) / pr.sum()
        else:  # worst case per output dim: each weight pushed 2^-8 toward that dim's outliers
            for c in range(d):
                o = (p @ V[:, g, c]) / p.sum()
                pr = p * (1 + 2.0 ** -8 * np.sign(V[:, g, c] - o))
                out[h, c] = (pr @ V[:, g, c]) / pr.sum()
    return _bf16(out)


@pytest.mark.parametrize("worst", [False, True])
def test_bf16_attention_bound_holds_for_rounded_weights_and_catches_a_dropped_key(worst):
    rng = np.random.default_rng(11)
    n, Hkv, Hq, d = 120, 2, 8, 64
    q = _bf16(rng.standard_normal((Hq, d)))
    K = _bf16(rng.standard_normal((n, Hkv, d)))
    V = _bf16(rng.standard_normal((n, Hkv, d)))
    ref = O.decode_attention(q, lambda j: K[j], lambda j: V[j], n, 0, 0, Hkv)
    ref_abs = O.decode_attention(q, lambda j: K[j], lambda j: np.abs(V[j]), n, 0, 0, Hkv)
    got = _attention_with_rounded_weights(q, K, V, Hkv, sign=True if worst else None)
    assert_bf16_attention(got, ref, ref_abs)
    # each key's largest effect on an output: w_hj |v_j - out_h| over heads and dims
    eff = np.zeros(n)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = K[:, g, :] @ q[h] / np.sqrt(d)
        w = np.exp(s - s.max())
        w /= w.sum()
        eff = np.maximum(eff, np.max(w[:, None] * np.abs(V[:, g, :] - ref[h]), axis=1))
    # a key whose loss moves some output by 0.006-0.017: inside 2e-2 + 1e-2 |ref|, well outside the
    # rounding bound (~0.0035 here)
    j = int(np.argmin(np.abs(eff - 0.012)))
    assert 0.006 < eff[j] < 0.017
    keep = np.r_[0:j, j + 1:n]
    dropped = _attention_with_rounded_weights(q, K[keep], V[keep], Hkv)
    assert_bf16_close(dropped, ref)
    with pytest.raises(AssertionError):
        assert_bf16_attention(dropped, ref, ref_abs)
