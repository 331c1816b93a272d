"""Pins of the oracle's int8 key variants: the orthonormal Walsh-Hadamard
transform, Hadamard-rotated int8 rows and their re-rotation, and the
keep-scale-unless-overflow re-rotation.

Each pin is something other than the oracle's own formula: a library routine
(scipy's Sylvester Hadamard matrix), closed forms, invariants, the error bounds
[DYN] ("Measured on this branch", the rotation against writing at the new
factor) states for its int8 and int8 + Hadamard paths, and engineered rows
whose outcome is known by construction.
"""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth


def _cfg(s, r=64, d=128, neox=True):
    return O.RopeCfg(head_dim=d, rotary_dim=r, rope_theta=5e5, yarn_factor=s, orig_max_pos=262144, neox=neox)


# ------------------------------------------------------------------ Hadamard transform

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 128, 256])
def test_hadamard_matches_sylvester_matrix(n):
    x = synth.normal((7, n), 900 + n).astype(np.float64)
    want = x @ (scipy.linalg.hadamard(n).T / math.sqrt(n))
    assert np.max(np.abs(O.hadamard(x) - want)) <= 1e-12


def test_hadamard_closed_form_entries_and_involution():
    n = 128
    eye = np.eye(n)
    h = O.hadamard(eye)  # row j = H e_j (H is symmetric)
    i = np.arange(n)
    pop = np.array([[bin(a & b).count("1") for b in i] for a in i])
    assert np.max(np.abs(h - ((-1.0) ** pop) / math.sqrt(n))) <= 1e-15
    assert np.allclose(h[0], 1.0 / math.sqrt(n), atol=0, rtol=1e-15)
    x = synth.normal((5, n), 901).astype(np.float64)
    assert np.max(np.abs(O.hadamard(O.hadamard(x)) - x)) <= 1e-14
    # orthonormal: norms and dot products survive, so attention scores can be taken in the H domain
    hx = O.hadamard(x)
    assert np.allclose(np.linalg.norm(hx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert abs(float(hx[0] @ hx[1]) - float(x[0] @ x[1])) <= 1e-12
    with pytest.raises(ValueError):
        O.hadamard(np.zeros(96))


# ------------------------------------------------------------------ error bounds against the truth

def _turn_stats(turned, written, truth, step):
    """RMS(turned - truth) / RMS(written - truth) and the worst element of turned - truth in steps."""
    et = turned - truth
    ew = written - truth
    ratio = float(np.sqrt(np.mean(et * et)) / np.sqrt(np.mean(ew * ew)))
    worst = float(np.max(np.abs(et) / step))
    return ratio, worst


@pytest.mark.parametrize("fa,fb", [(1.0, 2.0), (1.5, 2.0), (2.0, 1.0), (1.0, 1.125)])
def test_hadamard_rerotation_within_pages_bounds(fa, fb):
    # raw keys at positions on both sides of the trained 262,144, rotated at A and at B in fp64;
    # A's rows stored as int8 of H k, turned to B, compared with the fp64 key at B (in the H domain)
    ca, cb = _cfg(fa), _cfg(fb)
    n = 3000
    pos = synth.uniform_ints(n, 0, 520000, 910)
    raw = synth.normal((n, 128), 911).astype(np.float64)
    ka = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(ca)), 64, True, O.mscale(ca))
    kb = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(cb)), 64, True, O.mscale(cb))
    codes_a, sa = O.quant_int8_hadamard_rows(ka)
    codes_t, st = O.rerotate_int8_hadamard_rows(codes_a, sa, pos, ca, cb)
    codes_b, sb = O.quant_int8_hadamard_rows(kb)
    truth = O.hadamard(kb)
    ratio, worst = _turn_stats(O.dequant_int8_rows(codes_t, st), O.dequant_int8_rows(codes_b, sb), truth,
                               sb.astype(np.float64)[:, None])
    # [DYN] reports 1.39x - 1.42x and at most 1.95 steps; its bounds are 1.6x RMS and 3 steps
    assert ratio <= 1.6 and worst <= 3.0, (ratio, worst)
    # and the turn matters: the unturned A rows miss B by far more
    ratio_a, _ = _turn_stats(O.dequant_int8_rows(codes_a, sa), O.dequant_int8_rows(codes_b, sb), truth,
                             sb.astype(np.float64)[:, None])
    assert ratio_a > 10


# ------------------------------------------------------------------ the plain per-row quantiser

@pytest.mark.parametrize("kind", ["f64", "f32", "bf16"])
def test_int8_codes_are_the_nearest_multiples_of_the_row_scale(kind):
    # brute force over every code: each code c minimises |x - c * scale| for the stored scale,
    # except where two codes are within float32 rounding of a tie (then it is one of those two)
    rng = synth.rng(930)
    x = rng.standard_normal((200, 128)) * rng.uniform(1e-3, 1e3, (200, 1))
    if kind == "f32":
        x = x.astype(np.float32).astype(np.float64)
    elif kind == "bf16":
        x = O.round_bf16(x)
    codes, scale = O.quant_int8_rows(x)
    s = scale.astype(np.float64)
    assert np.all(np.max(np.abs(codes.astype(np.int32)), axis=1) == 127)
    cand = np.arange(-127, 128, dtype=np.float64)
    dist = np.abs(x[..., None] - cand * s[:, None, None])  # [rows, d, 255]
    order = np.sort(dist, axis=-1)
    best = cand[np.argmin(dist, axis=-1)]
    near_tie = (order[..., 1] - order[..., 0]) <= 4 * 2.0 ** -24 * 127 * s[:, None]
    assert np.array_equal(codes[~near_tie], best[~near_tie].astype(np.int8))
    got_dist = np.abs(x - codes * s[:, None])
    assert np.all(got_dist[near_tie] <= order[..., 0][near_tie] + 4 * 2.0 ** -24 * 127 * s[:, None].repeat(128, 1)[near_tie])
    # scale: the largest entry reconstructs to within the float32 rounding of the stored scale
    amax = np.max(np.abs(x), axis=1)
    assert np.all(np.abs(127 * s - amax) <= amax * 2.0 ** -23)


def test_int8_quantiser_ties_go_to_even():
    # row max 127 makes the scale exactly 1, so the quotients are exact half-integers
    row = np.array([[127.0, 63.5, -0.5, 1.5, 2.5, -3.5, 0.49, -126.5]])
    codes, scale = O.quant_int8_rows(row)
    assert scale[0] == np.float32(1.0)
    assert codes[0].tolist() == [127, 64, 0, 2, 2, -4, 0, -126]


# ------------------------------------------------------------------ plain int8 re-rotation

@pytest.mark.parametrize("fa,fb", [(1.0, 2.0), (1.5, 2.0), (2.0, 1.0), (1.0, 1.125)])
def test_int8_rerotation_within_pages_bounds(fa, fb):
    # per-row int8 keys written at A, dequantised, turned to B and requantised, against the fp64 key
    # at B; [DYN] "Measured on this branch" reports 1.33x - 1.36x RMS and at most 1.17 steps for its
    # int8 path and states the bounds 1.6x RMS and 2 steps
    ca, cb = _cfg(fa), _cfg(fb)
    n = 3000
    pos = synth.uniform_ints(n, 0, 520000, 940)
    raw = synth.normal((n, 128), 941).astype(np.float64)
    ka = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(ca)), 64, True, O.mscale(ca))
    kb = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(cb)), 64, True, O.mscale(cb))
    codes_a, sa = O.quant_int8_rows(ka)
    codes_t, st = O.rerotate_int8_rows(codes_a, sa, pos, ca, cb)
    codes_b, sb = O.quant_int8_rows(kb)
    step = sb.astype(np.float64)[:, None]
    ratio, worst = _turn_stats(O.dequant_int8_rows(codes_t, st), O.dequant_int8_rows(codes_b, sb), kb, step)
    assert ratio <= 1.6 and worst <= 2.0, (ratio, worst)
    # negative controls: rows left at A, or turned the wrong way, miss B by far more
    ratio_a, _ = _turn_stats(O.dequant_int8_rows(codes_a, sa), O.dequant_int8_rows(codes_b, sb), kb, step)
    codes_w, sw = O.rerotate_int8_rows(codes_a, sa, pos, cb, ca)
    ratio_w, _ = _turn_stats(O.dequant_int8_rows(codes_w, sw), O.dequant_int8_rows(codes_b, sb), kb, step)
    assert ratio_a > 10 and ratio_w > 10, (ratio_a, ratio_w)


def test_int8_rerotation_a_to_a_is_identity():
    # a turn by zero angles with gain 1 must return the quantiser's rows bit for bit: the row max
    # is 127 codes, so the new scale is max|c s| / 127 = s and every quotient c s / s = c
    c = _cfg(1.375)
    pos = synth.uniform_ints(500, 0, 520000, 950)
    raw = synth.normal((500, 128), 951).astype(np.float64)
    k = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(c)), 64, True, O.mscale(c))
    codes, s = O.quant_int8_rows(k)
    codes[7] = 0
    s[7] = 0.0
    codes2, s2 = O.rerotate_int8_rows(codes, s, pos, c, c)
    assert np.array_equal(codes2, codes) and np.array_equal(s2, s)


@pytest.mark.parametrize("neox,r", [(True, 64), (False, 64), (False, 48)])
def test_hadamard_turn_of_leading_half_by_half_transforms(neox, r):
    # The half-row form a kernel may use when the turn R moves only dims < 64 of a 128-dim row:
    # with the unnormalised Sylvester H of order 128, H R H c = 128 c + [H64 D; H64 D],
    # D = (R - I) H64 (c_lo + c_hi).  Checked in fp64 against the oracle's orthonormal transform
    # (H = sqrt(n) * O.hadamard) and a direct turn of the pairs.
    rng = synth.rng(2200 + r + neox)
    c = rng.integers(-127, 128, size=(9, 128)).astype(np.float64)
    ang = rng.uniform(-4.0, 4.0, size=(9, r // 2))
    g = 1.07
    cs, sn = g * np.cos(ang), g * np.sin(ang)

    def turn(x):
        y = np.array(x, copy=True)
        for i in range(r // 2):
            a, b = (i, i + r // 2) if neox else (2 * i, 2 * i + 1)
            y[:, a] = x[:, a] * cs[:, i] - x[:, b] * sn[:, i]
            y[:, b] = x[:, b] * cs[:, i] + x[:, a] * sn[:, i]
        return y

    h128 = lambda x: O.hadamard(x) * math.sqrt(128)
    h64 = lambda x: O.hadamard(x) * 8.0
    full = h128(turn(h128(c)))
    x = np.zeros_like(c)
    x[:, :64] = h64(c[:, :64] + c[:, 64:])
    dd = (turn(x) - x)[:, :64]
    assert np.all(dd[:, r:] == 0)  # dims past r do not move
    h = h64(dd)
    half = 128 * c + np.concatenate([h, h], axis=1)
    np.testing.assert_allclose(half, full, rtol=0, atol=1e-9 * np.max(np.abs(full)))


def test_hadamard_rerotation_identity_turn():
    c = _cfg(1.5)
    pos = synth.uniform_ints(200, 0, 500000, 920)
    k = synth.normal((200, 128), 921).astype(np.float64)
    codes, s = O.quant_int8_hadamard_rows(k)
    codes2, s2 = O.rerotate_int8_hadamard_rows(codes, s, pos, c, c)
    assert np.array_equal(codes2, codes)
    np.testing.assert_allclose(s2, s, rtol=2.0 ** -23, atol=0)


def test_hadamard_storage_keeps_scores():
    # scores against a Hadamard-stored key equal scores of the H-transformed query against H k
    k = synth.normal((50, 128), 925).astype(np.float64)
    q = synth.normal((128,), 926).astype(np.float64)
    codes, s = O.quant_int8_hadamard_rows(k)
    hk = O.dequant_int8_rows(codes, s)
    got = hk @ O.hadamard(q)
    want = O.hadamard(hk) @ q  # the key the codes stand for, back in the plain domain
    assert np.max(np.abs(got - want)) <= 1e-12


# ------------------------------------------------------------------ keep the scale unless a code overflows

@pytest.mark.parametrize("fa,fb", [(1.0, 2.0), (1.5, 2.0), (2.0, 1.0), (1.0, 1.125)])
def test_keep_scale_tail_bitwise_and_bounds(fa, fb):
    ca, cb = _cfg(fa), _cfg(fb)
    n = 3000
    pos = synth.uniform_ints(n, 0, 520000, 930)
    raw = synth.normal((n, 128), 931).astype(np.float64)
    ka = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(ca)), 64, True, O.mscale(ca))
    kb = O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(cb)), 64, True, O.mscale(cb))
    codes_a, sa = O.quant_int8_rows(ka)
    codes_t, st, over = O.rerotate_int8_keep_scale_rows(codes_a, sa, pos, ca, cb)
    keep = ~over
    # the pages' observation: past the rotary slice, codes and scales are what was written
    assert np.array_equal(codes_t[keep, 64:], codes_a[keep, 64:])
    assert np.array_equal(st[keep], sa[keep])
    # rows that overflowed are the whole-row requantisation of the turned row
    full_codes, full_scale = O.quant_int8_rows(O.rerotate_rows(O.dequant_int8_rows(codes_a, sa), pos, ca, cb))
    assert np.array_equal(codes_t[over], full_codes[over]) and np.array_equal(st[over], full_scale[over])
    # a gain mscale_B / mscale_A > 1 grows the rotary slice: some rows must overflow then
    if O.mscale(cb) / O.mscale(ca) > 1.0:
        assert over.any()
    # error against the fp64 key at B, rotary dims, in B's steps (written at B = the yardstick)
    codes_b, sb = O.quant_int8_rows(kb)
    ratio, worst = _turn_stats(O.dequant_int8_rows(codes_t, st)[:, :64], O.dequant_int8_rows(codes_b, sb)[:, :64],
                               kb[:, :64], st.astype(np.float64)[:, None])
    # [DYN] reports 1.33x - 1.36x and at most 1.17 steps for int8; its bounds are 1.6x RMS and 2 steps
    assert ratio <= 1.6 and worst <= 2.0, (ratio, worst)


def test_keep_scale_identity_and_engineered_overflow():
    c = _cfg(1.0)
    pos = synth.uniform_ints(300, 0, 500000, 940)
    k = synth.normal((300, 128), 941).astype(np.float64)
    codes, s = O.quant_int8_rows(k)
    codes2, s2, over = O.rerotate_int8_keep_scale_rows(codes, s, pos, c, c)
    assert not over.any() and np.array_equal(codes2, codes) and np.array_equal(s2, s)
    # at position 0 every angle is 0 and the turn is the gain mscale(8) / mscale(1) = 0.1 ln 8 + 1
    ca, cb = _cfg(1.0), _cfg(8.0)
    gain = 0.1 * math.log(8.0) + 1.0
    rng = synth.rng(942)
    row_keep = rng.uniform(-0.8, 0.8, 128)
    row_keep[100] = 1.0           # the row's largest value sits in the tail: codes <= 102, x gain < 127
    row_over = rng.uniform(-0.5, 0.5, 128)
    row_over[5] = 1.0             # the largest value is rotary: 127 x gain = 153 overflows
    q, sc = O.quant_int8_rows(np.stack([row_keep, row_over]))
    qt, st, over = O.rerotate_int8_keep_scale_rows(q, sc, np.array([0, 0]), ca, cb)
    assert over.tolist() == [False, True]
    assert np.array_equal(qt[0, 64:], q[0, 64:]) and st[0] == sc[0]
    assert np.max(np.abs(qt[0, :64] - q[0, :64].astype(np.float64) * gain)) <= 0.5 + 1e-4
    # the overflowing row is requantised whole: its rotary maximum is 127 again, the scale grew by the gain
    assert int(np.max(np.abs(qt[1, :64]))) == 127
    assert abs(float(st[1]) / float(sc[1]) - gain) <= 1e-6
