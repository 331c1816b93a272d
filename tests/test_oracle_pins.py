"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it checks.  None of these re-types the oracle's
own formula: they compare with printed numbers, closed forms, invariants,
brute force over small cases, or a second formulation of the same rule.
"""
import math

import numpy as np
import pytest

from oracle import ropekv_oracle as O
from tests.conftest import read_golden

GOLD = read_golden("rope_worked_numbers.txt")
RNG = np.random.default_rng(20260)


def _f(key):
    return [float(x) for x in GOLD[key].split()]


# ---------------------------------------------------------------- frequencies


def test_omega16_worked_number():
    # "A worked number": pair 16 at b = 1e4, r = 128 turns 0.1 rad per token.
    w = O.plain_inv_freq(128, 1e4)
    assert abs(w[16] - _f("omega16")[0]) < 1e-15
    # wavelength 62.8 tokens
    assert abs(2 * math.pi / w[16] - 62.8) < 0.05


def test_score_shift_5_3_vs_105_103():
    # q(16) = k(16) = (1, 0): the score at (5, 3) and at (105, 103) both equal cos(0.2).
    cfg = O.RopeCfg(head_dim=128, rotary_dim=128, rope_theta=1e4)
    table = O.build_table(cfg, 200)
    q = np.zeros((1, 128))
    k = np.zeros((1, 128))
    q[0, 16] = 1.0  # NeoX pair 16 = (16, 80)
    k[0, 16] = 1.0
    s1 = (O.rope_apply(q, [5], table, 128, True) * O.rope_apply(k, [3], table, 128, True)).sum()
    s2 = (O.rope_apply(q, [105], table, 128, True) * O.rope_apply(k, [103], table, 128, True)).sum()
    want = _f("score_5_3")[0]
    assert abs(s1 - want) < 5e-8 and abs(s2 - want) < 5e-8
    assert abs(s1 - s2) < 1e-14
    # the rotated vectors themselves moved
    assert np.abs(O.rope_apply(q, [5], table, 128, True) - O.rope_apply(q, [105], table, 128, True)).max() > 0.5


@pytest.mark.parametrize("key,r,b,L0", [("band_128_1e4_4096", 128, 1e4, 4096),
                                        ("band_128_5e5_4096", 128, 5e5, 4096),
                                        ("band_128_5e5_8192", 128, 5e5, 8192)])
def test_yarn_bands(key, r, b, L0):
    low, high = O.yarn_correction_range(32, 1, r, b, L0)
    assert [low, high] == [int(x) for x in GOLD[key].split()]


def test_yarn_rotation_counts_at_band_edges():
    # pairs 20 / 21 / 45 / 46 turn 36.66 / 31.75 / 1.00 / 0.87 times within L0 = 4096.
    w = O.plain_inv_freq(128, 1e4)
    got = [4096 * w[i] / (2 * math.pi) for i in (20, 21, 45, 46)]
    for g, want in zip(got, _f("rotations_20_21_45_46")):
        assert abs(g - want) < 0.006


def test_yarn_blend_direction():
    # "YaRN, precisely": pairs 0-20 keep their frequency, 46-63 are divided by s,
    # 21-45 lie strictly between (r=128, b=1e4, L0=4096).
    s = 8.0
    cfg = O.RopeCfg(head_dim=128, rotary_dim=128, rope_theta=1e4, yarn_factor=s, orig_max_pos=4096)
    w = O.inv_freq(cfg)
    base = O.plain_inv_freq(128, 1e4)
    np.testing.assert_array_equal(w[:21], base[:21])
    np.testing.assert_allclose(w[46:], base[46:] / s, rtol=1e-15)
    mid = w[21:46] / base[21:46]
    assert np.all(mid < 1.0) and np.all(mid > 1.0 / s)
    assert np.all(np.diff(mid) < 0)  # the interpolated share grows monotonically with i


def test_mscale_s8():
    assert abs(O.yarn_mscale(8.0) - _f("mscale_8")[0]) < 5e-5
    assert abs(O.yarn_mscale(8.0) ** 2 - _f("mscale_sq_8")[0]) < 5e-4
    assert O.yarn_mscale(1.0) == 1.0 and O.yarn_mscale(0.5) == 1.0


def test_pair63_wavelength():
    w = O.plain_inv_freq(128, 5e5)
    wl = 2 * math.pi / w[63]
    assert abs(wl / _f("pair63_wavelength")[0] - 1) < 0.005
    assert abs(8192 / wl - _f("pair63_revolutions_8192")[0]) < 0.00005


def test_factor_one_is_plain_rope():
    # s = 1 gives the unscaled table exactly ("--rope-scaling dynamic": a short dialog keeps the trained angles).
    a = O.build_table(O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=1024), 3000)
    b = O.build_table(O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=5e5), 3000)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- table


@pytest.mark.parametrize("s", [1.0, 1.125, 2.0, 8.0])
def test_table_group_law(s):
    # Rows are mu * (cos, sin) of m*w: row 0 is (mu, 0), |row|^2 = mu^2, and
    # R(m)R(1) = R(m+1) (angle addition) holds row to row.
    cfg = O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=5e5, yarn_factor=s, orig_max_pos=1024)
    T = O.build_table(cfg, 4096)
    mu = O.mscale(cfg)
    h = 32
    c, sn = T[:, :h] / mu, T[:, h:] / mu
    np.testing.assert_allclose(T[0, :h], mu, rtol=0, atol=0)
    np.testing.assert_allclose(T[0, h:], 0.0, atol=0)
    np.testing.assert_allclose(c * c + sn * sn, 1.0, atol=1e-14)
    c1, s1 = c[1], sn[1]
    nxt_c = c[:-1] * c1 - sn[:-1] * s1
    nxt_s = sn[:-1] * c1 + c[:-1] * s1
    np.testing.assert_allclose(nxt_c, c[1:], atol=2e-12)
    np.testing.assert_allclose(nxt_s, sn[1:], atol=2e-12)
    # column i turns at the pair's own frequency: the angle from atan2 grows by w_i per step
    ang = np.unwrap(np.arctan2(sn[:64, 5], c[:64, 5]))
    np.testing.assert_allclose(np.diff(ang), O.inv_freq(cfg)[5], rtol=1e-9)


# ---------------------------------------------------------------- rotation


def test_relative_property_random():
    # "Why the dot product only sees m - n": q.k after rotation depends only on m - n.
    cfg = O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=1e4)
    T = O.build_table(cfg, 5000)
    q = RNG.standard_normal((1, 64))
    k = RNG.standard_normal((1, 64))
    for neox in (True, False):
        ref = None
        for m in (7, 107, 1007, 4007):
            n = m - 5
            s = (O.rope_apply(q, [m], T, 64, neox) * O.rope_apply(k, [n], T, 64, neox)).sum()
            ref = s if ref is None else ref
            assert abs(s - ref) < 1e-12


def test_neox_vs_gptj_permutation():
    # Same mathematics, different memory layout: permuting dims maps one pairing onto the other.
    cfg = O.RopeCfg(head_dim=48, rotary_dim=32, rope_theta=1e4)
    T = O.build_table(cfg, 100)
    x = RNG.standard_normal((6, 48))
    pos = np.array([0, 1, 5, 17, 63, 99])
    perm = np.arange(48)
    perm[:32] = np.stack([np.arange(16), np.arange(16) + 16], axis=1).reshape(-1)  # gptj slot -> neox dim
    y_neox = O.rope_apply(x, pos, T, 32, True)
    y_gptj = O.rope_apply(x[:, perm], pos, T, 32, False)
    np.testing.assert_allclose(y_gptj, y_neox[:, perm], atol=1e-15)


def test_tail_unchanged_and_norm():
    cfg = O.RopeCfg(head_dim=128, rotary_dim=64, rope_theta=5e5)
    T = O.build_table(cfg, 1000)
    x = RNG.standard_normal((10, 3, 128))
    pos = RNG.integers(0, 1000, 10)
    y = O.rope_apply(x, pos, T, 64, True)
    np.testing.assert_array_equal(y[..., 64:], x[..., 64:])
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_group_law_twice_rotation():
    # R(a) R(c) = R(a + c): rotating by a then c equals rotating by a + c.
    cfg = O.RopeCfg(head_dim=32, rotary_dim=32, rope_theta=1e4)
    T = O.build_table(cfg, 300)
    x = RNG.standard_normal((4, 32))
    a = np.array([3, 10, 50, 100])
    c = np.array([7, 90, 149, 199])
    two = O.rope_apply(O.rope_apply(x, a, T, 32, True), c, T, 32, True)
    one = O.rope_apply(x, a + c, T, 32, True)
    np.testing.assert_allclose(two, one, atol=1e-12)


# ---------------------------------------------------------------- visible set


def test_visible_table_c6_s2_t10():
    gold = read_golden("sink_visible_c6_s2_t10.txt")
    C, S = 6, 2
    for i in range(10):
        want = [int(x) for x in gold[str(i)].split()]
        assert O.visible_positions(i, S, C - S) == want
    counts = [len(O.visible_positions(i, S, C - S)) for i in range(10)]
    assert counts == [1, 2, 3, 4, 5, 6, 6, 6, 6, 6]
    assert O.visible_positions(9, S, C - S) == [0, 1, 6, 7, 8, 9]


def _two_branch_visible(position, capacity, sinks):
    # The capacity form: all of 0..p while p < C, else S sinks and the last C - S positions.
    if position < capacity:
        return list(range(position + 1))
    start = max(sinks, position - (capacity - sinks) + 1)
    return list(range(sinks)) + list(range(start, position + 1))


def test_visible_predicate_equals_capacity_form_bruteforce():
    for C in range(1, 20):
        for S in range(0, C):
            for p in range(60):
                assert O.visible_positions(p, S, C - S) == _two_branch_visible(p, C, S), (C, S, p)


def test_visible_full_attention():
    assert O.visible_positions(5, 4, 0) == list(range(6))


# ---------------------------------------------------------------- ring buffer


def test_ring_rollover_order():
    # window 3 (no sinks), seven single-token appends carrying payloads 1..7: read-out [5, 6, 7].
    ring = O.RingSeq(sinks=0, window=3)
    payload = {}
    for t in range(7):
        kept = ring.append(1)
        for p, s in kept.items():
            payload[s] = p + 1
    assert [payload[s] for s in ring.chronological_slots()] == [5, 6, 7]
    assert ring.count == 3


def test_ring_count_caps_and_first_write_rules():
    # prompt of T >= W: last W kept in order, head 0, count W; T < W: count T, head T % W.
    r = O.RingSeq(sinks=0, window=8)
    kept = r.append(20)
    assert (r.head, r.count) == (0, 8)
    assert sorted(kept) == list(range(12, 20)) and [kept[p] for p in range(12, 20)] == list(range(8))
    r2 = O.RingSeq(sinks=0, window=8)
    r2.append(5)
    assert (r2.head, r2.count) == (5, 5)
    for _ in range(10):
        r2.append(1)
        assert r2.count <= 8
    assert r2.count == 8


@pytest.mark.parametrize("S,W", [(0, 3), (2, 4), (4, 12), (3, 5)])
def test_ring_chunked_equals_token_by_token(S, W):
    rng = np.random.default_rng(S * 31 + W)
    for _ in range(30):
        chunks = list(rng.integers(1, 2 * (S + W) + 3, size=rng.integers(1, 6)))
        a = O.RingSeq(sinks=S, window=W)
        b = O.RingSeq(sinks=S, window=W)
        pa, pb = {}, {}
        for c in chunks:
            for p, s in a.append(int(c)).items():
                pa[s] = p
            for _ in range(int(c)):
                for p, s in b.append(1).items():
                    pb[s] = p
        ra = [pa[s] for s in a.chronological_slots()]
        rb = [pb[s] for s in b.chronological_slots()]
        assert ra == rb
        n = a.seq_len
        # the read-out is exactly the visible set of the next query's predecessor (position n-1)
        assert ra == O.visible_positions(n - 1, S, W)


# ---------------------------------------------------------------- paged


def test_sliding_window_block_bound():
    assert O.sliding_window_max_blocks(4096, 16) == int(GOLD["sliding_blocks_4096"])
    assert O.cdiv(131072, 16) == int(GOLD["full_blocks_131072"])
    # the comment's example: block 4, 4 tokens -> 2 blocks
    assert O.sliding_window_max_blocks(5, 4) == 2


@pytest.mark.parametrize("S,W,bs", [(0, 5, 4), (4, 12, 16), (2, 7, 4), (4, 40, 16), (20, 9, 8)])
def test_paged_freeing_bruteforce(S, W, bs):
    # Replay growth step by step; after each call the nulled blocks are exactly the
    # blocks holding no position visible to the call's first query or any later one.
    rng = np.random.default_rng(S + 7 * W)
    nblk = 40
    table = list(range(nblk))
    n = 0
    freed_all = []
    while n < nblk * bs - 40:
        step = int(rng.integers(1, 12))
        freed = O.paged_free_expired(table, n, S, W, bs)
        freed_all += freed
        assert freed == sorted(freed, reverse=True)
        first_q = n
        needed = set()
        for j in range(first_q + 1):
            if j < S or first_q - j < W:
                needed.add(j // bs)
        for blk in range(nblk):
            if blk * bs >= first_q:
                continue  # not yet written
            if blk in needed:
                assert table[blk] == blk
            else:
                assert table[blk] == -1, (blk, n)
        n += step
    assert len(set(freed_all)) == len(freed_all)


def test_paged_full_attention_never_frees():
    t = list(range(10))
    assert O.paged_free_expired(t, 150, 4, 0, 16) == [] and t == list(range(10))


# ---------------------------------------------------------------- attention


def _sink_experiment(neox):
    # The [SINK] runnable experiment, re-run in the oracle: MHA, fp64, C=6, S=2, T=10, d=8.
    rng = np.random.default_rng(229)
    h, t, d = 2, 10, 8
    cfg = O.RopeCfg(head_dim=d, rotary_dim=d, rope_theta=1e4, neox=neox)
    T = O.build_table(cfg, 64)
    pos = np.arange(t)
    qraw = rng.standard_normal((t, h, d))
    kraw = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    q = O.rope_apply(qraw, pos, T, d, neox)
    k = O.rope_apply(kraw, pos, T, d, neox)
    return q, k, v, T


@pytest.mark.parametrize("neox", [False, True])
def test_incremental_equals_dense_and_differs_from_full(neox):
    q, k, v, _ = _sink_experiment(neox)
    C, S = 6, 2
    for head in range(2):
        dense, mask = O.dense_sink_attention(q[:, head], k[:, head], v[:, head], C, S)
        assert mask.sum(axis=1).tolist() == [1, 2, 3, 4, 5, 6, 6, 6, 6, 6]
        inc = O.prefill_attention(q[:, head:head + 1], lambda j: k[j, head:head + 1], lambda j: v[j, head:head + 1],
                                  0, S, C - S, 1)[:, 0]
        assert np.abs(inc - dense).max() < 1e-12
        full = O.full_causal_attention(q[:, head], k[:, head], v[:, head])
        assert np.abs(dense[C:] - full[C:]).max() > 1e-3
        np.testing.assert_allclose(dense[:C], full[:C], atol=1e-12)


def test_window_covering_everything_is_causal_softmax():
    rng = np.random.default_rng(5)
    t, d = 12, 16
    q, k, v = (rng.standard_normal((t, 1, d)) for _ in range(3))
    a = O.prefill_attention(q, lambda j: k[j], lambda j: v[j], 0, 0, 0, 1)[:, 0]
    b = O.prefill_attention(q, lambda j: k[j], lambda j: v[j], 0, 2, 100, 1)[:, 0]
    c = O.full_causal_attention(q[:, 0], k[:, 0], v[:, 0])
    np.testing.assert_allclose(a, c, atol=1e-13)
    np.testing.assert_allclose(b, c, atol=1e-13)


def test_single_visible_key_returns_value():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out = O.decode_attention(q, lambda j: k[j], lambda j: v[j], 1, 4, 12, 2)
    for h in range(4):
        np.testing.assert_allclose(out[h], v[0, h // 2], atol=1e-15)


def test_repeat_free_equals_repeat_kv():
    # [GOSS] 4.4 / 5.5: expanding KV heads (repeat_kv) then MHA equals the h -> h // n_rep map.
    rng = np.random.default_rng(7)
    Hq, Hkv, d, n = 8, 2, 16, 30
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    gqa = O.decode_attention(q, lambda j: K[j], lambda j: V[j], n, 3, 10, Hkv)
    Kr = np.repeat(K, Hq // Hkv, axis=1)
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    mha = O.decode_attention(q, lambda j: Kr[j], lambda j: Vr[j], n, 3, 10, Hq)
    np.testing.assert_allclose(gqa, mha, atol=1e-14)


def test_prefill_rows_equal_decode_and_chunking():
    # use_cache off == cached ([GOSS] 5.6); chunked prefill into a cached prefix == one shot.
    rng = np.random.default_rng(8)
    T, Hq, Hkv, d, S, W = 40, 4, 2, 8, 3, 9
    q = rng.standard_normal((T, Hq, d))
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    kb, vb = (lambda j: K[j]), (lambda j: V[j])
    one = O.prefill_attention(q, kb, vb, 0, S, W, Hkv)
    for t in (0, 5, 17, 39):
        np.testing.assert_allclose(one[t], O.decode_attention(q[t], kb, vb, t + 1, S, W, Hkv), atol=1e-14)
    parts = [O.prefill_attention(q[a:b], kb, vb, a, S, W, Hkv) for a, b in ((0, 11), (11, 12), (12, 40))]
    np.testing.assert_allclose(np.concatenate(parts), one, atol=1e-14)


# ---------------------------------------------------------------- rerotation


def test_rerotation_group_law_sink_experiment():
    # [SINK]: turning rotated keys from positions [3,4,5] to [2,3,4] equals rotating raw keys there,
    # and skipping the turn changes scores by more than 1e-3.
    d = 8
    cfg = O.RopeCfg(head_dim=d, rotary_dim=d, rope_theta=1e4, neox=False)
    T = O.build_table(cfg, 16)
    rng = np.random.default_rng(11)
    raw = rng.standard_normal((3, d))
    old = np.array([3, 4, 5])
    new = old - 1
    old_rot = O.rope_apply(raw, old, T, d, False)
    # turn by -1 position: the angle p*(w_B - w_A) form with a uniform delta
    w = O.inv_freq(cfg)
    turned = O.rotate_by_angle(old_rot, np.outer(new - old, w), d, False)
    np.testing.assert_allclose(turned, O.rope_apply(raw, new, T, d, False), atol=1e-12)
    query = O.rope_apply(rng.standard_normal((1, d)), [5], T, d, False)[0]
    wrong = old_rot @ query / math.sqrt(d)
    right = turned @ query / math.sqrt(d)
    assert np.abs(right - wrong).max() > 1e-3


@pytest.mark.parametrize("a,b", [(1.0, 2.0), (1.5, 2.0), (2.0, 1.0), (1.0, 1.125)])
def test_rerotation_equals_direct_rotation(a, b):
    # [DYN]: a key written at factor A becomes the key of factor B after one more turn by
    # p (w_B - w_A) and the mscale ratio.
    ca = O.RopeCfg(head_dim=128, rotary_dim=64, rope_theta=5e5, yarn_factor=a, orig_max_pos=262144)
    cb = O.RopeCfg(head_dim=128, rotary_dim=64, rope_theta=5e5, yarn_factor=b, orig_max_pos=262144)
    rng = np.random.default_rng(12)
    pos = np.array([0, 1, 1000, 262143, 262144, 400000, 519999])
    raw = rng.standard_normal((len(pos), 128))
    wa, wb = O.inv_freq(ca), O.inv_freq(cb)
    # rotate directly from the angle (no table of that length needed)
    ka = O.rotate_by_angle(raw, np.outer(pos, wa), 64, True, O.mscale(ca))
    kb = O.rotate_by_angle(raw, np.outer(pos, wb), 64, True, O.mscale(cb))
    turned = O.rerotate_rows(ka, pos, ca, cb)
    np.testing.assert_allclose(turned, kb, atol=1e-9)  # |angle| up to 5e5 rad: fp64 angle error ~1e-10
    np.testing.assert_array_equal(turned[:, 64:], raw[:, 64:])
    same = O.rerotate_rows(ka, pos, ca, ca)
    np.testing.assert_allclose(same, ka, atol=0)


def test_rerotation_matches_table_rows():
    # cross-check with the table path: keys written by rope_apply at A then turned == rope_apply at B.
    ca = O.RopeCfg(head_dim=64, rotary_dim=32, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=1024)
    cb = O.RopeCfg(head_dim=64, rotary_dim=32, rope_theta=5e5, yarn_factor=1.75, orig_max_pos=1024)
    Ta, Tb = O.build_table(ca, 2048), O.build_table(cb, 2048)
    rng = np.random.default_rng(13)
    pos = rng.integers(0, 2048, 50)
    raw = rng.standard_normal((50, 2, 64))
    turned = O.rerotate_rows(O.rope_apply(raw, pos, Ta, 32, True), pos, ca, cb)
    np.testing.assert_allclose(turned, O.rope_apply(raw, pos, Tb, 32, True), atol=1e-12)


def test_dynamic_factor_policy():
    # [DYN]: none inside 262,144; above it length / 262,144 rounded up to 0.125, capped at 2.
    assert O.dynamic_factor(262144, 262144) == 1.0
    assert O.dynamic_factor(262145, 262144) == 1.125
    assert O.dynamic_factor(300000, 262144) == 1.25
    assert O.dynamic_factor(524288, 262144) == 2.0
    assert O.dynamic_factor(600000, 262144) == 2.0


# ---------------------------------------------------------------- quantisers


def test_bf16_rounding_bits():
    one = 1.0
    assert O.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0            # tie -> even (down)
    assert O.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == one + 2 ** -6  # tie -> even (up)
    assert O.round_bf16(np.array([one + 2 ** -8 + 2 ** -20]))[0] == one + 2 ** -7
    x = RNG.standard_normal(1000)
    y = O.round_bf16(x)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2 ** -8 + 1e-300)
    assert np.array_equal(O.round_bf16(y), y)


def test_int8_rows():
    x = RNG.standard_normal((50, 128))
    x[3] = 0.0
    codes, scale = O.quant_int8_rows(x)
    assert scale[3] == 0 and np.all(codes[3] == 0)
    assert np.all(np.abs(codes) <= 127)
    assert np.all(np.max(np.abs(codes[np.arange(50) != 3]), axis=1) == 127)
    deq = O.dequant_int8_rows(codes, scale)
    err = np.abs(deq - x)
    assert np.all(err <= scale[:, None] * 0.5 + 1e-6)
    # the code is the nearest integer to x * 127 / max|x| (exact arithmetic), except where
    # that quotient sits within float32 rounding of a half-integer
    exact = x * 127.0 / np.max(np.abs(x), axis=1, keepdims=True).clip(1e-300)
    frac = np.abs(exact - np.floor(exact) - 0.5)
    safe = frac > 1e-4
    assert np.array_equal(codes[safe], np.rint(exact)[safe].astype(np.int8))
    # a row that is already a multiple of its step round-trips exactly
    k = RNG.integers(-127, 128, (5, 64)).astype(np.float64)
    k[:, 0] = 127
    c2, s2 = O.quant_int8_rows(k * 0.25)
    assert np.array_equal(c2, k.astype(np.int8)) and np.allclose(s2, 0.25)


# ---------------------------------------------------------------- learned sink logits


def test_learned_sink_is_a_zero_value_key():
    # A per-head logit in the denominator equals attending over one extra key whose
    # score is the logit and whose value is zero (a second formulation of the rule).
    rng = np.random.default_rng(31)
    d, n = 16, 23
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    scale = 1 / math.sqrt(d)
    for sink in (-10.0, -1.3, 0.0, 2.5, 15.0):
        got = O.attend(q, K, V, scale, sink)
        # extra key k* with k* . q * scale = sink: put it along q
        kstar = q * (sink / (scale * (q @ q)))
        ref = O.attend(q, np.vstack([K, kstar]), np.vstack([V, np.zeros(d)]), scale)
        np.testing.assert_allclose(got, ref, atol=1e-12)


def test_learned_sink_closed_forms():
    rng = np.random.default_rng(32)
    d = 8
    q = rng.standard_normal(d)
    k = rng.standard_normal((1, d))
    v = rng.standard_normal((1, d))
    s = float(k[0] @ q) / math.sqrt(d)
    for sink in (-4.0, 0.0, 3.0):
        # one visible key: the value scaled by the logistic of (score - sink)
        want = v[0] / (1.0 + math.exp(sink - s))
        np.testing.assert_allclose(O.attend(q, k, v, 1 / math.sqrt(d), sink), want, atol=1e-14)
    # a very negative sink is plain softmax attention; heads use their own logit
    K = rng.standard_normal((9, 2, d))
    V = rng.standard_normal((9, 2, d))
    Q = rng.standard_normal((4, d))
    plain = O.decode_attention(Q, lambda j: K[j], lambda j: V[j], 9, 2, 5, 2)
    far = O.decode_attention(Q, lambda j: K[j], lambda j: V[j], 9, 2, 5, 2, sink_logits=[-800.0] * 4)
    np.testing.assert_allclose(far, plain, atol=1e-15)
    mixed = O.decode_attention(Q, lambda j: K[j], lambda j: V[j], 9, 2, 5, 2, sink_logits=[-800.0, 1.0, -800.0, 1.0])
    np.testing.assert_allclose(mixed[0], plain[0], atol=1e-15)
    assert np.abs(mixed[1] - plain[1]).max() > 1e-3
    # the sink only removes mass: every output is a convex combination shrunk by the same factor
    assert np.linalg.norm(mixed[1]) < np.linalg.norm(plain[1]) + 1e-12


# ---------------------------------------------------------------- local-position shift


@pytest.mark.parametrize("neox", [True, False])
def test_shift_keys_group_law(neox):
    # [SINK] local rerotation: rotated keys at [3,4,5] moved to [2,3,4] equal keys rotated there
    # directly; moving by -p returns the raw key; two moves compose.
    cfg = O.RopeCfg(head_dim=40, rotary_dim=32, rope_theta=1e4, neox=neox)
    T = O.build_table(cfg, 64)
    rng = np.random.default_rng(41)
    raw = rng.standard_normal((3, 2, 40))
    old = np.array([3, 4, 5])
    rot = O.rope_apply(raw, old, T, 32, neox)
    np.testing.assert_allclose(O.shift_keys(rot, -1, cfg), O.rope_apply(raw, old - 1, T, 32, neox), atol=1e-12)
    back = np.stack([O.shift_keys(rot[i:i + 1], -int(old[i]), cfg)[0] for i in range(3)])
    np.testing.assert_allclose(back, raw, atol=1e-12)
    np.testing.assert_allclose(O.shift_keys(O.shift_keys(rot, 7, cfg), -3, cfg), O.shift_keys(rot, 4, cfg),
                               atol=1e-12)
    np.testing.assert_array_equal(O.shift_keys(rot, 5, cfg)[..., 32:], raw[..., 32:])


# ---------------------------------------------------------------- table variants


def test_linear_scaling_is_position_interpolation():
    # PI scales the position axis: the table at position s*m equals the plain table at m.
    base = O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=1e4)
    pi = O.RopeCfg(head_dim=64, rotary_dim=64, rope_theta=1e4, yarn_factor=4.0, rope_type="linear")
    Tp, Tb = O.build_table(pi, 4000), O.build_table(base, 1000)
    np.testing.assert_allclose(Tp[::4], Tb, atol=1e-12)
    assert O.mscale(pi) == 1.0


def test_ntk_fixed_and_dynamic():
    r, b = 128, 1e4
    cfg = O.RopeCfg(head_dim=r, rotary_dim=r, rope_theta=b, yarn_factor=8.0, rope_type="ntk")
    w, w0 = O.inv_freq(cfg), O.plain_inv_freq(r, b)
    # NTK-aware: the fastest pair is untouched, the slowest is interpolated exactly by s, geometric between
    assert w[0] == 1.0 and abs(w[-1] / w0[-1] - 1 / 8.0) < 1e-12
    ratio = w[1:] / w[:-1]
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-12)
    # dynamic NTK at the trained length is plain RoPE; at P it equals fixed NTK with s' = s P / L0 - (s - 1)
    dyn = O.RopeCfg(head_dim=r, rotary_dim=r, rope_theta=b, yarn_factor=2.0, rope_type="dynamic_ntk",
                    orig_max_pos=4096, served_len=4096)
    np.testing.assert_allclose(O.inv_freq(dyn), w0, rtol=1e-14)
    dyn2 = O.RopeCfg(head_dim=r, rotary_dim=r, rope_theta=b, yarn_factor=2.0, rope_type="dynamic_ntk",
                     orig_max_pos=4096, served_len=16384)
    fixed = O.RopeCfg(head_dim=r, rotary_dim=r, rope_theta=b, yarn_factor=2.0 * 4 - 1, rope_type="ntk")
    np.testing.assert_allclose(O.inv_freq(dyn2), O.inv_freq(fixed), rtol=1e-13)


def test_llama3_blend():
    r, b, L0, s = 128, 5e5, 8192, 8.0
    cfg = O.RopeCfg(head_dim=r, rotary_dim=r, rope_theta=b, yarn_factor=s, orig_max_pos=L0, rope_type="llama3",
                    low_freq_factor=1.0, high_freq_factor=4.0)
    w, w0 = O.inv_freq(cfg), O.plain_inv_freq(r, b)
    wl = 2 * math.pi / w0
    fast, slow = wl < L0 / 4.0, wl > L0 / 1.0
    assert fast.any() and slow.any() and (~fast & ~slow).any()
    np.testing.assert_array_equal(w[fast], w0[fast])
    np.testing.assert_allclose(w[slow], w0[slow] / s, rtol=1e-15)
    mid = w[~fast & ~slow] / w0[~fast & ~slow]
    assert np.all(mid < 1) and np.all(mid > 1 / s) and np.all(np.diff(mid) < 0)
    # continuous at both thresholds: the smoothing weight is 1 at L0/wl = 4 and 0 at L0/wl = 1
    for k, want in ((4.0, 1.0), (1.0, 1.0 / s)):
        smooth = (k - 1.0) / 3.0
        assert abs(((1 - smooth) / s + smooth) - want) < 1e-15


def test_pruned_pairs_are_identity():
    cfg = O.RopeCfg(head_dim=96, rotary_dim=96, rope_theta=1e4, pruned_pairs=12)
    T = O.build_table(cfg, 300)
    np.testing.assert_array_equal(T[:, :12], 1.0)
    np.testing.assert_array_equal(T[:, 48:60], 0.0)
    full = O.build_table(O.RopeCfg(head_dim=96, rotary_dim=96, rope_theta=1e4), 300)
    np.testing.assert_array_equal(T[:, 12:48], full[:, 12:48])
    x = RNG.standard_normal((300, 96))
    y = O.rope_apply(x, np.arange(300), T, 96, True)
    np.testing.assert_array_equal(y[:, :12], x[:, :12])
    np.testing.assert_array_equal(y[:, 48:60], x[:, 48:60])
