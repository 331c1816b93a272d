"""Invariants the pages fix, checked on GPU outputs (not only on the oracle).

- Re-rotation round trips and the factor sequence of a growing dialog, against
  "#2961 rope: --rope-scaling dynamic" ("The rotation against writing at the
  new factor"): a turn re-codes once more, so one turn's error is the written
  key's plus the carried one, sqrt(2) for equal steps, bounded there by 1.6x
  RMS and a worst element of 3 fp16 ulps / 2 int8 steps / 3 steps with the
  Hadamard.  Read the same way, one turn may add at most (1.6^2 - 1) times the
  written key's error variance, so after k turns the RMS bound is
  sqrt(1 + 1.56 k) (1.6 at k = 1), and each further turn adds at most one
  rounding to the worst element: w1 + (k - 1) u (u = 1 ulp / 1 step / 1.5
  steps).  The written key is the fp64 key at the target factor as the
  oracle's storage holds it (fp16 rounding to nearest, or the oracle's row
  quantiser), so no yardstick comes from the kernels under test.
- q . k depends only on m - n through apply_append ("RoPE, scaling, sliding
  window, attention sinks", "A worked number": q at 5 against k at 3 equals q
  at 105 against k at 103, both cos(0.2) = 0.9800666 for pair 16 at b = 1e4),
  and end to end through decode over a window.
- A prefill row equals the decode at that position ("Inference & 128K Long
  Context", 5.6 generate: prefill vs decode, use_cache on / off), both on GPU.
"""
import math

import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (DevPaged, DevRing, assert_bf16_close, decode_int8, oracle_cfg, oracle_written, rowwise,
                            to_np64, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    return R, torch, dev


def _table(R, torch, dev, cfg, P):
    t = torch.empty(P, cfg.rotary_dim, dtype=torch.float32, device=dev)
    R.build_table(cfg, P, t)
    return t


def _write(R, torch, dev, cfg, table, raw, kind, pos0):
    """Raw keys [T, Hkv, d] (fp16 on the device) written at cfg by apply_append into a CONTIG layer."""
    T, Hkv, d = raw.shape
    mode = {"i8_keep": R.I8_KEEP_SCALE, "i8_hadamard": R.I8_HADAMARD}.get(kind, 0)
    if kind == "f16":
        kc, sc, dt = torch.zeros(T, Hkv, d, dtype=torch.float16, device=dev), None, R.F16
    else:
        kc = torch.zeros(T, Hkv, d, dtype=torch.int8, device=dev)
        sc = torch.zeros(T, Hkv, dtype=torch.float32, device=dev)
        dt = R.I8
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, dt, Hkv, d, kc, capacity=T, pos0=pos0, k_scale=sc, err_word=err, k_int8_mode=mode)
    pos = torch.arange(pos0, pos0 + T, dtype=torch.int32, device=dev)
    R.apply_append(cfg, table, table.shape[0], None, 0, raw.clone(), None, R.F16, T, pos, None, desc)
    torch.cuda.synchronize()
    assert err.item() == 0
    return kc, sc, desc, err


def _values(kind, kc, sc):
    """The keys a cache holds, read back as float64 (Hadamard rows in the H domain of their codes)."""
    if kind == "f16":
        return to_np64(kc)
    return decode_int8(kc.cpu().numpy(), sc.cpu().numpy())


W1 = {"f16": 3.0, "i8": 2.0, "i8_keep": 2.0, "i8_hadamard": 3.0}


def rms_bound(k):
    """RMS ratio bound after k turns: the one-turn bound 1.6, each turn adding at most 1.6^2 - 1."""
    return math.sqrt(1.0 + (1.6 ** 2 - 1.0) * k)
WSTEP = {"f16": 1.0, "i8": 1.0, "i8_keep": 1.0, "i8_hadamard": 1.5}


def _stats(kind, turned, written, truth, unit):
    """RMS(turned - truth) / RMS(written - truth) and the worst |turned - truth| in units; turned and
    written as the cache holds them (Hadamard rows in the transformed domain, where their codes
    live), truth the plain fp64 key."""
    if kind == "i8_hadamard":
        truth = O.hadamard(truth)
    ratio = float(np.sqrt(np.mean((turned - truth) ** 2)) / np.sqrt(np.mean((written - truth) ** 2)))
    worst = float(np.max(np.abs(turned - truth) / unit))
    return ratio, worst


def _truth(raw, pos, cfg):
    o = oracle_cfg(cfg)
    return O.rotate_by_angle(raw, np.outer(pos, O.inv_freq(o))[:, None, :], cfg.rotary_dim, bool(cfg.neox), O.mscale(o))


def _cfg(R, s):
    return R.rope_cfg(128, 64, rope_theta=5e5, yarn_factor=s, orig_max_pos=262144)


@pytest.mark.parametrize("kind", ["f16", "i8", "i8_keep", "i8_hadamard"])
@pytest.mark.parametrize("fa,fb", [(1.0, 2.0), (1.5, 1.125)])
def test_rerotate_round_trip(env, kind, fa, fb):
    # keys written at A by apply_append, turned A -> B -> A, against the fp64 key at A; the key as
    # the oracle's storage holds it written directly at A (or B, after one turn) is the yardstick
    R, torch, dev = env
    T, Hkv, d = 512, 8, 128
    P = 524288
    ca, cb = _cfg(R, fa), _cfg(R, fb)
    ta = _table(R, torch, dev, ca, P)
    for pos0 in (262144 - T // 2, 519999 - T + 1):
        raw = torch.from_numpy(synth.normal((T, Hkv, d), 3000 + pos0 % 89)).to(dev, torch.float16)
        rawn = to_np64(raw)
        pos = np.arange(pos0, pos0 + T)
        kc, sc, desc, err = _write(R, torch, dev, ca, ta, raw, kind, pos0)
        truth_a, truth_b = _truth(rawn, pos, ca), _truth(rawn, pos, cb)
        written, unit = oracle_written(kind, truth_a)
        # there: one turn, against the key written directly at B
        R.rerotate(ca, cb, desc, 1)
        torch.cuda.synchronize()
        written_b, unit_b = oracle_written(kind, truth_b)
        r1, w1 = _stats(kind, _values(kind, kc, sc), written_b, truth_b, unit_b)
        assert r1 <= 1.6 and w1 <= W1[kind], (pos0, r1, w1)
        # and back: two turns, against the key written at A
        R.rerotate(cb, ca, desc, 1)
        torch.cuda.synchronize()
        assert err.item() == 0
        if kind == "f16":  # dims past the rotary slice never move
            assert torch.equal(kc[..., 64:], raw.to(torch.float16)[..., 64:])
        ratio, worst = _stats(kind, _values(kind, kc, sc), written, truth_a, unit)
        k = 2
        print(f"round trip {kind} {fa}->{fb}->{fa} pos0 {pos0}: one turn {r1:.3f}x {w1:.2f}; back {ratio:.3f}x {worst:.2f}")
        assert ratio <= rms_bound(k), (pos0, ratio)
        assert worst <= W1[kind] + (k - 1) * WSTEP[kind], (pos0, worst)


@pytest.mark.parametrize("kind", ["f16", "i8", "i8_keep"])
def test_rerotate_factor_sequence(env, kind):
    # one cache written at factor 1, turned 1 -> 1.125 -> ... -> 2, then 2 -> 1 and 1 -> 2 (the
    # growing dialog of the page's band runs); after every switch, against the fp64 key at that
    # factor with the key written directly at it (by the oracle's storage) as the yardstick, k turns
    # so far
    R, torch, dev = env
    T, Hkv, d, P = 512, 8, 128, 524288
    pos0 = 519999 - T + 1
    raw = torch.from_numpy(synth.normal((T, Hkv, d), 3100)).to(dev, torch.float16)
    rawn = to_np64(raw)
    pos = np.arange(pos0, pos0 + T)
    factors = [1.0 + 0.125 * i for i in range(9)]
    steps = list(zip(factors[:-1], factors[1:])) + [(2.0, 1.0), (1.0, 2.0)]
    kc, sc, desc, err = _write(R, torch, dev, _cfg(R, 1.0), _table(R, torch, dev, _cfg(R, 1.0), P), raw, kind, pos0)
    kept = []
    for k, (fa, fb) in enumerate(steps, start=1):
        before = sc.clone() if sc is not None else None
        R.rerotate(_cfg(R, fa), _cfg(R, fb), desc, 1)
        torch.cuda.synchronize()
        assert err.item() == 0
        if kind == "i8_keep":
            kept.append(float((sc == before).float().mean().item()))
        truth = _truth(rawn, pos, _cfg(R, fb))
        written, unit = oracle_written(kind, truth)
        ratio, worst = _stats(kind, _values(kind, kc, sc), written, truth, unit)
        print(f"sequence {kind} step {k} {fa}->{fb}: {ratio:.3f}x (bound {rms_bound(k):.3f}), "
              f"worst {worst:.2f} (bound {W1[kind] + (k - 1) * WSTEP[kind]:.1f})"
              + (f", kept {kept[-1]:.4f}" if kept else ""))
        assert ratio <= rms_bound(k), (k, fa, fb, ratio)
        assert worst <= W1[kind] + (k - 1) * WSTEP[kind], (k, fa, fb, worst)
    if kind == "i8_keep":
        assert all(0.0 < f <= 1.0 for f in kept) and kept[0] < 1.0


@pytest.mark.parametrize("neox", [True, False])
def test_qk_depends_only_on_offset_through_append(env, neox):
    # the worked number: pair 16 at b = 1e4, r = 128, q = k = (1, 0) before rotation; q at 5 against
    # k at 3, and q at 105 against k at 103, both cos(0.2); then random q, k at (m, n) and (m + s, n + s)
    R, torch, dev = env
    d, Hkv, P = 128, 1, 512
    cfg = R.rope_cfg(d, d, rope_theta=1e4, neox=neox)
    table = _table(R, torch, dev, cfg, P)

    def rotated(vec_q, vec_k, m, n):
        # q of the token at m and k of the token at n, rotated by apply_append (a contiguous cache
        # written at positions n and m)
        q = torch.zeros(2, 1, d, dtype=torch.float32, device=dev)
        k = torch.zeros(2, 1, d, dtype=torch.float32, device=dev)
        q[1, 0] = torch.from_numpy(vec_q)
        k[0, 0] = torch.from_numpy(vec_k)
        kc = torch.zeros(P, Hkv, d, dtype=torch.float32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        desc = R.kv_cache(R.CONTIG, R.F32, Hkv, d, kc, capacity=P, pos0=0, err_word=err)
        pos = torch.tensor([n, m], dtype=torch.int32, device=dev)
        R.apply_append(cfg, table, P, q, 1, k, None, R.F32, 2, pos, None, desc)
        torch.cuda.synchronize()
        assert err.item() == 0
        return float((q[1, 0].double() * kc[n, 0].double()).sum().item())

    e16 = np.zeros(d, dtype=np.float32)
    e16[16 if neox else 32] = 1.0  # the first member of pair 16
    s53 = rotated(e16, e16, 5, 3)
    s_far = rotated(e16, e16, 105, 103)
    assert abs(s53 - 0.9800666) < 5e-7 and abs(s_far - 0.9800666) < 5e-7, (s53, s_far)
    rng = synth.rng(3200 + neox)
    for _ in range(4):
        vq = rng.standard_normal(d).astype(np.float32)
        vk = rng.standard_normal(d).astype(np.float32)
        m, n = sorted(rng.integers(0, 200, 2).tolist(), reverse=True)
        shift = int(rng.integers(1, 300))
        a = rotated(vq, vk, m, n)
        b = rotated(vq, vk, m + shift, n + shift)
        scale = float(np.linalg.norm(vq) * np.linalg.norm(vk))
        assert abs(a - b) <= 2e-6 * scale, (m, n, shift, a, b)


def test_windowed_decode_is_shift_invariant(env):
    # the same 40 raw tokens appended at positions 0.. of sequence 0 and at positions 1000.. of
    # sequence 1 (behind 1000 other tokens); a window of 40 (no sinks) sees exactly those tokens, so
    # the two decodes' outputs agree: attention reads only relative positions
    R, torch, dev = env
    Hq, Hkv, d, W, N, lead = 8, 4, 64, 40, 40, 1000
    cfg = R.rope_cfg(d, d, rope_theta=1e4)
    P = lead + N
    table = _table(R, torch, dev, cfg, P)
    cache = DevRing(R, torch, dev, torch.float32, 2, Hkv, d, 0, W)
    qr = torch.from_numpy(synth.normal((N, Hq, d), 3300)).to(dev)
    kr = torch.from_numpy(synth.normal((N, Hkv, d), 3301)).to(dev)
    vr = torch.from_numpy(synth.normal((N, Hkv, d), 3302)).to(dev)
    junk_k = torch.from_numpy(synth.normal((lead, Hkv, d), 3303)).to(dev)
    junk_v = torch.from_numpy(synth.normal((lead, Hkv, d), 3304)).to(dev)
    # sequence 1: the lead tokens first (no queries kept)
    R.apply_append(cfg, table, P, None, 0, junk_k, junk_v, R.F32, lead, torch.arange(lead, dtype=torch.int32, device=dev),
                   torch.ones(lead, dtype=torch.int32, device=dev), cache.desc)
    q0, q1 = qr.clone(), qr.clone()
    R.apply_append(cfg, table, P, q0, Hq, kr.clone(), vr, R.F32, N, torch.arange(N, dtype=torch.int32, device=dev),
                   torch.zeros(N, dtype=torch.int32, device=dev), cache.desc)
    R.apply_append(cfg, table, P, q1, Hq, kr.clone(), vr, R.F32, N,
                   torch.arange(lead, lead + N, dtype=torch.int32, device=dev),
                   torch.ones(N, dtype=torch.int32, device=dev), cache.desc)
    qd = torch.stack([q0[N - 1], q1[N - 1]])
    out = torch.empty_like(qd)
    ws = torch.empty(R.decode_workspace_size(2, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(qd, 2, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    assert cache.seq_len.cpu().tolist() == [N, lead + N]
    a, b = to_np64(out[0]), to_np64(out[1])
    assert rowwise(b, a) <= 1e-5
    # and the rotated queries differ (the positions did move them)
    assert float(np.max(np.abs(to_np64(q0[N - 1]) - to_np64(q1[N - 1])))) > 0.1


@pytest.mark.parametrize("dtype_name,S,W", [("f32", 4, 60), ("bf16", 4, 60), ("f32", 0, 0)])
def test_prefill_rows_equal_decode(env, dtype_name, S, W):
    # one chunk of T tokens through prefill, and the same tokens appended one at a time with a decode
    # after each: prefill row t equals the decode at position t (both kernels' outputs)
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    act = R.F32 if dtype_name == "f32" else R.BF16
    T, Hq, Hkv, d = 150, 16, 4, 128
    cfg = R.rope_cfg(d, d, rope_theta=5e5)
    table = _table(R, torch, dev, cfg, T)
    q = torch.from_numpy(synth.normal((T, Hq, d), 3400)).to(dev, dtype)
    k = torch.from_numpy(synth.normal((T, Hkv, d), 3401)).to(dev, dtype)
    v = torch.from_numpy(synth.normal((T, Hkv, d), 3402)).to(dev, dtype)
    max_blocks = T // 16 + 1
    tab = synth.block_table_permutation(1, max_blocks, max_blocks, 3403)
    # prefill: rotate the chunk (its own cache write is not used), attend with the chunk's keys
    c1 = DevPaged(R, torch, dev, dtype, 1, Hkv, d, S, W, tab, max_blocks)
    qp, kp = q.clone(), k.clone()
    R.apply_append(cfg, table, T, qp, Hq, kp, v, act, T, torch.arange(T, dtype=torch.int32, device=dev),
                   torch.zeros(T, dtype=torch.int32, device=dev), c1.desc)
    pre = torch.empty_like(qp)
    R.prefill_attn(qp, kp, v, T, 0, Hq, c1.desc, 0, 0.0, pre)
    # decode: one token at a time into a fresh cache
    c2 = DevPaged(R, torch, dev, dtype, 1, Hkv, d, S, W, tab, max_blocks)
    dec = torch.empty(T, Hq, d, dtype=dtype, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    for t in range(T):
        qt = q[t:t + 1].clone()
        R.apply_append(cfg, table, T, qt, Hq, k[t:t + 1].clone(), v[t:t + 1], act, 1,
                       torch.tensor([t], dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev),
                       c2.desc)
        R.decode_attn(qt, 1, Hq, c2.desc, 0.0, dec[t:t + 1], ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert c1.err.item() == 0 and c2.err.item() == 0
    a, b = to_np64(pre), to_np64(dec)
    if dtype_name == "f32":
        assert rowwise(a, b) <= 2e-5  # two fp32 paths, each within 1e-5 of the exact value
    else:
        assert_bf16_close(a, b, atol=4e-2, rtol=2e-2)  # two bf16 results, each within 2e-2 + 1e-2 |ref|
