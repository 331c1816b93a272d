"""GPU parity: every entry point of libropekv.so against the fp64 oracle.

Integer state (ring head / count, seq_len, block tables, freed ids, visible
slots) must match bit for bit.  fp32 paths: max |gpu - ref| / max |ref|
<= 1e-5 per tensor (per row for attention).  bf16 rotations: one rounding of
the exact value (half a bf16 ulp plus 1e-6 of the row's largest value for the
fp32 arithmetic).  bf16 attention: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise.  Oracle inputs are the host copies of the
seeded inputs (rounded to the activation dtype by torch before upload); no
oracle input or expected value comes from the HIP path.
"""
import math

import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (bf16_attention_ref, bf16_round, EPS_TURN_I8, DevPaged, DevRing, assert_bf16_close, assert_bf16_rounded, assert_int8_codes_valid, assert_rounded_once, attend_set,
                            decode_e4m3, decode_int8, excess, int8_turn_quotients, needle_dirs, needle_kv, normwise, oracle_cfg,
                            oracle_written, plant_queries_, rowwise, to_np64, torch_dev)

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


# ------------------------------------------------------------------ table

TABLE_CASES = [
    (dict(head_dim=64, rotary_dim=64, rope_theta=1e4), 80),
    (dict(head_dim=128, rotary_dim=128, rope_theta=5e5), 32768),
    (dict(head_dim=128, rotary_dim=64, rope_theta=5e5, yarn_factor=2.0, orig_max_pos=262144), 524288),
    (dict(head_dim=128, rotary_dim=128, rope_theta=1e4, yarn_factor=8.0, orig_max_pos=4096), 32768),
    (dict(head_dim=96, rotary_dim=32, rope_theta=1e4, yarn_factor=1.125, orig_max_pos=100, neox=False), 1000),
    (dict(head_dim=64, rotary_dim=64, rope_theta=1e4, yarn_factor=4.0, rope_type=1), 4000),
    (dict(head_dim=128, rotary_dim=128, rope_theta=1e4, yarn_factor=8.0, rope_type=2), 32768),
    (dict(head_dim=128, rotary_dim=128, rope_theta=1e4, yarn_factor=2.0, rope_type=3, orig_max_pos=4096,
          served_len=16384), 16384),
    (dict(head_dim=128, rotary_dim=128, rope_theta=5e5, yarn_factor=8.0, rope_type=4, orig_max_pos=8192,
          low_freq_factor=1.0, high_freq_factor=4.0), 65536),
    (dict(head_dim=96, rotary_dim=96, rope_theta=1e4, pruned_pairs=12), 3000),
    (dict(head_dim=128, rotary_dim=128, rope_theta=1e4, yarn_factor=4.0, orig_max_pos=4096, pruned_pairs=16), 8000),
]


@pytest.mark.parametrize("args,P", TABLE_CASES)
def test_table_matches_oracle(env, args, P):
    R, torch, dev = env
    cfg = R.rope_cfg(**args)
    ms = torch.zeros(1, dtype=torch.float32, device=dev)
    t = torch.empty(P, cfg.rotary_dim, dtype=torch.float32, device=dev)
    R.build_table(cfg, P, t, ms)
    torch.cuda.synchronize()
    got = t.cpu().numpy().astype(np.float64)
    oc = oracle_cfg(cfg)
    ref = O.build_table(oc, P)
    # one fp32 ulp of the value, plus the conditioning of the fp64 angle m*w itself: its own
    # rounding (a few ulps of |m w|) moves cos / sin by up to that much on either side
    ang = np.outer(np.arange(P, dtype=np.float64), O.inv_freq(oc))
    ang = np.concatenate([ang, ang], axis=1)
    tol = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 4 * 2.0 ** -52 * ang * O.mscale(oc)
    assert np.all(np.abs(got - ref) <= tol), float(np.max(np.abs(got - ref) / tol))
    assert abs(float(ms.item()) - O.mscale(oc)) < 1e-7
    # the result does not depend on the launch shape: a shorter build is a bitwise prefix
    P2 = P // 2 + 3
    t2 = _table(R, torch, dev, cfg, P2)
    assert torch.equal(t2, t[:P2])


def test_table_factor_one_is_plain(env):
    R, torch, dev = env
    a = _table(R, torch, dev, R.rope_cfg(128, 64, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=262144), 4096)
    b = _table(R, torch, dev, R.rope_cfg(128, 64, rope_theta=5e5), 4096)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ ring: 16-slot cache (S 4 + W 12) end to end

def _ring_end_to_end(env, neox, dtype_name, chunks, S=4, W=12):
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    act = {"f32": R.F32, "bf16": R.BF16}[dtype_name]
    B, Hq, Hkv, d = 1, 8, 4, 64
    n_total = sum(chunks)
    cfg = R.rope_cfg(d, d, rope_theta=1e4, neox=neox)
    ocfg = oracle_cfg(cfg)
    table = _table(R, torch, dev, cfg, n_total)
    otab = O.build_table(ocfg, n_total)
    # inputs rounded to the activation dtype by torch; the oracle reads the rounded values
    qd = torch.from_numpy(synth.normal((n_total, Hq, d), 101)).to(dev, dtype)
    kd = torch.from_numpy(synth.normal((n_total, Hkv, d), 102)).to(dev, dtype)
    vd = torch.from_numpy(synth.normal((n_total, Hkv, d), 103)).to(dev, dtype)
    qraw, kraw, vraw = to_np64(qd), to_np64(kd), to_np64(vd)
    qrot = O.rope_apply(qraw, np.arange(n_total), otab, d, neox)
    krot = O.rope_apply(kraw, np.arange(n_total), otab, d, neox)
    cache = DevRing(R, torch, dev, dtype, B, Hkv, d, S, W)
    oring = O.RingSeq(sinks=S, window=W)
    out = torch.empty(1, Hq, d, dtype=dtype, device=dev)
    ws = torch.empty(R.decode_workspace_size(1, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    tol = 1e-5 if dtype_name == "f32" else None
    p0 = 0
    for T in chunks:
        q = qd[p0:p0 + T].clone()
        k = kd[p0:p0 + T].clone()
        v = vd[p0:p0 + T].clone()
        pos = torch.arange(p0, p0 + T, dtype=torch.int32, device=dev)
        seq = torch.zeros(T, dtype=torch.int32, device=dev)
        R.apply_append(cfg, table, n_total, q, Hq, k, v, act, T, pos, seq, cache.desc)
        oring.append(T)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        # rotated q, k in place
        if tol:
            assert normwise(to_np64(q), qrot[p0:p0 + T]) <= tol
            assert normwise(to_np64(k), krot[p0:p0 + T]) <= tol
        else:
            assert_bf16_rounded(to_np64(q), qrot[p0:p0 + T])
            assert_bf16_rounded(to_np64(k), krot[p0:p0 + T])
        # integer ring state
        assert (cache.head.item(), cache.count.item(), cache.seq_len.item()) == (oring.head, oring.count,
                                                                                  oring.seq_len)
        # cache contents: every live slot holds the rotated key / raw value of its position
        kc = to_np64(cache.k[0])
        vc = to_np64(cache.v[0])
        for slot, p in oring.slot_pos.items():
            if tol:
                assert normwise(kc[:, slot], krot[p]) <= tol
            else:
                assert_bf16_rounded(kc[:, slot], krot[p])
            assert np.array_equal(vc[:, slot], vraw[p])
        # visible slots, chronological, bit-exact
        n_out = torch.zeros(1, dtype=torch.int32, device=dev)
        vp = torch.zeros(64, dtype=torch.int32, device=dev)
        vo = torch.zeros(64, dtype=torch.int64, device=dev)
        R.visible_slots(cache.desc, 0, vp, vo, 64, n_out)
        torch.cuda.synchronize()
        nv = n_out.item()
        want_pos = O.visible_positions(oring.seq_len - 1, S, W)
        assert vp[:nv].cpu().tolist() == want_pos
        want_slots = oring.chronological_slots()
        assert (vo[:nv].cpu().numpy() // d).tolist() == want_slots
        # the attention reads the oracle's rotated keys and queries as the cache and activations
        # hold them (rounded once to bf16; fp32 holds them to 1e-7)
        kbp = {j: krot[j] if tol else bf16_round(krot[j]) for j in range(n_total)}
        qref = qrot if tol else bf16_round(qrot)
        if T > 1:
            o = torch.empty(T, Hq, d, dtype=dtype, device=dev)
            R.prefill_attn(q, k, v, T, p0, Hq, cache.desc, 0, 0.0, o)
            torch.cuda.synchronize()
            # prefix keys the chunk's queries need, and whether the ring still holds them
            needed = {j for t in range(p0, p0 + T) for j in O.visible_positions(t, S, W) if j < p0}
            present = set(oring.slot_pos.values())
            if needed <= present:
                assert cache.err.item() == 0
                args = (qref[p0:p0 + T], lambda j: kbp[j], lambda j: vraw[j], p0, S, W, Hkv)
                if tol:
                    assert rowwise(to_np64(o), O.prefill_attention(*args)) <= tol
                else:
                    bf16_attention_ref(to_np64(o), O.prefill_attention, *args)
            else:
                assert cache.err.item() & R.DEV_PREFIX_LOST
                cache.err.zero_()
        R.decode_attn(q[T - 1:T], 1, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
        torch.cuda.synchronize()
        args = (qref[p0 + T - 1], lambda j: kbp[j], lambda j: vraw[j], p0 + T, S, W, Hkv)
        if tol:
            assert rowwise(to_np64(out[0]), O.decode_attention(*args)) <= tol
        else:
            bf16_attention_ref(to_np64(out[0]), O.decode_attention, *args)
        p0 += T


@pytest.mark.parametrize("neox", [True, False])
def test_ring_c16_prefill_then_decode(env, neox):
    # the tiny fp32 case: prefill 0..63, then 16 decode steps
    _ring_end_to_end(env, neox, "f32", [64] + [1] * 16)


@pytest.mark.parametrize("chunks", [[3, 1, 1, 20, 1, 7, 1], [2, 2, 9, 13, 1], [30, 1, 2]])
def test_ring_chunked_appends(env, chunks):
    # chunks that fit (pos0 + T <= C), that wrap, and that exceed the window in one call
    _ring_end_to_end(env, True, "f32", chunks)


def test_ring_bf16(env):
    _ring_end_to_end(env, True, "bf16", [40, 1, 1, 1, 5])


@pytest.mark.parametrize("S,dtype_name", [(2, "f32"), (0, "f32"), (3, "bf16")])
def test_ring_window_of_one(env, S, dtype_name):
    # the degenerate window W = 1: every query sees the sinks and itself; each token overwrites the
    # single ring slot, chunks longer than the ring keep only their last token
    _ring_end_to_end(env, True, dtype_name, [5, 1, 1, 3, 1, 2], S=S, W=1)


def _random_ring_case(seed):
    """(neox, dtype, S, W, chunks): a seeded ring geometry and a chunk sequence that fills the sinks
    in pieces, wraps the ring several times, and appends chunks shorter than, equal to and longer
    than the window into a non-empty ring."""
    rng = synth.rng(seed)
    S = int(rng.integers(0, 6))
    W = int(rng.choice([1, 2, int(rng.integers(3, 41))]))
    lens = [int(rng.choice([1, 1, 2, W, W + 1, int(rng.integers(1, 3 * W + 2))])) for _ in range(10)]
    return bool(seed % 2), ("bf16" if seed % 3 == 0 else "f32"), S, W, lens


@pytest.mark.parametrize("seed", [2501, 2502, 2503, 2504, 2505, 2506])
def test_ring_random_chunk_sequences(env, seed):
    neox, dtype_name, S, W, chunks = _random_ring_case(seed)
    _ring_end_to_end(env, neox, dtype_name, chunks, S=S, W=W)


# ------------------------------------------------------------------ rope + append over head shapes

APPEND_SHAPES = [
    # layout, dtype, d, r, neox, Hq, Hkv, unaligned activations, YaRN factor
    ("ring", "bf16", 512, 512, True, 4, 2, False, 1.0),     # the largest head (16-byte unit path)
    ("contig", "f32", 512, 128, False, 0, 3, False, 1.0),   # keys only, no q, CONTIG rows from pos0 1000
    ("ring", "f16", 256, 64, True, 6, 2, False, 4.0),       # partial rotary, YaRN table (mscale != 1)
    ("ring", "bf16", 128, 36, True, 4, 1, False, 1.0),      # r / 2 = 18: not whole units, element path
    ("ring", "f32", 34, 18, False, 2, 2, False, 1.0),       # d not a whole number of units
    ("ring", "f16", 2, 2, True, 1, 1, False, 1.0),          # the smallest head
    ("contig", "bf16", 6, 4, False, 3, 1, False, 1.0),
    ("ring", "bf16", 128, 128, True, 8, 2, True, 1.0),      # unit-shaped rows at 2-byte offsets: element path
    ("ring", "f32", 512, 2, True, 2, 1, False, 1.0),        # one rotary pair in the largest head
]


@pytest.mark.parametrize("layout,dtype_name,d,r,neox,Hq,Hkv,unaligned,yarn", APPEND_SHAPES)
def test_append_head_shapes(env, layout, dtype_name, d, r, neox, Hq, Hkv, unaligned, yarn):
    # every head shape the append accepts runs one of two paths (16-byte units when the rotary
    # halves, the tail and the addresses allow, else element by element); both against the oracle:
    # q and k rotated in place and the cached k one rounding of the exact rotation, the tail and v
    # bit for bit, slots past the appended run untouched
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype_name]
    act = {"f32": R.F32, "bf16": R.BF16, "f16": R.F16}[dtype_name]
    n = 37
    pos0 = 1000 if layout == "contig" else 0
    kw = dict(yarn_factor=yarn, orig_max_pos=16) if yarn > 1.0 else {}
    cfg = R.rope_cfg(d, r, rope_theta=1e4, neox=neox, **kw)
    table = _table(R, torch, dev, cfg, pos0 + n)
    otab = O.build_table(oracle_cfg(cfg), pos0 + n)
    positions = np.arange(pos0, pos0 + n)

    def upload(shape, seed):
        host = torch.from_numpy(synth.normal(shape, seed)).to(dtype)
        if not unaligned:
            return host.to(dev)
        buf = torch.empty(host.numel() + 1, dtype=dtype, device=dev)  # one element in: off 16-byte alignment
        view = buf[1:].view(shape)
        view.copy_(host.to(dev))
        return view

    q = upload((n, Hq, d), 301) if Hq else None
    k = upload((n, Hkv, d), 302)
    v = upload((n, Hkv, d), 303)
    q_raw = to_np64(q) if Hq else None
    k_raw, v_raw = to_np64(k), to_np64(v)
    pos = torch.from_numpy(positions.astype(np.int32)).to(dev)
    if layout == "ring":
        S = 2
        cache = DevRing(R, torch, dev, dtype, 1, Hkv, d, S, n + 5)
        desc, err = cache.desc, cache.err
        seq = torch.zeros(n, dtype=torch.int32, device=dev)
    else:
        kc = torch.zeros(n, Hkv, d, dtype=dtype, device=dev)
        vc = torch.zeros_like(kc) if Hq else None  # the keys-only case has no value cache
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        desc = R.kv_cache(R.CONTIG, act, Hkv, d, kc, vc, capacity=n, pos0=pos0, err_word=err)
        seq = None
        if vc is None:
            v, v_raw = None, None
    R.apply_append(cfg, table, pos0 + n, q, Hq, k, v, act, n, pos, seq, desc)
    torch.cuda.synchronize()
    assert err.item() == 0
    k_want = O.rope_apply(k_raw, positions, otab, r, neox)
    got_k = to_np64(k)
    assert_rounded_once(got_k, k_want, dtype_name)
    assert np.array_equal(got_k[..., r:], k_raw[..., r:])
    if Hq:
        got_q = to_np64(q)
        assert_rounded_once(got_q, O.rope_apply(q_raw, positions, otab, r, neox), dtype_name)
        assert np.array_equal(got_q[..., r:], q_raw[..., r:])
    if layout == "ring":
        # an empty ring takes a run shorter than W at slots p (sinks p < S, then S + p - S)
        oring = O.RingSeq(sinks=S, window=n + 5)
        oring.append(n)
        assert (cache.head.item(), cache.count.item(), cache.seq_len.item()) == (oring.head, oring.count,
                                                                                  oring.seq_len)
        assert sorted(oring.slot_pos.items()) == [(s, s) for s in range(n)]  # slot -> position
        kc_rows = to_np64(cache.k[0].permute(1, 0, 2))  # [C, Hkv, d]
        vc_rows = to_np64(cache.v[0].permute(1, 0, 2))
    else:
        kc_rows = to_np64(kc)
        vc_rows = to_np64(vc) if vc is not None else None
    assert_rounded_once(kc_rows[:n], k_want, dtype_name)
    assert np.array_equal(kc_rows[:n], got_k)  # the cached key is the in-place rotated key
    assert not np.any(kc_rows[n:])
    if vc_rows is not None:
        assert np.array_equal(vc_rows[:n], v_raw)
        assert not np.any(vc_rows[n:])


# ------------------------------------------------------------------ paged append + freeing + decode

def _paged_end_to_end(env, dtype_name, S, W, B, Hq, Hkv, d, rounds, seed, bs=16):
    """Mixed rounds of chunk appends and single-token steps into a paged cache of bs-token blocks:
    integer state, freed ids and cache contents against the oracle after every round, and (for the
    16-token blocks the decode takes) the decode of every sequence."""
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    act = {"f32": R.F32, "bf16": R.BF16}[dtype_name]
    rng = synth.rng(seed)
    max_len = 200
    max_blocks = max_len // bs + 1
    num_blocks = B * max_blocks + 7
    table = synth.block_table_permutation(B, max_blocks, num_blocks, seed + 1)
    cfg = R.rope_cfg(d, d, rope_theta=5e5)
    ocfg = oracle_cfg(cfg)
    gtab = _table(R, torch, dev, cfg, max_len)
    otab = O.build_table(ocfg, max_len)
    cache = DevPaged(R, torch, dev, dtype, B, Hkv, d, S, W, table, num_blocks, bs=bs)
    otable = [list(map(int, row)) for row in table]
    qall = synth.normal((B, max_len, Hq, d), seed + 2)
    kall = synth.normal((B, max_len, Hkv, d), seed + 3)
    vall = synth.normal((B, max_len, Hkv, d), seed + 4)
    # round through the device dtype once so both sides see identical inputs
    kall = to_np64(torch.from_numpy(kall).to(dtype))
    vall = to_np64(torch.from_numpy(vall).to(dtype))
    qall = to_np64(torch.from_numpy(qall).to(dtype))
    krot = np.stack([O.rope_apply(kall[b], np.arange(max_len), otab, d, True) for b in range(B)])
    qrot = np.stack([O.rope_apply(qall[b], np.arange(max_len), otab, d, True) for b in range(B)])
    n = [0] * B
    freed_dev = torch.full((B * max_blocks,), -7, dtype=torch.int32, device=dev)
    nfreed = torch.zeros(1, dtype=torch.int32, device=dev)
    if bs == 16:
        ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    vis_p = torch.zeros(max_len + 8, dtype=torch.int32, device=dev)
    vis_o = torch.zeros(max_len + 8, dtype=torch.int64, device=dev)
    vis_n = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(rounds):
        # a mixed step: some sequences prefill a chunk, some decode one token, some idle
        toks, poss, seqs, oracle_freed = [], [], [], []
        for b in range(B):
            step = int(rng.choice([0, 1, 1, int(rng.integers(2, 40))]))
            step = min(step, max_len - n[b])
            if step == 0:
                continue
            oracle_freed += O.paged_free_expired(otable[b], n[b], S, W, bs)
            for p in range(n[b], n[b] + step):
                toks.append((b, p))
            n[b] += step
        if not toks:
            continue
        N = len(toks)
        q = torch.from_numpy(np.stack([qall[b, p] for b, p in toks])).to(dev, dtype)
        k = torch.from_numpy(np.stack([kall[b, p] for b, p in toks])).to(dev, dtype)
        v = torch.from_numpy(np.stack([vall[b, p] for b, p in toks])).to(dev, dtype)
        pos = torch.tensor([p for _, p in toks], dtype=torch.int32, device=dev)
        seq = torch.tensor([b for b, _ in toks], dtype=torch.int32, device=dev)
        nfreed.zero_()
        R.apply_append(cfg, gtab, max_len, q, Hq, k, v, act, N, pos, seq, cache.desc, freed_dev, freed_dev.numel(),
                       nfreed)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        assert cache.seq_len.cpu().tolist() == n
        assert cache.table.cpu().numpy().tolist() == otable
        nf = nfreed.item()
        assert sorted(freed_dev[:nf].cpu().tolist()) == sorted(oracle_freed)
        # contents of every live (non-null) block at written positions
        kc = to_np64(cache.k)
        vc = to_np64(cache.v)
        for b in range(B):
            for p in range(n[b]):
                bid = otable[b][p // bs]
                if bid < 0:
                    continue
                got_k = kc[bid, :, p % bs]
                if dtype_name == "f32":
                    assert normwise(got_k, krot[b, p]) <= 1e-5
                else:
                    assert_bf16_rounded(got_k, krot[b, p])
                assert np.array_equal(vc[bid, :, p % bs], vall[b, p])
        # visible positions of each sequence's next query, chronological, with the element offset of
        # each key row (head 0) through the oracle's block table; no visible key sits in a freed block
        for b in range(B):
            vis_n.zero_()
            R.visible_slots(cache.desc, b, vis_p, vis_o, vis_p.numel(), vis_n)
            torch.cuda.synchronize()
            nv = vis_n.item()
            want = O.visible_positions(n[b] - 1, S, W) if n[b] > 0 else []
            assert vis_p[:nv].cpu().tolist() == want
            offs = [((otable[b][j // bs] * Hkv) * bs + j % bs) * d for j in want]
            assert all(otable[b][j // bs] >= 0 for j in want)
            assert vis_o[:nv].cpu().tolist() == offs
        if bs != 16:
            continue
        # decode for every sequence with its latest query
        qd = torch.from_numpy(np.stack([qrot[b, max(n[b] - 1, 0)] for b in range(B)])).to(dev, dtype)
        out = torch.empty(B, Hq, d, dtype=dtype, device=dev)
        R.decode_attn(qd, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        got = to_np64(out)
        qused = to_np64(qd)  # the oracle's rotated queries, rounded to the activation dtype by torch
        kref = krot if dtype_name == "f32" else bf16_round(krot)  # the rotated keys as the cache holds them
        for b in range(B):
            if n[b] == 0:
                assert np.all(got[b] == 0)
                continue
            args = (qused[b], lambda j: kref[b, j], lambda j: vall[b, j], n[b], S, W, Hkv)
            if dtype_name == "f32":
                assert rowwise(got[b], O.decode_attention(*args)) <= 1e-5
            else:
                bf16_attention_ref(got[b], O.decode_attention, *args)


@pytest.mark.parametrize("bs,S,W", [(1, 2, 5), (8, 4, 20), (32, 3, 40), (5, 0, 17)])
def test_paged_append_block_sizes(env, bs, S, W):
    # the append's slot rule, window edge and null-block freeing with blocks other than 16 tokens
    # (one token per block, a block smaller than the sinks' span, larger ones, an odd size)
    _paged_end_to_end(env, "bf16", S, W, B=5, Hq=8, Hkv=2, d=64, rounds=8, seed=2400 + bs, bs=bs)


@pytest.mark.parametrize("S,W", [(4, 12), (0, 20), (4, 0), (3, 33), (2, 1), (0, 1)])
def test_paged_small_shapes(env, S, W):
    _paged_end_to_end(env, "f32", S, W, B=3, Hq=8, Hkv=4, d=64, rounds=14, seed=7 + S + W)


def test_paged_bf16_gqa4(env):
    _paged_end_to_end(env, "bf16", 4, 40, B=4, Hq=32, Hkv=8, d=128, rounds=12, seed=300)


# ------------------------------------------------------------------ decode at larger shapes (synthetic caches)

def _fill(torch, t, seed):
    synth.device_normal_(t, seed)
    return t


@pytest.mark.parametrize("n_rep,d,dt", [(4, 128, "bf16"), (8, 128, "bf16"), (2, 64, "bf16"), (1, 128, "bf16"),
                                         (1, 128, "f32"), (4, 128, "f32"), (8, 128, "f32")])
def test_decode_paged_random_table(env, n_rep, d, dt):
    # Llama-3-8B-layer-shaped heads (8 KV heads): paged 16-token blocks, random block table, ragged
    # lengths incl. 1 and block edges;
    # fp32 caches at d 128 run the kernels whose P . V is on the VALU (the largest register use)
    R, torch, dev = env
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    Hkv = 8
    Hq = Hkv * n_rep
    lens = [1, 15, 16, 17, 300, 1024, 2000, 2049]
    B = len(lens)
    max_blocks = 130
    num_blocks = B * max_blocks + 11
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 41)
    cache = DevPaged(R, torch, dev, tdt, B, Hkv, d, 0, 0, table, num_blocks)
    _fill(torch, cache.k, 42)
    _fill(torch, cache.v, 43)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=tdt, device=dev), 44)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kp = to_np64(cache.k)
    vp = to_np64(cache.v)
    qq = to_np64(q)
    got = to_np64(out)
    for b, n in enumerate(lens):
        rows = [table[b, j // 16] for j in range(n)]
        K = np.stack([kp[rows[j], :, j % 16] for j in range(n)])
        V = np.stack([vp[rows[j], :, j % 16] for j in range(n)])
        args = (qq[b], lambda j: K[j], lambda j: V[j], n, 0, 0, Hkv)
        if dt == "bf16":
            bf16_attention_ref(got[b], O.decode_attention, *args)
        else:
            assert rowwise(got[b], O.decode_attention(*args)) <= 1e-5


@pytest.mark.parametrize("B,Hkv,n", [(1, 8, 19999), (2, 2, 5003)])
def test_decode_paged_few_long_sequences(env, B, Hkv, n):
    # a small batch spreads each sequence over many splits (the plan keeps ~512 workgroups):
    # 64 splits of 20 tiles for one sequence of 8 KV heads, up to 128 splits for 2 x 2
    R, torch, dev = env
    n_rep, d = 4, 128
    Hq = Hkv * n_rep
    max_blocks = (n + 15) // 16 + 3
    num_blocks = B * max_blocks + 5
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 51 + n)
    cache = DevPaged(R, torch, dev, torch.bfloat16, B, Hkv, d, 0, 0, table, num_blocks)
    _fill(torch, cache.k, 52)
    _fill(torch, cache.v, 53)
    lens = [n - 7 * b for b in range(B)]
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 54)
    ws_bytes = R.decode_workspace_size(B, Hq, cache.desc)
    # needles at the first and last keys and on both sides of every split edge
    splits = ws_bytes // (B * Hkv * n_rep * (d + 2) * 4)
    sp = 16 * ((max_blocks + splits - 1) // splits) if splits else 16 * (max_blocks // 2)
    u = needle_dirs(Hkv, d, 55)
    for b, nb in enumerate(lens):
        edges = list(range(sp, nb, sp))
        edges = sorted({edges[0], edges[1], edges[len(edges) // 2], edges[-1]})
        pos = sorted({0, nb - 1} | {e + o for e in edges for o in (-1, 0)})
        Kn, Vn = needle_kv(u, len(pos), 56 + b)
        blk = torch.tensor([int(table[b, j // 16]) for j in pos], device=dev)
        slot = torch.tensor([j % 16 for j in pos], device=dev)
        cache.k[blk, :, slot] = torch.from_numpy(Kn).to(dev, torch.bfloat16)
        cache.v[blk, :, slot] = torch.from_numpy(Vn).to(dev, torch.bfloat16)
        plant_queries_(torch, q[b], u)
    out = torch.empty_like(q)
    ws = torch.empty(ws_bytes // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kp = to_np64(cache.k)
    vp = to_np64(cache.v)
    qq = to_np64(q)
    got = to_np64(out)
    for b, nb in enumerate(lens):
        rows = np.array([table[b, j // 16] for j in range(nb)])
        slots = np.arange(nb) % 16
        K = kp[rows, :, slots]
        V = vp[rows, :, slots]
        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], lambda j: K[j], lambda j: V[j], nb, 0, 0, Hkv)
        assert np.max(np.abs(ref)) > 1.0
        every = np.arange(nb)
        # negative controls: drop the block after the middle needle split edge, or the last key
        e = edges[len(edges) // 2]
        for idx in (np.r_[every[:e], every[e + 16:]], every[:-1]):
            assert excess(attend_set(qq[b], K, V, idx, Hkv), ref) > 0


def test_decode_paged_window_with_null_blocks(env):
    # sink + window paged decode where every block below the window edge is null (-1):
    # the kernel must never touch them and must still see the sinks in block 0.
    R, torch, dev = env
    Hkv, n_rep, d, S, W = 8, 4, 128, 4, 100
    Hq = Hkv * n_rep
    lens = [5, 99, 100, 101, 104, 117, 500, 1000]
    B = len(lens)
    max_blocks = 64
    num_blocks = B * max_blocks
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 51)
    for b, n in enumerate(lens):
        edge = max(0, (n - 1) - W + 1)
        for j in range(1, max_blocks):
            if 16 * j + 16 <= edge:
                table[b, j] = -1
    cache = DevPaged(R, torch, dev, torch.bfloat16, B, Hkv, d, S, W, table, num_blocks)
    _fill(torch, cache.k, 52)
    _fill(torch, cache.v, 53)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 54)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kp, vp, qq, got = to_np64(cache.k), to_np64(cache.v), to_np64(q), to_np64(out)
    for b, n in enumerate(lens):
        def kb(j, b=b):
            return kp[table[b, j // 16], :, j % 16]

        def vb(j, b=b):
            return vp[table[b, j // 16], :, j % 16]

        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], kb, vb, n, S, W, Hkv)


def test_decode_ring_random_head(env):
    # a sink + window ring layer (S 4, W 300): full ring (count = W), head at a random offset, long positions
    R, torch, dev = env
    Hkv, n_rep, d, S, W = 8, 4, 128, 4, 300
    Hq = Hkv * n_rep
    B = 5
    cache = DevRing(R, torch, dev, torch.bfloat16, B, Hkv, d, S, W)
    _fill(torch, cache.k, 61)
    _fill(torch, cache.v, 62)
    heads = synth.uniform_ints(B, 0, W, 63)
    lens = [131072, 5000, 305, 304 + 7, 9999]
    cache.head.copy_(torch.from_numpy(heads))
    cache.count.fill_(W)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 64)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    kc, vc, qq, got = to_np64(cache.k), to_np64(cache.v), to_np64(q), to_np64(out)
    for b in range(B):
        ring = O.RingSeq(sinks=S, window=W, head=int(heads[b]), count=W, seq_len=lens[b])
        slots = ring.chronological_slots()
        vis = O.visible_positions(lens[b] - 1, S, W)
        slot_of = dict(zip(vis, slots))
        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], lambda j: kc[b, :, slot_of[j]], lambda j: vc[b, :, slot_of[j]], lens[b], S,
                                 W, Hkv)


# ------------------------------------------------------------------ prefill (bf16 MFMA)

@pytest.mark.parametrize("T,S,W,n_rep,d", [(300, 4, 100, 8, 128), (200, 0, 0, 4, 128), (129, 4, 64, 2, 64),
                                           (77, 3, 1000, 1, 128), (333, 4, 65, 8, 64), (150, 2, 1, 4, 128),
                                           (70, 0, 1, 8, 64)])
def test_prefill_chunk_from_zero(env, T, S, W, n_rep, d):
    R, torch, dev = env
    Hkv = 8 if n_rep > 1 else 4
    Hq = Hkv * n_rep
    cache = DevRing(R, torch, dev, torch.bfloat16, 1, Hkv, d, S, max(W, 1)) if W else \
        DevPaged(R, torch, dev, torch.bfloat16, 1, Hkv, d, S, 0, np.zeros((1, 1), np.int32), 1)
    q = _fill(torch, torch.empty(T, Hq, d, dtype=torch.bfloat16, device=dev), 71)
    k = _fill(torch, torch.empty(T, Hkv, d, dtype=torch.bfloat16, device=dev), 72)
    v = _fill(torch, torch.empty(T, Hkv, d, dtype=torch.bfloat16, device=dev), 73)
    out = torch.empty_like(q)
    R.prefill_attn(q, k, v, T, 0, Hq, cache.desc, 0, 0.0, out)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    qq, kk, vv = to_np64(q), to_np64(k), to_np64(v)
    ref = bf16_attention_ref(to_np64(out), O.prefill_attention, qq, lambda j: kk[j], lambda j: vv[j], 0, S, W, Hkv)


@pytest.mark.parametrize("seq_id", [0, 2])
def test_prefill_with_paged_prefix_equals_one_shot(env, seq_id):
    # chunked prefill into a cached prefix == the same rows of one-shot prefill; the prefix belongs to
    # sequence seq_id of three, the other sequences' blocks hold different (decoy) rows
    R, torch, dev = env
    Hkv, n_rep, d, S, W = 8, 8, 128, 4, 100
    Hq = Hkv * n_rep
    B, T_all, pos0 = 3, 400, 230
    max_blocks = T_all // 16 + 1
    table = synth.block_table_permutation(B, max_blocks, B * max_blocks + 3, 81)
    cache = DevPaged(R, torch, dev, torch.bfloat16, B, Hkv, d, S, W, table, B * max_blocks + 3)
    _fill(torch, cache.k, 85)
    _fill(torch, cache.v, 86)
    q = _fill(torch, torch.empty(T_all, Hq, d, dtype=torch.bfloat16, device=dev), 82)
    k = _fill(torch, torch.empty(T_all, Hkv, d, dtype=torch.bfloat16, device=dev), 83)
    v = _fill(torch, torch.empty(T_all, Hkv, d, dtype=torch.bfloat16, device=dev), 84)
    # place the prefix keys / values in their blocks (plumbing: a torch copy, no kernel of ours)
    for p in range(pos0):
        cache.k[table[seq_id, p // 16], :, p % 16] = k[p]
        cache.v[table[seq_id, p // 16], :, p % 16] = v[p]
    cache.seq_len.fill_(pos0)
    T = T_all - pos0
    out = torch.empty(T, Hq, d, dtype=torch.bfloat16, device=dev)
    R.prefill_attn(q[pos0:], k[pos0:], v[pos0:], T, pos0, Hq, cache.desc, seq_id, 0.0, out)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    qq, kk, vv = to_np64(q), to_np64(k), to_np64(v)
    ref = bf16_attention_ref(to_np64(out), O.prefill_attention, qq[pos0:], lambda j: kk[j], lambda j: vv[j], pos0, S, W, Hkv)


def test_prefill_ring_prefix_lost_is_flagged(env):
    # a ring that no longer holds the chunk's prefix keys: flagged, not silently wrong
    R, torch, dev = env
    Hkv, d, S, W = 4, 64, 2, 8
    cache = DevRing(R, torch, dev, torch.bfloat16, 1, Hkv, d, S, W)
    cache.seq_len.fill_(40)
    cache.count.fill_(W)
    q = torch.zeros(6, 8, d, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(6, Hkv, d, dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    R.prefill_attn(q, kv, kv, 6, 34, 8, cache.desc, 0, 0.0, out)  # needs keys from position 27, ring holds 32..39
    torch.cuda.synchronize()
    assert cache.err.item() & R.DEV_PREFIX_LOST


# ------------------------------------------------------------------ rerotation (fp16 / int8), d 128 / r 64 caches

def _contig_write(R, torch, dev, cfg, table, raw_dev, kv_dtype, L, T, Hkv, d, pos0):
    """Write raw keys for positions pos0.. into a CONTIG cache via apply_append (one call per layer)."""
    if kv_dtype == R.F16:
        kc = torch.zeros(L, T, Hkv, d, dtype=torch.float16, device=dev)
        sc = None
    else:
        kc = torch.zeros(L, T, Hkv, d, dtype=torch.int8, device=dev)
        sc = torch.zeros(L, T, Hkv, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    pos = torch.arange(pos0, pos0 + T, dtype=torch.int32, device=dev)
    for layer in range(L):
        desc = R.kv_cache(R.CONTIG, kv_dtype, Hkv, d, kc[layer], capacity=T, pos0=pos0,
                          k_scale=None if sc is None else sc[layer], err_word=err)
        kin = raw_dev[layer].clone()
        R.apply_append(cfg, table, table.shape[0], None, 0, kin, None, R.F16, T, pos, None, desc)
    torch.cuda.synchronize()
    assert err.item() == 0
    desc_all = R.kv_cache(R.CONTIG, kv_dtype, Hkv, d, kc, capacity=T, pos0=pos0, k_scale=sc, err_word=err)
    return kc, sc, desc_all


def _turn_stats(turned, written, truth, unit):
    """RMS(turned - truth) / RMS(written - truth) and worst |turned - truth| / unit."""
    rt = np.sqrt(np.mean((turned - truth) ** 2))
    rw = np.sqrt(np.mean((written - truth) ** 2))
    worst = float(np.max(np.abs(turned - truth) / unit))
    return rt / rw, worst


@pytest.mark.parametrize("kind", ["f16", "i8"])
@pytest.mark.parametrize("fa,fb", [(1.0, 2.0), (1.5, 2.0), (2.0, 1.0), (1.0, 1.125)])
def test_rerotate_bounds(env, kind, fa, fb):
    # keys written at factor A by apply_append, turned to B, compared with the fp64 key at B;
    # the error of the key written directly at B (as the oracle's storage holds it: fp16 rounding or
    # its row quantiser) is the yardstick (RMS <= 1.6x; worst <= 3 fp16 ulps of the row max, or
    # <= 2 int8 steps of B's row scale).
    R, torch, dev = env
    L, T, Hkv, d, r = 2, 512, 8, 128, 64
    base_kw = dict(rope_theta=5e5, orig_max_pos=262144)
    ca, cb = R.rope_cfg(d, r, yarn_factor=fa, **base_kw), R.rope_cfg(d, r, yarn_factor=fb, **base_kw)
    oa, ob = oracle_cfg(ca), oracle_cfg(cb)
    P = 524288
    ta = _table(R, torch, dev, ca, P)
    kv_dtype = R.F16 if kind == "f16" else R.I8
    for pos0 in (262144 - T // 2, 519999 - T + 1):
        raw = torch.from_numpy(synth.normal((L, T, Hkv, d), 90 + pos0 % 97)).to(dev, torch.float16)
        kc, sc, desc = _contig_write(R, torch, dev, ca, ta, raw, kv_dtype, L, T, Hkv, d, pos0)
        before = kc.clone()
        R.rerotate(ca, cb, desc, L)
        torch.cuda.synchronize()
        rawn = to_np64(raw)
        pos = np.arange(pos0, pos0 + T)
        truth = np.stack([O.rotate_by_angle(rawn[l].reshape(T, Hkv, d), np.outer(pos, O.inv_freq(ob))[:, None, :],
                                            r, True, O.mscale(ob)) for l in range(L)])
        written, unit = oracle_written(kind, truth)
        if kind == "f16":
            turned = to_np64(kc)
            assert np.array_equal(kc[..., r:].cpu().numpy(), before[..., r:].cpu().numpy())  # tail bitwise
        else:
            turned = decode_int8(kc.cpu().numpy(), sc.cpu().numpy())
        ratio, worst = _turn_stats(turned, written, truth, unit)
        assert ratio <= 1.6, ratio
        assert worst <= (3.0 if kind == "f16" else 2.0), worst


def test_rerotate_identity_and_oracle_parity(env):
    R, torch, dev = env
    L, T, Hkv, d, r = 1, 256, 8, 128, 64
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.25, orig_max_pos=262144)
    cb = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.875, orig_max_pos=262144)
    pos0 = 400000
    k = torch.from_numpy(synth.normal((L, T, Hkv, d), 95)).to(dev, torch.float16)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.F16, Hkv, d, k, capacity=T, pos0=pos0, err_word=err)
    before = k.clone()
    R.rerotate(ca, ca, desc, L)  # A -> A: bitwise identity
    torch.cuda.synchronize()
    assert torch.equal(k, before)
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    ref = O.rerotate_rows(to_np64(before[0]).reshape(T, Hkv, d), np.arange(pos0, pos0 + T), oracle_cfg(ca),
                          oracle_cfg(cb))
    got = to_np64(k[0])
    unit = np.maximum(np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64), 1e-6)
    assert np.all(np.abs(got - ref) <= unit)  # within one fp16 ulp of the fp64 turn (fp32 math floor 1e-6)
    # GPT-J pairing and bf16 / fp32 storage through the same kernel family
    for dt, tdt in ((R.BF16, torch.bfloat16), (R.F32, torch.float32)):
        for neox in (True, False):
            a2 = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=262144, neox=neox)
            b2 = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=2.0, orig_max_pos=262144, neox=neox)
            k2 = torch.from_numpy(synth.normal((2, 64, Hkv, d), 96)).to(dev, tdt)
            d2 = R.kv_cache(R.CONTIG, dt, Hkv, d, k2, capacity=64, pos0=300000, err_word=err)
            b4 = to_np64(k2)
            R.rerotate(a2, b2, d2, 2)
            torch.cuda.synchronize()
            ref2 = np.stack([O.rerotate_rows(b4[l], np.arange(300000, 300064), oracle_cfg(a2), oracle_cfg(b2))
                             for l in range(2)])
            if dt == R.F32:
                assert rowwise(to_np64(k2), ref2) <= 1e-5
            else:
                assert_bf16_rounded(to_np64(k2), ref2)


@pytest.mark.parametrize("mode", [0, 1])
def test_rerotate_int8_identity(env, mode):
    # A -> A over quantised keys (the oracle's codes of seeded keys rotated at A: a row's largest code
    # is +-127): codes and scales bit for bit, for the requantising turn (mode 0) and the keep-scale
    # turn (mode 1); the oracle's turn is the identity too
    R, torch, dev = env
    L, T, Hkv, d, r = 2, 96, 8, 128, 64
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.375, orig_max_pos=262144)
    oa = oracle_cfg(ca)
    raw = synth.normal((L, T, Hkv, d), 98)
    angles = np.outer(np.arange(400000, 400000 + T), O.inv_freq(oa))[:, None, :]
    key = np.stack([O.rotate_by_angle(raw[l], angles, r, True, O.mscale(oa)) for l in range(L)])
    c0, s0 = O.quant_int8_rows(key)
    s0 = np.asarray(s0, dtype=np.float32)
    kc, sc = torch.from_numpy(c0).to(dev), torch.from_numpy(s0).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, kc, capacity=T, pos0=400000, k_scale=sc, err_word=err,
                      k_int8_mode=mode)
    R.rerotate(ca, ca, desc, L)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), c0) and np.array_equal(sc.cpu().numpy(), s0)
    pos = np.repeat(np.arange(400000, 400000 + T), Hkv)
    wc, ws_ = O.rerotate_int8_rows(c0[0].reshape(-1, d), s0[0].reshape(-1), pos, oracle_cfg(ca), oracle_cfg(ca))
    assert np.array_equal(wc, c0[0].reshape(-1, d)) and np.array_equal(ws_, s0[0].reshape(-1))


@pytest.mark.parametrize("r,neox", [(128, True), (32, True), (96, True), (64, False), (32, False), (64, True)])
def test_rerotate_int8_shapes_vs_oracle(env, r, neox):
    # every int8 code path (lane-local pairs with 2, 4 or 8 codes per half, GPT-J, and the
    # shuffle fallback for r = 96) against the oracle's dequantise-turn-requantise
    R, torch, dev = env
    L, T, Hkv, d = 2, 48, 4, 128
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=262144, neox=neox)
    cb = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.625, orig_max_pos=262144, neox=neox)
    pos0 = 300007
    g = torch.Generator(device=dev)
    g.manual_seed(97 + r)
    codes = torch.randint(-127, 128, (L, T, Hkv, d), dtype=torch.int8, device=dev, generator=g)
    scale = torch.rand(L, T, Hkv, dtype=torch.float32, device=dev, generator=g) * 0.02 + 0.01
    scale[0, 3, 1] = 0.0  # an all-zero row
    codes[0, 3, 1] = 0
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, codes, capacity=T, pos0=pos0, k_scale=scale, err_word=err)
    c0, s0 = codes.cpu().numpy(), scale.cpu().numpy()
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    c1, s1 = codes.cpu().numpy(), scale.cpu().numpy()
    pos = np.repeat(np.arange(pos0, pos0 + T), Hkv)
    for l in range(L):
        cl, sl = c0[l].reshape(-1, d), s0[l].reshape(-1)
        wc, ws_ = O.rerotate_int8_rows(cl, sl, pos, oracle_cfg(ca), oracle_cfg(cb))
        np.testing.assert_allclose(s1[l].reshape(-1), ws_, rtol=5e-6)
        quot = int8_turn_quotients("i8", cl, sl, pos, oracle_cfg(ca), oracle_cfg(cb), ws_)
        assert_int8_codes_valid(c1[l].reshape(-1, d), wc, quot, EPS_TURN_I8)
    assert s1[0, 3, 1] == 0 and np.all(c1[0, 3, 1] == 0)


# ------------------------------------------------------------------ learned per-head sink logits

@pytest.mark.parametrize("dtype_name,n_rep,d", [("bf16", 4, 128), ("f32", 2, 64), ("bf16", 8, 128)])
def test_decode_learned_sink_logits(env, dtype_name, n_rep, d):
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    Hkv = 4
    Hq = Hkv * n_rep
    lens = [0, 1, 17, 300, 1000]
    B = len(lens)
    max_blocks = 64
    table = synth.block_table_permutation(B, max_blocks, B * max_blocks, 111)
    cache = DevPaged(R, torch, dev, dtype, B, Hkv, d, 4, 200, table, B * max_blocks)
    _fill(torch, cache.k, 112)
    _fill(torch, cache.v, 113)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=dtype, device=dev), 114)
    sinks = torch.from_numpy(synth.normal((Hq,), 115) * 3.0).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4, sink_logits=sinks)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kp, vp, qq, got = to_np64(cache.k), to_np64(cache.v), to_np64(q), to_np64(out)
    sk = sinks.cpu().numpy().astype(np.float64)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
            continue
        args = (qq[b], lambda j: kp[table[b, j // 16], :, j % 16], lambda j: vp[table[b, j // 16], :, j % 16], n,
                4, 200, Hkv)
        if dtype_name == "f32":
            assert rowwise(got[b], O.decode_attention(*args, sink_logits=sk)) <= 1e-5
        else:
            bf16_attention_ref(got[b], O.decode_attention, *args, sink_logits=sk)


@pytest.mark.parametrize("dtype_name,layout,sinks_on", [("f32", "paged", True), ("bf16", "paged", False),
                                                        ("f32", "ring", False), ("bf16", "ring", True)])
def test_decode_direct_plan(env, dtype_name, layout, sinks_on):
    # 32 sequences x 8 KV heads = 256 units with short visible runs: the plan gives each
    # (sequence, KV head) one wide workgroup that writes its output directly (no workspace, no
    # combine); ragged lengths incl. an empty sequence and runs shorter than the workgroup's waves
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    B, Hkv, n_rep, d, S, W = 32, 8, 4, 128, 4, 300
    Hq = Hkv * n_rep
    lens = [0, 1, 2, 5, 17, 100, 303, 304, 305, 1000] + [int(x) for x in synth.uniform_ints(B - 10, 1, 5000, 130)]
    if layout == "paged":
        max_blocks = 5000 // 16 + 2
        table = synth.block_table_permutation(B, max_blocks, B * max_blocks, 131)
        cache = DevPaged(R, torch, dev, dtype, B, Hkv, d, S, W, table, B * max_blocks)
    else:
        cache = DevRing(R, torch, dev, dtype, B, Hkv, d, S, W)
        heads = synth.uniform_ints(B, 0, W, 132)
        # a full ring for sequences past the window, a partly filled one (head = count) below it
        count = [min(max(n - S, 0), W) for n in lens]
        cache.head.copy_(torch.tensor([int(h) if c == W else c % W for h, c in zip(heads, count)], dtype=torch.int32))
        cache.count.copy_(torch.tensor(count, dtype=torch.int32))
    _fill(torch, cache.k, 133)
    _fill(torch, cache.v, 134)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    assert R.decode_workspace_size(B, Hq, cache.desc) == 0  # the direct plan needs no partials
    q = _fill(torch, torch.empty(B, Hq, d, dtype=dtype, device=dev), 135)
    sinks = torch.from_numpy(synth.normal((Hq,), 136) * 3.0).to(dev) if sinks_on else None
    out = torch.full_like(q, float("nan"))
    ws = torch.empty(1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, 4, sink_logits=sinks)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kc, vc, qq, got = to_np64(cache.k), to_np64(cache.v), to_np64(q), to_np64(out)
    sk = sinks.cpu().numpy().astype(np.float64) if sinks_on else None
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(got[b] == 0)
            continue
        if layout == "paged":
            def kf(j, b=b):
                return kc[table[b, j // 16], :, j % 16]

            def vf(j, b=b):
                return vc[table[b, j // 16], :, j % 16]
        else:
            ring = O.RingSeq(sinks=S, window=W, head=int(cache.head[b].item()), count=count[b], seq_len=n)
            slot_of = dict(zip(O.visible_positions(n - 1, S, W), ring.chronological_slots()))

            def kf(j, b=b, slot_of=slot_of):
                return kc[b, :, slot_of[j]]

            def vf(j, b=b, slot_of=slot_of):
                return vc[b, :, slot_of[j]]
        if dtype_name == "f32":
            assert rowwise(got[b], O.decode_attention(qq[b], kf, vf, n, S, W, Hkv, sink_logits=sk)) <= 1e-5, b
        else:
            bf16_attention_ref(got[b], O.decode_attention, qq[b], kf, vf, n, S, W, Hkv, sink_logits=sk)


@pytest.mark.parametrize("dtype_name", ["bf16", "f32"])
def test_prefill_learned_sink_logits(env, dtype_name):
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    T, Hkv, n_rep, d, S, W = 150, 4, 4, 64, 4, 40
    Hq = Hkv * n_rep
    cache = DevRing(R, torch, dev, dtype, 1, Hkv, d, S, W)
    q = _fill(torch, torch.empty(T, Hq, d, dtype=dtype, device=dev), 121)
    k = _fill(torch, torch.empty(T, Hkv, d, dtype=dtype, device=dev), 122)
    v = _fill(torch, torch.empty(T, Hkv, d, dtype=dtype, device=dev), 123)
    sinks = torch.from_numpy(synth.normal((Hq,), 124) * 3.0).to(dev)
    out = torch.empty_like(q)
    R.prefill_attn(q, k, v, T, 0, Hq, cache.desc, 0, 0.0, out, sink_logits=sinks)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    qq, kk, vv = to_np64(q), to_np64(k), to_np64(v)
    args = (qq, lambda j: kk[j], lambda j: vv[j], 0, S, W, Hkv)
    sl = sinks.cpu().numpy().astype(np.float64)
    if dtype_name == "f32":
        assert rowwise(to_np64(out), O.prefill_attention(*args, sink_logits=sl)) <= 1e-5
    else:
        bf16_attention_ref(to_np64(out), O.prefill_attention, *args, sink_logits=sl)


# ------------------------------------------------------------------ local-position key shift

@pytest.mark.parametrize("dtype_name,r,neox,delta", [("bf16", 64, True, -1), ("f32", 32, True, 5),
                                                      ("f32", 64, False, -3), ("bf16", 48, True, -1)])
def test_shift_keys_ring(env, dtype_name, r, neox, delta):
    # only valid ring slots move (by delta positions); sinks, empty slots and values stay bitwise
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    B, Hkv, d, S, W = 3, 4, 64, 4, 12
    cfg = R.rope_cfg(d, r, rope_theta=1e4, neox=neox)
    cache = DevRing(R, torch, dev, dtype, B, Hkv, d, S, W)
    _fill(torch, cache.k, 131)
    _fill(torch, cache.v, 132)
    heads, counts, lens = [5, 0, 7], [5, 12, 12], [9, 100, 16]
    cache.head.copy_(torch.tensor(heads, dtype=torch.int32))
    cache.count.copy_(torch.tensor(counts, dtype=torch.int32))
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    k0, v0 = cache.k.clone(), cache.v.clone()
    R.shift_keys(cfg, cache.desc, delta)
    torch.cuda.synchronize()
    assert torch.equal(cache.v, v0)
    k0n, k1n = to_np64(k0), to_np64(cache.k)
    ocfg = oracle_cfg(cfg)
    for b in range(B):
        ring = O.RingSeq(sinks=S, window=W, head=heads[b], count=counts[b], seq_len=lens[b])
        live = set(ring.chronological_slots()[min(S, lens[b]):])
        for slot in range(S + W):
            if slot in live:
                ref = O.shift_keys(k0n[b, :, slot], delta, ocfg)
                if dtype_name == "f32":
                    assert normwise(k1n[b, :, slot], ref) <= 1e-5
                else:
                    assert_bf16_rounded(k1n[b, :, slot], ref)
                assert np.array_equal(k1n[b, :, slot, r:], k0n[b, :, slot, r:])
            else:
                assert np.array_equal(k1n[b, :, slot], k0n[b, :, slot])


def test_shift_keys_contig_f16_roundtrip(env):
    # shifting by +7 then -7 returns the keys within fp16 rounding; every row of every layer moves
    R, torch, dev = env
    L, T, Hkv, d, r = 2, 40, 4, 128, 64
    cfg = R.rope_cfg(d, r, rope_theta=5e5)
    k = _fill(torch, torch.empty(L, T, Hkv, d, dtype=torch.float16, device=dev), 141)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.F16, Hkv, d, k, capacity=T, err_word=err)
    k0 = to_np64(k)
    R.shift_keys(cfg, desc, 7, L)
    torch.cuda.synchronize()
    ref = O.shift_keys(k0.reshape(-1, d), 7, oracle_cfg(cfg)).reshape(k0.shape)
    unit = np.maximum(np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64), 1e-6)
    assert np.all(np.abs(to_np64(k) - ref) <= unit)
    R.shift_keys(cfg, desc, -7, L)
    torch.cuda.synchronize()
    assert np.max(np.abs(to_np64(k) - k0)) < 1e-2


def test_rerotate_across_schemes(env):
    # a key written under one scheme is turned to another: PI -> Llama-3 -> NTK, fp32 cache
    R, torch, dev = env
    T, Hkv, d, r = 64, 4, 128, 128
    cfgs = [R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=4.0, rope_type=1),
            R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=8.0, rope_type=4, orig_max_pos=8192),
            R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=2.0, rope_type=2)]
    k = _fill(torch, torch.empty(1, T, Hkv, d, dtype=torch.float32, device=dev), 151)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.F32, Hkv, d, k, capacity=T, pos0=100000, err_word=err)
    cur = to_np64(k[0])
    pos = np.arange(100000, 100000 + T)
    for a_, b_ in zip(cfgs[:-1], cfgs[1:]):
        R.rerotate(a_, b_, desc, 1)
        torch.cuda.synchronize()
        cur = O.rerotate_rows(cur, pos, oracle_cfg(a_), oracle_cfg(b_))
        assert rowwise(to_np64(k[0]), cur) <= 1e-5


# ------------------------------------------------------------------ an explicit softmax scale

@pytest.mark.parametrize("dtype_name", ["f32", "bf16", "i8", "fp8"])
def test_decode_and_prefill_explicit_scale(env, dtype_name):
    # scale != 0 replaces 1/sqrt(d) in the decode (fp32, bf16 and int8 caches) and the prefill (fp32,
    # bf16): a sharper 0.3 and a flatter 0.02 against the oracle at the same scale
    R, torch, dev = env
    B, Hkv, n_rep, d, S, W = 3, 2, 4, 64, 4, 40
    Hq = Hkv * n_rep
    lens = [5, 60, 130]
    table = synth.block_table_permutation(B, 16, B * 16, 170)
    store = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "fp8": "fp8"}[dtype_name]
    cache = DevPaged(R, torch, dev, store, B, Hkv, d, S, W, table, B * 16)
    if dtype_name == "fp8":
        # finite E4M3 bytes (the two NaN codes 0x7f / 0xff replaced by 0), row scales U(2/448, 3.5/448)
        g = torch.Generator(device=dev)
        g.manual_seed(171)
        for buf, sc in ((cache.k, cache.k_scale), (cache.v, cache.v_scale)):
            codes = torch.randint(0, 256, tuple(buf.shape), dtype=torch.int32, device=dev, generator=g)
            codes[(codes & 0x7F) == 0x7F] = 0
            buf.copy_(codes.to(torch.uint8))
            sc.copy_(torch.rand(tuple(sc.shape), device=dev, generator=g) * (1.5 / 448) + 2.0 / 448)
        kp = decode_e4m3(cache.k.cpu().numpy()) * cache.k_scale.cpu().numpy().astype(np.float64)[..., None]
        vp = decode_e4m3(cache.v.cpu().numpy()) * cache.v_scale.cpu().numpy().astype(np.float64)[..., None]
        qdt = torch.bfloat16
    elif dtype_name == "i8":
        g = torch.Generator(device=dev)
        g.manual_seed(171)
        for buf, sc in ((cache.k, cache.k_scale), (cache.v, cache.v_scale)):
            buf.copy_(torch.randint(-127, 128, tuple(buf.shape), dtype=torch.int8, device=dev, generator=g))
            sc.copy_(torch.rand(tuple(sc.shape), device=dev, generator=g) * 0.02 + 0.01)
        kp = decode_int8(cache.k.cpu().numpy(), cache.k_scale.cpu().numpy())
        vp = decode_int8(cache.v.cpu().numpy(), cache.v_scale.cpu().numpy())
        qdt = torch.bfloat16
    else:
        _fill(torch, cache.k, 172)
        _fill(torch, cache.v, 173)
        kp, vp = to_np64(cache.k), to_np64(cache.v)
        qdt = store
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=qdt, device=dev), 174)
    qq = to_np64(q)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    for scale in (0.3, 0.02):
        R.decode_attn(q, B, Hq, cache.desc, scale, out, ws, ws.numel() * 4)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        got = to_np64(out)
        for b, n in enumerate(lens):
            args = (qq[b], lambda j, b=b: kp[table[b, j // 16], :, j % 16], lambda j, b=b: vp[table[b, j // 16], :, j % 16],
                    n, S, W, Hkv)
            if dtype_name == "f32":
                assert rowwise(got[b], O.decode_attention(*args, scale=scale)) <= 1e-5
            else:
                bf16_attention_ref(got[b], O.decode_attention, *args, scale=scale)
    if dtype_name in ("i8", "fp8"):
        return
    # the prefill of a 20-token chunk from position 0 (no prefix), same scales
    T = 20
    pq = _fill(torch, torch.empty(T, Hq, d, dtype=store, device=dev), 175)
    pk = _fill(torch, torch.empty(T, Hkv, d, dtype=store, device=dev), 176)
    pv = _fill(torch, torch.empty(T, Hkv, d, dtype=store, device=dev), 177)
    po = torch.empty_like(pq)
    Q, K, V = to_np64(pq), to_np64(pk), to_np64(pv)
    for scale in (0.3, 0.02):
        R.prefill_attn(pq, pk, pv, T, 0, Hq, cache.desc, 0, scale, po)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        got = to_np64(po)
        args = (Q, lambda j: K[j], lambda j: V[j], 0, S, W, Hkv)
        want = O.prefill_attention(*args, scale=scale)
        if dtype_name == "f32":
            assert rowwise(got, want) <= 1e-5
        else:
            for t in range(T):
                bf16_attention_ref(got[t], O.decode_attention, Q[t], lambda j: K[j], lambda j: V[j], t + 1, S, W, Hkv,
                                   scale=scale)


def test_decode_first_sequences_of_a_larger_cache(env):
    # batch 2 over a cache of 3 sequences: rows 0 and 1 of q / out only, against the oracle
    R, torch, dev = env
    Bc, B, Hkv, n_rep, d, S, W = 3, 2, 2, 4, 128, 4, 50
    Hq = Hkv * n_rep
    table = synth.block_table_permutation(Bc, 8, Bc * 8, 180)
    cache = DevPaged(R, torch, dev, torch.float32, Bc, Hkv, d, S, W, table, Bc * 8)
    _fill(torch, cache.k, 181)
    _fill(torch, cache.v, 182)
    lens = [70, 33, 100]
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = _fill(torch, torch.empty(B, Hq, d, dtype=torch.float32, device=dev), 183)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kp, vp, qq, got = to_np64(cache.k), to_np64(cache.v), to_np64(q), to_np64(out)
    for b in range(B):
        want = O.decode_attention(qq[b], lambda j: kp[table[b, j // 16], :, j % 16],
                                  lambda j: vp[table[b, j // 16], :, j % 16], lens[b], S, W, Hkv)
        assert rowwise(got[b], want) <= 1e-5


def test_prefill_ring_prefix_of_sequence_one(env):
    # a 6-token chunk at pos0 30 over the ring prefix of sequence 1 of two (sinks 2, window 20, head at
    # 7, full ring): the ring rows are placed where the oracle's ring model puts each position, the
    # other sequence holds decoys; fp32, against the oracle
    R, torch, dev = env
    B, Hkv, n_rep, d, S, W = 2, 2, 4, 64, 2, 20
    Hq = Hkv * n_rep
    pos0, T, head = 30, 6, 7
    cache = DevRing(R, torch, dev, torch.float32, B, Hkv, d, S, W)
    _fill(torch, cache.k, 190)
    _fill(torch, cache.v, 191)
    prefix_k = synth.normal((pos0, Hkv, d), 192)
    prefix_v = synth.normal((pos0, Hkv, d), 193)
    ring = O.RingSeq(sinks=S, window=W, head=head, count=W, seq_len=pos0)
    slot_of = dict(zip(O.visible_positions(pos0 - 1, S, W), ring.chronological_slots()))
    for p, slot in slot_of.items():  # plumbing: torch copies into sequence 1's slots
        cache.k[1, :, slot] = torch.from_numpy(prefix_k[p]).to(dev)
        cache.v[1, :, slot] = torch.from_numpy(prefix_v[p]).to(dev)
    cache.head.copy_(torch.tensor([0, head], dtype=torch.int32))
    cache.count.copy_(torch.tensor([W, W], dtype=torch.int32))
    cache.seq_len.copy_(torch.tensor([pos0, pos0], dtype=torch.int32))
    q = _fill(torch, torch.empty(T, Hq, d, dtype=torch.float32, device=dev), 194)
    k = _fill(torch, torch.empty(T, Hkv, d, dtype=torch.float32, device=dev), 195)
    v = _fill(torch, torch.empty(T, Hkv, d, dtype=torch.float32, device=dev), 196)
    out = torch.empty_like(q)
    R.prefill_attn(q, k, v, T, pos0, Hq, cache.desc, 1, 0.0, out)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kk, vv = to_np64(k), to_np64(v)

    def kf(j):
        return kk[j - pos0] if j >= pos0 else prefix_k[j].astype(np.float64)

    def vf(j):
        return vv[j - pos0] if j >= pos0 else prefix_v[j].astype(np.float64)

    want = O.prefill_attention(to_np64(q), kf, vf, pos0, S, W, Hkv)
    assert rowwise(to_np64(out), want) <= 1e-5
