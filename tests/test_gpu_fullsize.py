"""Parity at the benchmark's full sizes, in the launch configuration bench.py times.

Sampled outputs are checked one by one against the fp64 oracle: whole
sequences for decode, single query rows for prefill, random rows for the
re-rotation.  Inputs are the seeded device buffers of the workload (filled by
torch's generator), read back to the host for the oracle.  The attention
checks plant needle keys (tests/gpu_util.py) at sinks, window edges, 16-key
block and split boundaries, and show with negative controls that the oracle
over a wrong visible set fails the same tolerance.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (bf16_attention_ref, bf16_round, EPS_APPEND_FP8, EPS_APPEND_I8, EPS_TURN_HADAMARD, EPS_TURN_I8, assert_bf16_close, assert_bf16_rounded,
                            assert_fp8_codes_valid, assert_int8_codes_valid, attend_set, check_keep_scale_rows,
                            excess, int8_turn_quotients, needle_dirs, needle_kv, oracle_cfg, plant_queries_,
                            to_np64, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R
    from sliding_window_kv_amd import workloads as WL

    return R, torch, dev, WL


def _split_keys(R, wl, max_tiles):
    """Keys per split of the decode plan (read back from the workspace size).  A plan without
    partials (one workgroup per sequence and KV head, its waves taking tiles in turn) has no split
    edge: a tile edge in the middle of the run stands in for it."""
    n_rep = wl.Hq // wl.Hkv
    splits = wl.ws_bytes // (wl.B * wl.Hkv * n_rep * (wl.d + 2) * 4)
    if splits == 0:
        return 16 * (max_tiles // 2)
    return 16 * ((max_tiles + splits - 1) // splits)


def _paged_full_needles(R, torch, wl, seqs, seed, sink_logits=None):
    """Full-attention paged decode with needles, in the workload's own launch: needles at the first
    and last keys, 16-key block edges, split edges and mid-sequence; negative controls drop key 0,
    the last key, the block after the first split edge, or shift the set by 64.  With sink_logits
    (device fp32 [Hq]) the decode takes them, and the negative control is the oracle without them."""
    n, d, Hkv = wl.ctx, wl.d, wl.Hkv
    sp = _split_keys(R, wl, wl.max_blocks)
    pos = sorted({0, 15, 16, sp - 1, sp, n // 2 - 1, n // 2, n - sp - 1, n - sp, n - 2, n - 1})
    u = needle_dirs(Hkv, d, seed)
    Kn, Vn = needle_kv(u, len(pos), seed + 1)
    # fresh seeded queries (a step before this one rotated the workload's queries in place); the last
    # key, the one a step appends, is among the planted rows
    synth.device_normal_(wl.q, seed + 2)
    planted = [(wl.k, Kn, wl.k_scale), (wl.v, Vn, wl.v_scale)]
    if wl.kv8:  # 8-bit caches: the needle rows as the oracle quantises them (codes + row scales)
        quant = O.quant_int8_rows if wl.kv8 == "i8" else O.quant_fp8_rows
        planted = [(buf, quant(rows), sc) for buf, rows, sc in planted]
    for b in seqs:
        blk = torch.tensor([int(wl.table_host[b, j // 16]) for j in pos], device=wl.k.device)
        slot = torch.tensor([j % 16 for j in pos], device=wl.k.device)
        for buf, rows, sc in planted:
            if wl.kv8:
                codes, scale = rows
                buf[blk, :, slot] = torch.from_numpy(codes.view(np.uint8)).to(buf.device).view(buf.dtype)
                sc[blk, :, slot] = torch.from_numpy(scale).to(buf.device)
            else:
                buf[blk, :, slot] = torch.from_numpy(rows).to(buf.device, buf.dtype)
        plant_queries_(torch, wl.q[b], u)
    if sink_logits is None:
        wl.decode()
    else:
        R.decode_attn(wl.q, wl.B, wl.Hq, wl.desc, 0.0, wl.out, wl.ws, wl.ws_bytes, sink_logits=sink_logits)
    torch.cuda.synchronize()
    assert wl.err.item() == 0
    out, q = to_np64(wl.out), to_np64(wl.q)
    sk = None if sink_logits is None else sink_logits.cpu().numpy().astype(np.float64)
    for b in seqs:
        if wl.kv8:
            dequant = O.dequant_int8_rows if wl.kv8 == "i8" else O.dequant_fp8_rows
            kc, ks, vc, vs = wl.codes_of(b)
            K, V = dequant(kc, ks), dequant(vc, vs)
        else:
            K, V = wl.kv_of(b)
        ref = bf16_attention_ref(out[b], O.decode_attention, q[b], lambda j: K[j], lambda j: V[j], n, 0, 0, Hkv,
                                 sink_logits=sk)
        assert np.max(np.abs(ref)) > 1.0  # the needles carry the output
        if sk is not None:
            assert excess(O.decode_attention(q[b], lambda j: K[j], lambda j: V[j], n, 0, 0, Hkv), ref) > 0
            continue
        every = np.arange(n)
        wrong = [every[1:], every[:-1], np.r_[every[:sp], every[sp + 16:]], every[:-64]]
        for idx in wrong:
            assert excess(attend_set(q[b], K, V, idx, Hkv), ref) > 0


def test_paged_decode_b64_ctx32768(env):
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev)
    # the appended token's rope + write, checked against the oracle for two sequences
    q_raw = to_np64(wl.q)
    k_raw = to_np64(wl.k_new)
    v_raw = to_np64(wl.v_new)
    wl.step()
    torch.cuda.synchronize()
    assert wl.err.item() == 0
    assert wl.seq_len.cpu().tolist() == [wl.ctx] * wl.B
    otab_row = O.build_table(oracle_cfg(wl.cfg), wl.ctx)
    q_rot = to_np64(wl.q)
    out = to_np64(wl.out)
    for b in (0, 37, 63):
        p = wl.ctx - 1
        want_q = O.rope_apply(q_raw[b:b + 1], [p], otab_row, wl.d, True)[0]
        assert_bf16_rounded(q_rot[b], want_q)
        k, v = wl.kv_of(b)
        want_k = O.rope_apply(k_raw[b:b + 1], [p], otab_row, wl.d, True)[0]
        assert_bf16_rounded(k[p], want_k)
        assert np.array_equal(v[p], v_raw[b])
        # the attention over the oracle's own values: its rotated q and new key as bf16 holds them,
        # the seeded new value, the seeded cache rows before them
        k_ref, v_ref = k.copy(), v.copy()
        k_ref[p], v_ref[p] = bf16_round(want_k), v_raw[b]
        bf16_attention_ref(out[b], O.decode_attention, bf16_round(want_q), lambda j: k_ref[j], lambda j: v_ref[j],
                           wl.ctx, 0, 0, wl.Hkv)
    # needles: the same layer decoded again with planted keys and queries
    _paged_full_needles(R, torch, wl, (0, 37, 63), 2100)


def test_paged_decode_b64_ctx32768_learned_sinks(env):
    # the learned-sink decode row's launch: the batch-64 x 32768 paged decode with one sink logit per query head,
    # after a step; needles score about 16, and the sink logits run from 14 (a few per cent of the
    # needles' weight) to 22 (most of it), so the oracle without them fails the same tolerance
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev)
    wl.step()
    torch.cuda.synchronize()
    sinks = torch.linspace(14.0, 22.0, wl.Hq, device=dev)
    _paged_full_needles(R, torch, wl, (0, 37, 63), 2200, sink_logits=sinks)


def test_decode_step_graph_b64_ctx32768(env):
    # the headline step as bench.py times it: seq_len reset, rope + append and the split-K decode
    # captured in a HIP graph; every replay (eager work and synchronisations between them) gives the
    # eager step's outputs and rotated q bit for bit, and the eager step matches the oracle
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev)
    q0, k0, v0 = wl.q.clone(), wl.k_new.clone(), wl.v_new.clone()

    def step():
        wl.q.copy_(q0)
        wl.k_new.copy_(k0)
        wl.v_new.copy_(v0)
        wl.step()

    step()
    torch.cuda.synchronize()
    assert wl.err.item() == 0
    eager_out, eager_q = wl.out.clone(), wl.q.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        wl.out.fill_(float("nan"))
        torch.randn(1 << 20, device=dev).mul_(2.0).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        assert wl.err.item() == 0
        assert torch.equal(wl.out, eager_out), f"replay {rep} differs from the eager step"
        assert torch.equal(wl.q, eager_q)
    p = wl.ctx - 1
    otab = O.build_table(oracle_cfg(wl.cfg), wl.ctx)
    b = 11
    want_q = O.rope_apply(to_np64(q0)[b:b + 1], [p], otab, wl.d, True)[0]
    want_k = O.rope_apply(to_np64(k0)[b:b + 1], [p], otab, wl.d, True)[0]
    assert_bf16_rounded(to_np64(eager_q)[b], want_q)
    k, v = wl.kv_of(b)
    assert_bf16_rounded(k[p], want_k)
    k[p], v[p] = bf16_round(want_k), to_np64(v0)[b]
    bf16_attention_ref(to_np64(eager_out)[b], O.decode_attention, bf16_round(want_q), lambda j: k[j], lambda j: v[j],
                       wl.ctx, 0, 0, wl.Hkv)


def test_paged_decode_b32_ctx131072(env):
    # the full-attention layer of the windowed 128k stack: 32 sequences of 131072 keys, 8192 blocks each
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev, B=32, ctx=131072, seed=3100)
    wl.seq_len.fill_(wl.ctx)
    _paged_full_needles(R, torch, wl, (0, 31), 3150)


@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_paged_decode_b64_ctx32768_8bit(env, kind):
    # the same step over an 8-bit cache (int8 or E4M3 codes + per-row scales): the appended
    # token quantised, decode over codes x scales
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev, kv8=kind)
    quant = O.quant_int8_rows if kind == "i8" else O.quant_fp8_rows
    dequant = O.dequant_int8_rows if kind == "i8" else O.dequant_fp8_rows
    q_raw, k_raw, v_raw = to_np64(wl.q), to_np64(wl.k_new), to_np64(wl.v_new)
    wl.step()
    torch.cuda.synchronize()
    assert wl.err.item() == 0
    otab_row = O.build_table(oracle_cfg(wl.cfg), wl.ctx)
    q_rot = to_np64(wl.q)
    out = to_np64(wl.out)
    p = wl.ctx - 1
    for b in (0, 41, 63):
        kc, ks, vc, vs = wl.codes_of(b)
        want_k = O.rope_apply(k_raw[b:b + 1], [p], otab_row, wl.d, True)[0]
        wk_codes, wk_scale = quant(want_k)
        # a rotated key may round to the neighbouring code (float32 vs fp64 rotation), only at an edge
        quot = O.row_quotients(want_k, wk_scale)
        if kind == "i8":
            assert_int8_codes_valid(kc[p], wk_codes, quot, EPS_APPEND_I8)
        else:
            assert_fp8_codes_valid(kc[p], wk_codes, quot, EPS_APPEND_FP8)
        np.testing.assert_allclose(ks[p], wk_scale, rtol=1e-6, atol=0)
        wv_codes, wv_scale = quant(v_raw[b])
        assert np.array_equal(vc[p].view(np.uint8), wv_codes.view(np.uint8)) and np.array_equal(vs[p], wv_scale)
        # the attention over the oracle's own values: its rotated q as bf16, its codes of the new
        # key and value, the seeded code rows before them
        kc_ref, ks_ref, vc_ref, vs_ref = kc.copy(), ks.copy(), vc.copy(), vs.copy()
        kc_ref[p], ks_ref[p] = wk_codes, wk_scale
        vc_ref[p], vs_ref[p] = wv_codes, wv_scale
        k = dequant(kc_ref, ks_ref)
        v = dequant(vc_ref, vs_ref)
        want_q = O.rope_apply(q_raw[b:b + 1], [p], otab_row, wl.d, True)[0]
        assert_bf16_rounded(q_rot[b], want_q)
        bf16_attention_ref(out[b], O.decode_attention, bf16_round(want_q), lambda j: k[j], lambda j: v[j], wl.ctx, 0,
                           0, wl.Hkv)
    _paged_full_needles(R, torch, wl, (0, 63), 2200 + len(kind))


def test_ring_decode_128k(env):
    # one ring layer (head at a random offset, full ring): needles in the sink slots, the first and
    # last ring slots, tile edges and the split edge; every ring slot is visible, so the negative
    # controls drop the sinks, the tile after the split edge or the last slot
    R, torch, dev, WL = env
    r = WL.RingDecode(R, torch, dev)
    C = r.C
    sp = _split_keys(R, r, (C + 15) // 16)
    slots = sorted({0, 3, 4, 15, 16, sp - 1, sp, 1000, 1001, C - 17, C - 16, C - 1})
    u = needle_dirs(r.Hkv, r.d, 3050)
    Kn, Vn = needle_kv(u, len(slots), 3051)
    seqs = (0, 17, 31)
    sl = torch.tensor(slots, device=r.k.device)
    for b in seqs:
        r.k[b][:, sl] = torch.from_numpy(Kn.transpose(1, 0, 2).copy()).to(r.k.device, r.k.dtype)
        r.v[b][:, sl] = torch.from_numpy(Vn.transpose(1, 0, 2).copy()).to(r.k.device, r.k.dtype)
        plant_queries_(torch, r.q[b], u)
    r.decode()
    torch.cuda.synchronize()
    assert r.err.item() == 0
    heads = r.head.cpu().numpy()
    out = to_np64(r.out)
    q = to_np64(r.q)
    for b in seqs:
        kc = to_np64(r.k[b])
        vc = to_np64(r.v[b])
        ring = O.RingSeq(sinks=r.S, window=r.W, head=int(heads[b]), count=r.W, seq_len=r.n)
        slot_of = dict(zip(O.visible_positions(r.n - 1, r.S, r.W), ring.chronological_slots()))
        ref = bf16_attention_ref(out[b], O.decode_attention, q[b], lambda j: kc[:, slot_of[j]], lambda j: vc[:, slot_of[j]], r.n, r.S, r.W,
                                 r.Hkv)
        assert np.max(np.abs(ref)) > 1.0
        K, V = kc.transpose(1, 0, 2), vc.transpose(1, 0, 2)  # by slot
        every = np.arange(C)
        for idx in (every[r.S:], np.r_[every[:sp], every[sp + 16:]], every[:-1]):
            assert excess(attend_set(q[b], K, V, idx, r.Hkv), ref) > 0


def test_shift_keys_ring_w4096_b32(env):
    # the local-shift row: one ring layer (32 sequences, 8 KV heads, S 4 + W 4096, full ring, head at
    # a seeded offset) moved back by one position; sampled rows against the oracle's shift (one bf16
    # rounding), sink rows and all values bitwise unchanged
    R, torch, dev, WL = env
    r = WL.RingDecode(R, torch, dev)
    cfg = R.rope_cfg(r.d, r.d, rope_theta=5e5)
    rng = synth.rng(3300)
    n = 40
    bs = rng.integers(0, r.B, n)
    hs = rng.integers(0, r.Hkv, n)
    slots = rng.integers(0, r.C, n)
    slots[:6] = [0, r.S - 1, r.S, r.S + 1, r.C - 2, r.C - 1]  # sinks, both ends of the ring
    idx = (torch.from_numpy(bs).to(dev), torch.from_numpy(hs).to(dev), torch.from_numpy(slots).to(dev))
    before = to_np64(r.k[idx])
    v0 = r.v.clone()
    R.shift_keys(cfg, r.desc, -1)
    torch.cuda.synchronize()
    after = to_np64(r.k[idx])
    assert torch.equal(r.v, v0)
    sink = slots < r.S
    assert np.array_equal(after[sink], before[sink])
    want = O.shift_keys(before[~sink], -1, oracle_cfg(cfg))
    assert_bf16_rounded(after[~sink], want)
    assert not np.array_equal(after[~sink], before[~sink])


def test_windowed_paged_decode_b256(env):
    # 256 sequences of the sink + window layer, lengths in [1k, 128k], blocks outside sinks and window
    # null: needles at the sinks, at key 4 (inside the pinned sink block, invisible), at the key just
    # outside the window (its block is live when it shares a block with the first visible key), the
    # first visible key, block edges in the window and the newest key
    R, torch, dev, WL = env
    wd = WL.WindowedPagedDecode(R, torch, dev)
    S, W = wd.S, wd.W
    shares = [b for b in range(wd.B) if (int(wd.lens[b]) - W) % 16 != 0 and int(wd.lens[b]) > W + 40]
    seqs = sorted({0, 100, 255, shares[0], shares[1]})
    u = needle_dirs(wd.Hkv, wd.d, 5050)
    planted = {}
    for i, b in enumerate(seqs):
        n = int(wd.lens[b])
        p = n - 1
        cand = {0, 3, 4, 5, p - W, p - W + 1, p - W + 16 - (p - W + 1) % 16, p - 16, p - 1, p}
        row = wd.table_host[b]
        pos = sorted(j for j in cand if 0 <= j <= p and row[j // 16] >= 0)
        Kn, Vn = needle_kv(u, len(pos), 5051 + i)
        blk = torch.tensor([int(row[j // 16]) for j in pos], device=wd.k.device)
        slot = torch.tensor([j % 16 for j in pos], device=wd.k.device)
        wd.k[blk, :, slot] = torch.from_numpy(Kn).to(wd.k.device, wd.k.dtype)
        wd.v[blk, :, slot] = torch.from_numpy(Vn).to(wd.k.device, wd.k.dtype)
        plant_queries_(torch, wd.q[b], u)
        planted[b] = pos
    wd.decode()
    torch.cuda.synchronize()
    assert wd.err.item() == 0
    out, q = to_np64(wd.out), to_np64(wd.q)
    kp, vp = wd.k, wd.v
    n_outside = checked = 0
    for b in seqs:
        n = int(wd.lens[b])
        p = n - 1
        row = wd.table_host[b]
        live = sorted({int(x) for x in row if x >= 0})
        idx = torch.tensor(live, dtype=torch.long, device=kp.device)
        kb = dict(zip(live, to_np64(kp[idx])))
        vb = dict(zip(live, to_np64(vp[idx])))

        def kf(j, row=row):
            return kb[int(row[j // 16])][:, j % 16]

        def vf(j, row=row):
            return vb[int(row[j // 16])][:, j % 16]

        ref = bf16_attention_ref(out[b], O.decode_attention, q[b], kf, vf, n, S, W, wd.Hkv)
        assert np.max(np.abs(ref)) > 1.0
        # negative controls: the oracle's visible set with no sinks, one sink more (admits key 4), the
        # window one shorter (drops the first visible key) and, when its block is live, one longer;
        # each one that changes which needles are visible must fail the tolerance
        needles = set(planted[b])
        vis = set(O.visible_positions(p, S, W)) & needles
        controls = [(0, W), (S + 1, W), (S, W - 1)]
        if p >= W and row[(p - W) // 16] >= 0:
            controls.append((S, W + 1))
            n_outside += 1
        for s2, w2 in controls:
            if set(O.visible_positions(p, s2, w2)) & needles != vis:
                bad = O.decode_attention(q[b], kf, vf, n, s2, w2, wd.Hkv)
                assert excess(bad, ref) > 0, (b, s2, w2)
                checked += 1
    assert n_outside >= 2  # the key just outside the window was planted in a live block
    assert checked >= 10


def test_prefill_t8192_sampled_rows(env):
    # the 8192-token chunk over sink(4) + window(4096): the sampled rows get planted query components,
    # and needle keys sit at the sinks, keys 4 and 5 (the first to leave the window, at rows 4100 and
    # 4101), 64-key tile edges, the window edges of the last row (4095 | 4096) and the newest keys
    R, torch, dev, WL = env
    pf = WL.Prefill(R, torch, dev)
    S, W = pf.S, pf.W
    rows = (0, 1, 15, 16, 63, 64, 4095, 4096, 4097, 4099, 4100, 4101, 5000, 8190, 8191)
    keys = [0, 3, 4, 5, 63, 64, 127, 128, 904, 4095, 4096, 4097, 8190, 8191]
    u = needle_dirs(pf.Hkv, pf.d, 6050)
    Kn, Vn = needle_kv(u, len(keys), 6051)
    kk = torch.tensor(keys, device=pf.k.device)
    pf.k[kk] = torch.from_numpy(Kn).to(pf.k.device, pf.k.dtype)
    pf.v[kk] = torch.from_numpy(Vn).to(pf.k.device, pf.k.dtype)
    for t in rows:
        plant_queries_(torch, pf.q[t], u)
    pf.run()
    torch.cuda.synchronize()
    assert pf.int_state[3].item() == 0
    q, k, v, out = to_np64(pf.q), to_np64(pf.k), to_np64(pf.v), to_np64(pf.out)
    needles = set(keys)
    checked = 0
    for t in rows:
        ref = bf16_attention_ref(out[t], O.decode_attention, q[t], lambda j: k[j], lambda j: v[j], t + 1, S, W, pf.Hkv)
        assert np.max(np.abs(ref)) > 1.0
        vis = set(O.visible_positions(t, S, W))
        for s2, w2 in ((0, W), (S + 1, W), (S, W - 1), (S, W + 1)):
            if set(O.visible_positions(t, s2, w2)) & needles != vis & needles:
                bad = O.decode_attention(q[t], lambda j: k[j], lambda j: v[j], t + 1, s2, w2, pf.Hkv)
                assert excess(bad, ref) > 0, (t, s2, w2)
                checked += 1
    assert checked >= 16


def test_rope_append_prefill_t8192(env):
    # the prefill chunk's rope + append row: 8192 tokens from position 0 into an empty sink(4) +
    # window(4096) ring; sampled tokens' q and k rotated in place (one bf16 rounding), the ring
    # state, and sampled slots holding the oracle's rotated key and the raw value of the position
    # the ring rule puts there (the sinks, then the chunk's last 4096 tokens from slot S on)
    R, torch, dev, WL = env
    pf = WL.Prefill(R, torch, dev)
    S, W, T = pf.S, pf.W, pf.T
    ring = O.RingSeq(sinks=S, window=W)
    ring.append(T)
    slots = sorted({0, 1, S - 1, S, S + 1, S + 63, S + 64, S + W // 2, S + W - 2, S + W - 1}
                   | {int(x) for x in synth.rng(6100).integers(0, S + W, 20)})
    toks = sorted({0, 1, S - 1, S, 100, 4095, 4096, 4097, 8000, T - 2, T - 1} | {ring.slot_pos[sl] for sl in slots})
    ti = torch.tensor(toks, device=dev)
    q_raw, k_raw, v_raw = to_np64(pf.q[ti]), to_np64(pf.k[ti]), to_np64(pf.v[ti])
    pf.append()
    torch.cuda.synchronize()
    st = pf.int_state.cpu().tolist()
    assert st[3] == 0
    assert (st[0], st[1], st[2]) == (ring.head, ring.count, ring.seq_len)
    otab = O.build_table(oracle_cfg(pf.cfg), T)
    want_q = O.rope_apply(q_raw, toks, otab, pf.d, True)
    want_k = O.rope_apply(k_raw, toks, otab, pf.d, True)
    assert_bf16_rounded(to_np64(pf.q[ti]), want_q)
    assert_bf16_rounded(to_np64(pf.k[ti]), want_k)
    row = {t: i for i, t in enumerate(toks)}
    si = torch.tensor(slots, device=dev)
    kc = to_np64(pf.kc[0][:, si]).transpose(1, 0, 2)  # [slot, Hkv, d]
    vc = to_np64(pf.vc[0][:, si]).transpose(1, 0, 2)
    for i, sl in enumerate(slots):
        t = ring.slot_pos[sl]
        assert_bf16_rounded(kc[i], want_k[row[t]])
        assert np.array_equal(vc[i], v_raw[row[t]])


def test_mixed_step_two_streams(env):
    # the mixed-step row's launches: the 8192-token prefill chunk on one stream and the 256-sequence
    # windowed decode on another, running at once, give bit for bit the outputs each gives on one
    # stream (three repetitions, outputs cleared to NaN before each); sampled rows of both against
    # the oracle (the needle tests of the same launches carry the visible-set power)
    R, torch, dev, WL = env
    pf = WL.Prefill(R, torch, dev)
    wd = WL.WindowedPagedDecode(R, torch, dev)
    pf.run()
    wd.decode()
    torch.cuda.synchronize()
    assert pf.int_state[3].item() == 0 and wd.err.item() == 0
    ref_pf, ref_wd = pf.out.clone(), wd.out.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        pf.out.fill_(float("nan"))
        wd.out.fill_(float("nan"))
        cur = torch.cuda.current_stream()
        s1.wait_stream(cur)
        s2.wait_stream(cur)
        pf.run(stream=s1)
        wd.decode(stream=s2)
        cur.wait_stream(s1)
        cur.wait_stream(s2)
        torch.cuda.synchronize()
        assert pf.int_state[3].item() == 0 and wd.err.item() == 0
        assert torch.equal(pf.out, ref_pf), f"prefill differs on two streams (repetition {rep})"
        assert torch.equal(wd.out, ref_wd), f"decode differs on two streams (repetition {rep})"
    q, k, v, out = to_np64(pf.q), to_np64(pf.k), to_np64(pf.v), to_np64(ref_pf)
    for t in (100, pf.T - 1):
        bf16_attention_ref(out[t], O.decode_attention, q[t], lambda j: k[j], lambda j: v[j], t + 1, pf.S, pf.W,
                           pf.Hkv)
    dq, dout = to_np64(wd.q), to_np64(ref_wd)
    for b in (0, wd.B - 1):
        n = int(wd.lens[b])
        row = wd.table_host[b]
        live = sorted({int(x) for x in row if x >= 0})
        idx = torch.tensor(live, dtype=torch.long, device=wd.k.device)
        kb = dict(zip(live, to_np64(wd.k[idx])))
        vb = dict(zip(live, to_np64(wd.v[idx])))
        bf16_attention_ref(dout[b], O.decode_attention, dq[b], lambda j: kb[int(row[j // 16])][:, j % 16],
                           lambda j: vb[int(row[j // 16])][:, j % 16], n, wd.S, wd.W, wd.Hkv)


@pytest.mark.parametrize("kind", ["f16", "i8", "i8_keep", "i8_hadamard"])
def test_rerotate_l64_t524288_sampled_rows(env, kind):
    R, torch, dev, WL = env
    rr = WL.Rerotate(R, torch, dev, kind=kind)
    rows = np.unique(synth.rng(77).integers(0, rr.L * rr.T * rr.Hkv, 512))
    flat = rr.k.view(-1, rr.d)
    idx = torch.from_numpy(rows).to(dev)
    positions = (rows // rr.Hkv) % rr.T
    ca, cb = oracle_cfg(rr.cfg(1.0)), oracle_cfg(rr.cfg(1.125))
    if kind in ("i8_keep", "i8_hadamard"):
        # the sampled rows hold the oracle's own codes of seeded keys rotated at factor 1 (the rest of
        # the cache was written by the append kernel, as in the benchmark), uploaded by a torch copy
        raw = synth.normal((len(rows), rr.d), 78)
        krot = O.rotate_by_angle(raw, np.outer(positions, O.inv_freq(ca)), rr.r, True, O.mscale(ca))
        codes0, sc0 = O.quant_int8_hadamard_rows(krot) if kind == "i8_hadamard" else O.quant_int8_rows(krot)
        flat[idx] = torch.from_numpy(codes0).to(dev)
        rr.scale.view(-1)[idx] = torch.from_numpy(np.asarray(sc0, dtype=np.float32)).to(dev)
        before, sc_before = codes0, np.asarray(sc0, dtype=np.float32)
    else:  # seeded device fills
        before = flat[idx].cpu().numpy()
        sc_before = rr.scale.view(-1)[idx].cpu().numpy() if kind != "f16" else None
    rr.run(1.0, 1.125)
    torch.cuda.synchronize()
    after = flat[idx].cpu().numpy()
    if kind == "f16":
        ref = O.rerotate_rows(before.astype(np.float64), positions, ca, cb)
        unit = np.maximum(np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64), 1e-6)
        assert np.all(np.abs(after.astype(np.float64) - ref) <= unit)
        assert np.array_equal(after[:, rr.r:], before[:, rr.r:])
    elif kind == "i8_keep":
        # every sampled row checked against the branch the kernel took; the keep decision may
        # differ from the oracle's only at the re-coding edge
        sc_after = rr.scale.view(-1)[idx].cpu().numpy()
        n_keep, n_req = check_keep_scale_rows(before, sc_before, after, sc_after, positions, ca, cb)
        assert n_keep > 0 and n_req > 0
    else:
        rot = O.rerotate_int8_hadamard_rows if kind == "i8_hadamard" else O.rerotate_int8_rows
        codes, scale = rot(before, sc_before, positions, ca, cb)
        sc_after = rr.scale.view(-1)[idx].cpu().numpy()
        np.testing.assert_allclose(sc_after, scale, rtol=1e-5 if kind == "i8_hadamard" else 5e-6)
        quot = int8_turn_quotients(kind, before, sc_before, positions, ca, cb, scale)
        assert_int8_codes_valid(after, codes, quot, EPS_TURN_HADAMARD if kind == "i8_hadamard" else EPS_TURN_I8)
