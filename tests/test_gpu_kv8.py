"""GPU parity of the 8-bit KV caches (int8 and E4M3 codes, one fp32 scale per row):
per-row quantised K and V in apply_append, decode over codes x scales.

Reference values: the oracle's row quantisers (scale = max|x| / qmax with qmax
127 for int8 and 448 for E4M3, code = the nearest code to x / scale, decided in
float32) applied to the oracle's fp64 rotation, and the oracle's decode over the
dequantised rows.  Values are not rotated, so their codes and scales must match
bit for bit; a rotated key may land on the other side of a rounding boundary
(float32 vs fp64 rotation), so its code may be the neighbouring one, and then
only where the oracle's exact quotient sits at that boundary.  Decode outputs
(bf16) meet |gpu - ref| <= 2e-2 + 1e-2 |ref|.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (bf16_attention_ref, bf16_round, EPS_APPEND_FP8, EPS_APPEND_I8, DevPaged, DevRing, assert_bf16_close,
                            assert_fp8_codes_valid, assert_int8_codes_valid, oracle_cfg, to_np64, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    return R, torch, dev


KINDS = ["i8", "fp8"]
QMAX = {"i8": 127.0, "fp8": 448.0}


def _store(torch, kind):
    return torch.int8 if kind == "i8" else "fp8"


def _dequant(kind, codes_t, scale_t):
    if kind == "i8":
        return O.dequant_int8_rows(codes_t.cpu().numpy(), scale_t.cpu().numpy())
    return O.dequant_fp8_rows(codes_t.cpu().numpy(), scale_t.cpu().numpy())


def _ws(R, torch, dev, B, Hq, desc):
    return torch.empty(R.decode_workspace_size(B, Hq, desc) // 4 + 1, dtype=torch.float32, device=dev)


def _random_codes(torch, cache, seed, kind):
    fill = synth.device_int8_codes_ if kind == "i8" else synth.device_fp8_codes_
    fill(cache.k, seed)
    fill(cache.v, seed + 1)
    qmax = QMAX[kind]
    synth.device_uniform_(cache.k_scale, 0.5 / qmax, 3.0 / qmax, seed + 2)
    synth.device_uniform_(cache.v_scale, 0.5 / qmax, 3.0 / qmax, seed + 3)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n_rep,d,S,W,sinks", [(4, 128, 0, 0, False), (8, 128, 4, 100, False), (1, 64, 0, 0, False),
                                               (2, 64, 4, 40, True), (4, 128, 4, 300, True)])
def test_kv8_decode_paged(env, kind, n_rep, d, S, W, sinks):
    # paged 16-token blocks, random block table (null below the window edge), ragged lengths
    R, torch, dev = env
    Hkv = 8
    Hq = Hkv * n_rep
    lens = [1, 15, 16, 17, 300, 1024, 2000, 2049]
    B = len(lens)
    max_blocks = 130
    num_blocks = B * max_blocks + 11
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 81 + d + S)
    if W:
        for b, n in enumerate(lens):
            edge = max(0, (n - 1) - W + 1)
            for j in range(1, max_blocks):
                if 16 * j + 16 <= edge:
                    table[b, j] = -1
    cache = DevPaged(R, torch, dev, _store(torch, kind), B, Hkv, d, S, W, table, num_blocks)
    _random_codes(torch, cache, 82, kind)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = synth.device_normal_(torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 86)
    sl = synth.device_normal_(torch.empty(Hq, dtype=torch.float32, device=dev), 87) if sinks else None
    out = torch.empty_like(q)
    ws = _ws(R, torch, dev, B, Hq, cache.desc)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4, sink_logits=sl)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kd = _dequant(kind, cache.k, cache.k_scale)
    vd = _dequant(kind, cache.v, cache.v_scale)
    qq, got = to_np64(q), to_np64(out)
    slh = None if sl is None else sl.cpu().numpy().astype(np.float64)
    for b, n in enumerate(lens):
        def kb(j, b=b):
            return kd[table[b, j // 16], :, j % 16]

        def vb(j, b=b):
            return vd[table[b, j // 16], :, j % 16]

        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], kb, vb, n, S, W, Hkv, sink_logits=slh)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n_rep,d", [(4, 128), (8, 64)])
def test_kv8_decode_ring(env, kind, n_rep, d):
    # windowed layer: full ring (count = W), head at a random offset, long positions, C not a multiple of 16
    R, torch, dev = env
    Hkv, S, W = 8, 4, 300
    Hq = Hkv * n_rep
    B = 5
    cache = DevRing(R, torch, dev, _store(torch, kind), B, Hkv, d, S, W)
    _random_codes(torch, cache, 91, kind)
    heads = synth.uniform_ints(B, 0, W, 95)
    lens = [131072, 5000, 305, 304 + 7, 9999]
    cache.head.copy_(torch.from_numpy(heads))
    cache.count.fill_(W)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = synth.device_normal_(torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 96)
    out = torch.empty_like(q)
    ws = _ws(R, torch, dev, B, Hq, cache.desc)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kd = _dequant(kind, cache.k, cache.k_scale)
    vd = _dequant(kind, cache.v, cache.v_scale)
    qq, got = to_np64(q), to_np64(out)
    for b in range(B):
        ring = O.RingSeq(sinks=S, window=W, head=int(heads[b]), count=W, seq_len=lens[b])
        slot_of = dict(zip(O.visible_positions(lens[b] - 1, S, W), ring.chronological_slots()))
        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], lambda j: kd[b, :, slot_of[j]], lambda j: vd[b, :, slot_of[j]], lens[b], S,
                                 W, Hkv)


def _check_rows(kind, got_codes, got_scale, want_codes, want_scale, quot=None):
    """Codes / scales of cached rows against the oracle quantiser: bit for bit for values
    (quot None), rounding-edge validity for rotated keys (quot = the oracle's exact quotients)."""
    if quot is not None:
        if kind == "i8":
            assert_int8_codes_valid(got_codes, want_codes, quot, EPS_APPEND_I8)
        else:
            assert_fp8_codes_valid(got_codes, want_codes, quot, EPS_APPEND_FP8)
        np.testing.assert_allclose(got_scale, want_scale, rtol=1e-6, atol=0)
    else:
        assert np.array_equal(np.asarray(got_codes).view(np.uint8), np.asarray(want_codes).view(np.uint8))
        assert np.array_equal(got_scale, want_scale)


def _oracle_quant(kind, rows):
    """(codes, scale, dequantised rows, exact quotients) of the oracle's quantiser."""
    if kind == "i8":
        codes, scale = O.quant_int8_rows(rows)
        return codes, scale, O.dequant_int8_rows(codes, scale), O.row_quotients(rows, scale)
    codes, scale = O.quant_fp8_rows(rows)
    return codes, scale, O.dequant_fp8_rows(codes, scale), O.row_quotients(rows, scale)


@pytest.mark.parametrize("kind", KINDS)
def test_kv8_paged_append_and_decode(env, kind):
    # bf16 activations into an 8-bit paged cache with sinks + window: mixed steps, freeing, decode each round
    R, torch, dev = env
    B, Hq, Hkv, d, S, W = 4, 32, 8, 128, 4, 40
    max_len, bs = 200, 16
    max_blocks = max_len // bs + 1
    num_blocks = B * max_blocks + 7
    rng = synth.rng(500)
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 501)
    cfg = R.rope_cfg(d, d, rope_theta=5e5)
    gtab = torch.empty(max_len, d, dtype=torch.float32, device=dev)
    R.build_table(cfg, max_len, gtab)
    otab = O.build_table(oracle_cfg(cfg), max_len)
    cache = DevPaged(R, torch, dev, _store(torch, kind), B, Hkv, d, S, W, table, num_blocks)
    otable = [list(map(int, row)) for row in table]
    bf = torch.bfloat16
    qall = to_np64(torch.from_numpy(synth.normal((B, max_len, Hq, d), 502)).to(bf))
    kall = to_np64(torch.from_numpy(synth.normal((B, max_len, Hkv, d), 503)).to(bf))
    vall = to_np64(torch.from_numpy(synth.normal((B, max_len, Hkv, d), 504)).to(bf))
    krot = np.stack([O.rope_apply(kall[b], np.arange(max_len), otab, d, True) for b in range(B)])
    qrot = np.stack([O.rope_apply(qall[b], np.arange(max_len), otab, d, True) for b in range(B)])
    kq_codes, kq_scale, kdeq, kquot = _oracle_quant(kind, krot)
    vq_codes, vq_scale, vdeq, _ = _oracle_quant(kind, vall)
    n = [0] * B
    freed_dev = torch.full((B * max_blocks,), -7, dtype=torch.int32, device=dev)
    nfreed = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _ws(R, torch, dev, B, Hq, cache.desc)
    for _ in range(10):
        toks, oracle_freed = [], []
        for b in range(B):
            step = min(int(rng.choice([0, 1, 1, int(rng.integers(2, 40))])), max_len - n[b])
            if step == 0:
                continue
            oracle_freed += O.paged_free_expired(otable[b], n[b], S, W, bs)
            toks += [(b, p) for p in range(n[b], n[b] + step)]
            n[b] += step
        if not toks:
            continue
        N = len(toks)
        q = torch.from_numpy(np.stack([qall[b, p] for b, p in toks])).to(dev, bf)
        k = torch.from_numpy(np.stack([kall[b, p] for b, p in toks])).to(dev, bf)
        v = torch.from_numpy(np.stack([vall[b, p] for b, p in toks])).to(dev, bf)
        pos = torch.tensor([p for _, p in toks], dtype=torch.int32, device=dev)
        seq = torch.tensor([b for b, _ in toks], dtype=torch.int32, device=dev)
        nfreed.zero_()
        R.apply_append(cfg, gtab, max_len, q, Hq, k, v, R.BF16, N, pos, seq, cache.desc, freed_dev,
                       freed_dev.numel(), nfreed)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        assert cache.seq_len.cpu().tolist() == n
        assert cache.table.cpu().numpy().tolist() == otable
        assert sorted(freed_dev[:nfreed.item()].cpu().tolist()) == sorted(oracle_freed)
        kc, ks = cache.k.cpu().numpy(), cache.k_scale.cpu().numpy()
        vc, vs = cache.v.cpu().numpy(), cache.v_scale.cpu().numpy()
        # rows written by this step (rows of freed blocks may be reused later and are not checked)
        gk, gks, wk, wks, wq, gv, gvs, wv, wvs = [], [], [], [], [], [], [], [], []
        for b, p in toks:
            bid = otable[b][p // bs]
            if bid < 0:
                continue
            gk.append(kc[bid, :, p % bs]), gks.append(ks[bid, :, p % bs])
            wk.append(kq_codes[b, p]), wks.append(kq_scale[b, p]), wq.append(kquot[b, p])
            gv.append(vc[bid, :, p % bs]), gvs.append(vs[bid, :, p % bs])
            wv.append(vq_codes[b, p]), wvs.append(vq_scale[b, p])
        if gk:
            _check_rows(kind, np.stack(gk), np.stack(gks), np.stack(wk), np.stack(wks), np.stack(wq))
            _check_rows(kind, np.stack(gv), np.stack(gvs), np.stack(wv), np.stack(wvs))
        qd = torch.from_numpy(np.stack([qrot[b, max(n[b] - 1, 0)] for b in range(B)])).to(dev, bf)
        out = torch.empty(B, Hq, d, dtype=bf, device=dev)
        R.decode_attn(qd, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        got, qused = to_np64(out), to_np64(qd)
        for b in range(B):
            if n[b] == 0:
                assert np.all(got[b] == 0)
                continue
            ref = bf16_attention_ref(got[b], O.decode_attention, qused[b], lambda j: kdeq[b, j], lambda j: vdeq[b, j], n[b], S, W, Hkv)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("chunks", [[40, 1, 1, 1, 5], [3, 1, 20, 1, 7, 1]])
def test_kv8_ring_append_and_decode(env, kind, chunks):
    # bf16 activations into an 8-bit ring (S = 4, W = 12): survivors quantised, ring state bit-exact
    R, torch, dev = env
    B, Hq, Hkv, d, S, W = 1, 8, 4, 64, 4, 12
    n_total = sum(chunks)
    cfg = R.rope_cfg(d, d, rope_theta=1e4)
    gtab = torch.empty(n_total, d, dtype=torch.float32, device=dev)
    R.build_table(cfg, n_total, gtab)
    otab = O.build_table(oracle_cfg(cfg), n_total)
    bf = torch.bfloat16
    qd = torch.from_numpy(synth.normal((n_total, Hq, d), 511)).to(dev, bf)
    kd = torch.from_numpy(synth.normal((n_total, Hkv, d), 512)).to(dev, bf)
    vd = torch.from_numpy(synth.normal((n_total, Hkv, d), 513)).to(dev, bf)
    qrot = O.rope_apply(to_np64(qd), np.arange(n_total), otab, d, True)
    krot = O.rope_apply(to_np64(kd), np.arange(n_total), otab, d, True)
    kq_codes, kq_scale, kdeq, kquot = _oracle_quant(kind, krot)
    vq_codes, vq_scale, vdeq, _ = _oracle_quant(kind, to_np64(vd))
    cache = DevRing(R, torch, dev, _store(torch, kind), B, Hkv, d, S, W)
    oring = O.RingSeq(sinks=S, window=W)
    out = torch.empty(1, Hq, d, dtype=bf, device=dev)
    ws = _ws(R, torch, dev, 1, Hq, cache.desc)
    p0 = 0
    for T in chunks:
        q = qd[p0:p0 + T].clone()
        pos = torch.arange(p0, p0 + T, dtype=torch.int32, device=dev)
        seq = torch.zeros(T, dtype=torch.int32, device=dev)
        R.apply_append(cfg, gtab, n_total, q, Hq, kd[p0:p0 + T].clone(), vd[p0:p0 + T].clone(), R.BF16, T, pos, seq,
                       cache.desc)
        oring.append(T)
        torch.cuda.synchronize()
        assert cache.err.item() == 0
        assert (cache.head.item(), cache.count.item(), cache.seq_len.item()) == (oring.head, oring.count,
                                                                                  oring.seq_len)
        kc, ks = cache.k[0].cpu().numpy(), cache.k_scale[0].cpu().numpy()
        vc, vs = cache.v[0].cpu().numpy(), cache.v_scale[0].cpu().numpy()
        slots = sorted(oring.slot_pos)
        ps = [oring.slot_pos[s] for s in slots]
        _check_rows(kind, kc[:, slots].transpose(1, 0, 2), ks[:, slots].T, kq_codes[ps], kq_scale[ps], kquot[ps])
        _check_rows(kind, vc[:, slots].transpose(1, 0, 2), vs[:, slots].T, vq_codes[ps], vq_scale[ps])
        R.decode_attn(q[T - 1:T], 1, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
        torch.cuda.synchronize()
        # the oracle's rotated query as the bf16 activation holds it, the oracle's codes of the keys
        bf16_attention_ref(to_np64(out[0]), O.decode_attention, bf16_round(qrot[p0 + T - 1]), lambda j: kdeq[j],
                           lambda j: vdeq[j], p0 + T, S, W, Hkv)
        p0 += T
