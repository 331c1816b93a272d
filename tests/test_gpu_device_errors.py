"""Conditions only device data can show: each sets its ROPEKV_DEV_* bit in the cache's err_word and
the kernel skips the offending token or tile, touching nothing out of bounds, while the rest of the
call proceeds (the header's error contract).  Each case plants one bad token or block beside good
ones and checks the bit, that nothing was written for the bad one, and the good ones against the
oracle.  Every kernel exits normally: these are the kernels' own bounds checks, not faults.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (DevPaged, DevRing, attend_set, bf16_attention_ref, decode_int8, oracle_cfg, rowwise, to_np64,
                            torch_dev)

pytestmark = pytest.mark.gpu

D, HKV, HQ, P = 64, 2, 4, 64


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    cfg = R.rope_cfg(D, D, rope_theta=1e4)
    table = torch.empty(P, D, dtype=torch.float32, device=dev)
    R.build_table(cfg, P, table)
    return R, torch, dev, cfg, table


def _append(env, desc, positions, seqs, seed, freed=None, cap=0, n_freed=None):
    R, torch, dev, cfg, table = env
    n = len(positions)
    q = torch.from_numpy(synth.normal((n, HQ, D), seed)).to(dev)
    k = torch.from_numpy(synth.normal((n, HKV, D), seed + 1)).to(dev)
    v = torch.from_numpy(synth.normal((n, HKV, D), seed + 2)).to(dev)
    raw_k = to_np64(k)
    pos = torch.tensor(positions, dtype=torch.int32, device=dev)
    seq = None if seqs is None else torch.tensor(seqs, dtype=torch.int32, device=dev)
    R.apply_append(cfg, table, P, q, HQ, k, v, R.F32, n, pos, seq, desc, freed, cap, n_freed)
    torch.cuda.synchronize()
    return raw_k, k, v


def _rotated(env, raw_k, p):
    R, torch, dev, cfg, table = env
    return O.rope_apply(raw_k[None], [p], O.build_table(oracle_cfg(cfg), P), D, True)[0]


def test_position_outside_the_table(env):
    R, torch, dev, cfg, table = env
    c = DevRing(R, torch, dev, torch.float32, 2, HKV, D, 2, 6)
    raw_k, k, v = _append(env, c.desc, [0, 70], [0, 1], 3100)
    assert c.err.item() == R.DEV_TABLE_RANGE
    assert np.array_equal(to_np64(k[1]), raw_k[1])  # the bad token is left as it was
    assert c.seq_len.cpu().tolist() == [1, 0]
    assert not c.k[1].any() and not c.v[1].any()
    assert rowwise(to_np64(c.k[0, :, 0]), _rotated(env, raw_k[0], 0)) <= 1e-6
    assert torch.equal(c.v[0, :, 0], v[0])


def test_sequence_outside_the_batch(env):
    R, torch, dev, cfg, table = env
    c = DevRing(R, torch, dev, torch.float32, 2, HKV, D, 2, 6)
    raw_k, k, v = _append(env, c.desc, [0, 0], [0, 2], 3200)
    assert c.err.item() == R.DEV_SEQ_RANGE
    assert c.seq_len.cpu().tolist() == [1, 0] and c.head.cpu().tolist() == [0, 0]
    assert not c.k[1].any()
    assert torch.equal(c.v[0, :, 0], v[0])


def test_token_not_at_its_next_position(env):
    R, torch, dev, cfg, table = env
    c = DevRing(R, torch, dev, torch.float32, 2, HKV, D, 2, 6)
    raw_k, k, v = _append(env, c.desc, [0, 5], [0, 1], 3300)  # sequence 1 holds 0 tokens: 5 is not next
    assert c.err.item() == R.DEV_POSITION
    assert c.seq_len.cpu().tolist() == [1, 0] and c.count.cpu().tolist() == [0, 0]
    assert not c.k[1].any() and not c.v[1].any()
    assert torch.equal(c.v[0, :, 0], v[0])


def test_null_block_and_block_range_in_the_append(env):
    R, torch, dev, cfg, table = env
    # sequence 1's first block is null; sequence 2 (32 tokens cached) needs a third block beyond max_blocks
    tab = np.array([[0, 1], [-1, 2], [3, 4]], dtype=np.int32)
    c = DevPaged(R, torch, dev, torch.float32, 3, HKV, D, 0, 0, tab, 5)
    c.seq_len.copy_(torch.tensor([0, 0, 32], dtype=torch.int32))
    raw_k, k, v = _append(env, c.desc, [0, 0, 32], [0, 1, 2], 3400)
    assert c.err.item() == R.DEV_NULL_BLOCK | R.DEV_BLOCK_RANGE
    assert c.seq_len.cpu().tolist() == [1, 1, 33]  # block errors still advance the state
    assert torch.equal(c.v[0, :, 0], v[0])  # sequence 0, block 0, slot 0
    assert not c.k[1:].any() and not c.v[1:].any()  # nothing else written anywhere in the pool
    assert rowwise(to_np64(c.k[0, :, 0]), _rotated(env, raw_k[0], 0)) <= 1e-6


def test_contig_row_outside_the_capacity(env):
    R, torch, dev, cfg, table = env
    kc = torch.zeros(8, HKV, D, dtype=torch.float32, device=dev)
    vc = torch.zeros_like(kc)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.F32, HKV, D, kc, vc, capacity=8, pos0=4, err_word=err)
    raw_k, k, v = _append(env, desc, [5, 12, 3], None, 3500)  # rows 1, 8 (past the end) and -1 (before it)
    assert err.item() == R.DEV_BLOCK_RANGE
    assert torch.equal(vc[1], v[0])
    written = [i for i in range(8) if vc[i].any()]
    assert written == [1]


def test_freed_block_list_too_short(env):
    R, torch, dev, cfg, table = env
    # one-token blocks, window 2: appending position 5 after 5 cached tokens expires blocks 0..3, four
    # ids for a list of two: nothing is freed and the bit is set; the token itself is written
    tab = np.arange(8, dtype=np.int32)[None]
    c = DevPaged(R, torch, dev, torch.float32, 1, HKV, D, 0, 2, tab, 8, bs=1)
    c.seq_len.fill_(5)
    freed = torch.full((2,), -7, dtype=torch.int32, device=dev)
    n_freed = torch.zeros(1, dtype=torch.int32, device=dev)
    raw_k, k, v = _append(env, c.desc, [5], [0], 3600, freed, 2, n_freed)
    assert c.err.item() == R.DEV_FREE_OVERFLOW
    assert c.table.cpu().numpy().tolist() == tab.tolist()  # no entry nulled
    assert freed.cpu().tolist() == [-7, -7]
    assert torch.equal(c.v[5, :, 0], v[0])
    assert c.seq_len.item() == 6


def test_decode_skips_a_null_block_it_must_read(env):
    # full-attention paged decode, fp32: sequence 1's second block (keys 16..31) is null; the bit is
    # set, that tile is skipped (the output is the attention over the other keys), sequence 0 exact
    R, torch, dev, cfg, table = env
    n, nb = 40, 3
    tab = np.array([[0, 1, 2], [3, -1, 5]], dtype=np.int32)
    c = DevPaged(R, torch, dev, torch.float32, 2, HKV, D, 0, 0, tab, 6)
    c.k.copy_(torch.from_numpy(synth.normal(tuple(c.k.shape), 3700)))
    c.v.copy_(torch.from_numpy(synth.normal(tuple(c.v.shape), 3701)))
    c.seq_len.fill_(n)
    q = torch.from_numpy(synth.normal((2, HQ, D), 3702)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(2, HQ, c.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, 2, HQ, c.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert c.err.item() == R.DEV_NULL_BLOCK
    kp, vp, qq, got = to_np64(c.k), to_np64(c.v), to_np64(q), to_np64(out)

    def rows(b):
        K = np.stack([kp[tab[b, j // 16], :, j % 16] if tab[b, j // 16] >= 0 else np.zeros((HKV, D)) for j in range(n)])
        V = np.stack([vp[tab[b, j // 16], :, j % 16] if tab[b, j // 16] >= 0 else np.zeros((HKV, D)) for j in range(n)])
        return K, V

    K0, V0 = rows(0)
    assert rowwise(got[0], attend_set(qq[0], K0, V0, np.arange(n), HKV)) <= 1e-5
    K1, V1 = rows(1)
    kept = [j for j in range(n) if not 16 <= j < 32]
    assert rowwise(got[1], attend_set(qq[1], K1, V1, kept, HKV)) <= 1e-5


def _att_over(n, idx):
    """The oracle's attention over keys 0..n-1 restricted to the rows idx (keys a kernel skipped are
    left out), as a callable of (q, key-by-position, value-by-position)."""
    def att(q, kf, vf):
        Ks = np.stack([kf(j) for j in range(n)])
        Vs = np.stack([vf(j) for j in range(n)])
        return attend_set(q, Ks, Vs, idx, HKV)
    return att


@pytest.mark.parametrize("dtype_name", ["f32", "bf16"])
def test_prefill_prefix_in_a_null_block(env, dtype_name):
    # an 8-token chunk at pos0 40 over a paged window-12 prefix whose blocks 0 (out of every query's
    # window) and 1 (keys 16..31) are null: queries 40..42 see keys 29..31, so the call sets
    # PREFIX_LOST and their rows are unspecified; queries 43..47 see no lost key and match the oracle
    # (fp32 kernel and bf16 MFMA kernel)
    R, torch, dev, cfg, table = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype_name]
    pos0, T, W = 40, 8, 12
    tab = np.array([[-1, -1, 2, 3]], dtype=np.int32)
    c = DevPaged(R, torch, dev, dtype, 1, HKV, D, 0, W, tab, 4)
    c.k.copy_(torch.from_numpy(synth.normal(tuple(c.k.shape), 3800)).to(dtype))
    c.v.copy_(torch.from_numpy(synth.normal(tuple(c.v.shape), 3801)).to(dtype))
    c.seq_len.fill_(pos0)
    q = torch.from_numpy(synth.normal((T, HQ, D), 3802)).to(dev, dtype)
    k = torch.from_numpy(synth.normal((T, HKV, D), 3803)).to(dev, dtype)
    v = torch.from_numpy(synth.normal((T, HKV, D), 3804)).to(dev, dtype)
    out = torch.empty_like(q)
    R.prefill_attn(q, k, v, T, pos0, HQ, c.desc, 0, 0.0, out)
    torch.cuda.synchronize()
    assert c.err.item() == R.DEV_PREFIX_LOST
    kp, vp, qq, got = to_np64(c.k), to_np64(c.v), to_np64(q), to_np64(out)
    kk, vv = to_np64(k), to_np64(v)

    def kf(j):
        return kk[j - pos0] if j >= pos0 else kp[tab[0, j // 16], :, j % 16]

    def vf(j):
        return vv[j - pos0] if j >= pos0 else vp[tab[0, j // 16], :, j % 16]

    for t in range(3, T):  # queries 43..47: window 32..47 at most, all keys present
        assert min(O.visible_positions(pos0 + t, 0, W)) >= 32
        args = (qq[t], kf, vf, pos0 + t + 1, 0, W, HKV)
        if dtype_name == "f32":
            assert rowwise(got[t], O.decode_attention(*args)) <= 1e-5
        else:
            bf16_attention_ref(got[t], O.decode_attention, *args)


def test_int8_decode_skips_a_null_block(env):
    # the 8-bit decode kernel, int8 codes with row scales: sequence 1's second block is null; the
    # bit is set, that tile skipped, sequence 0 matches the oracle over every key
    R, torch, dev, cfg, table = env
    n = 40
    tab = np.array([[0, 1, 2], [3, -1, 5]], dtype=np.int32)
    c = DevPaged(R, torch, dev, torch.int8, 2, HKV, D, 0, 0, tab, 6)
    g = torch.Generator(device=dev)
    g.manual_seed(3900)
    for buf, sc in ((c.k, c.k_scale), (c.v, c.v_scale)):
        buf.copy_(torch.randint(-127, 128, tuple(buf.shape), dtype=torch.int8, device=dev, generator=g))
        sc.copy_(torch.rand(tuple(sc.shape), device=dev, generator=g) * 0.02 + 0.01)
    c.seq_len.fill_(n)
    q = torch.from_numpy(synth.normal((2, HQ, D), 3901)).to(dev, torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(2, HQ, c.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, 2, HQ, c.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert c.err.item() == R.DEV_NULL_BLOCK
    kd = decode_int8(c.k.cpu().numpy(), c.k_scale.cpu().numpy())
    vd = decode_int8(c.v.cpu().numpy(), c.v_scale.cpu().numpy())
    qq, got = to_np64(q), to_np64(out)
    for b, idx in ((0, list(range(n))), (1, [j for j in range(n) if not 16 <= j < 32])):
        def kf(j, b=b):
            return kd[tab[b, j // 16], :, j % 16] if tab[b, j // 16] >= 0 else np.zeros((HKV, D))

        def vf(j, b=b):
            return vd[tab[b, j // 16], :, j % 16] if tab[b, j // 16] >= 0 else np.zeros((HKV, D))

        bf16_attention_ref(got[b], _att_over(n, idx), qq[b], kf, vf)


def test_decode_sequence_longer_than_its_block_table(env):
    # full-attention paged decode, fp32, two table columns (32 keys): sequence 1 claims 40 tokens; the
    # bit is set, the 8 keys no block covers are skipped (its output is the attention over keys
    # 0..31), sequence 0 (32 tokens) exact
    R, torch, dev, cfg, table = env
    tab = np.array([[0, 1], [2, 3]], dtype=np.int32)
    c = DevPaged(R, torch, dev, torch.float32, 2, HKV, D, 0, 0, tab, 4)
    c.k.copy_(torch.from_numpy(synth.normal(tuple(c.k.shape), 4000)))
    c.v.copy_(torch.from_numpy(synth.normal(tuple(c.v.shape), 4001)))
    c.seq_len.copy_(torch.tensor([32, 40], dtype=torch.int32))
    q = torch.from_numpy(synth.normal((2, HQ, D), 4002)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(2, HQ, c.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, 2, HQ, c.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert c.err.item() == R.DEV_BLOCK_RANGE
    kp, vp, qq, got = to_np64(c.k), to_np64(c.v), to_np64(q), to_np64(out)
    for b in (0, 1):
        K = np.stack([kp[tab[b, j // 16], :, j % 16] for j in range(32)])
        V = np.stack([vp[tab[b, j // 16], :, j % 16] for j in range(32)])
        assert rowwise(got[b], attend_set(qq[b], K, V, np.arange(32), HKV)) <= 1e-5
