"""GPU parity of the int8 key variants (k_int8_mode): keep-scale re-rotation and
Hadamard-rotated keys (append, decode, re-rotation), against the oracle.

Inputs are seeded codes and scales (or seeded raw keys for the append); the
expected values come from the oracle only.  A turned code may sit on the other
side of a rounding boundary (fp32 kernel math vs the oracle's fp64 turn), so a
code may differ by one step, and only where the oracle's exact quotient lies at
that boundary; scales agree to 1e-5 relative; kept scales and kept tail codes
are bitwise, and a keep / re-quantise decision may differ only at its edge.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (bf16_attention_ref, EPS_TURN_HADAMARD, DevPaged, assert_bf16_close, assert_int8_codes_valid,
                            check_keep_scale_rows, decode_int8, int8_turn_quotients, oracle_cfg, oracle_written, seeded_int8_rows, to_np64,
                            torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    return R, torch, dev


@pytest.mark.parametrize("r,neox", [(64, True), (128, True), (96, True), (64, False), (32, False)])
def test_keep_scale_rerotate_vs_oracle(env, r, neox):
    R, torch, dev = env
    L, T, Hkv, d = 2, 48, 4, 128
    # the gain mscale_to / mscale_from is 1 here (YaRN at factor 1 -> PI), so only the angles move keys
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=262144, neox=neox)
    cb = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.5, orig_max_pos=262144, neox=neox, rope_type=R.ROPE_LINEAR)
    pos0 = 200003
    c0, s0 = seeded_int8_rows((L, T, Hkv, d), 1200 + r, r, 80)
    s0[0, 5, 2] = 0.0
    c0[0, 5, 2] = 0
    codes = torch.from_numpy(c0).to(dev)
    scale = torch.from_numpy(s0).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, codes, capacity=T, pos0=pos0, k_scale=scale, err_word=err,
                      k_int8_mode=R.I8_KEEP_SCALE)
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    c1, s1 = codes.cpu().numpy(), scale.cpu().numpy()
    pos = np.repeat(np.arange(pos0, pos0 + T), Hkv)
    n_keep = n_over = 0
    for layer in range(L):
        k_, o_ = check_keep_scale_rows(c0[layer].reshape(-1, d), s0[layer].reshape(-1), c1[layer].reshape(-1, d),
                                       s1[layer].reshape(-1), pos, oracle_cfg(ca), oracle_cfg(cb))
        n_keep += k_
        n_over += o_
    assert n_keep > 20 and n_over > 20  # both branches exercised
    assert s1[0, 5, 2] == 0 and np.all(c1[0, 5, 2] == 0)


@pytest.mark.parametrize("r,neox,d,Hkv", [(64, True, 128, 4), (128, True, 128, 4), (64, False, 128, 4),
                                          (48, False, 128, 4), (16, False, 128, 4), (32, False, 128, 4),
                                          (96, False, 128, 4), (64, True, 64, 4), (128, True, 256, 4),
                                          (64, False, 256, 4), (64, True, 128, 3), (64, True, 128, 5)])
def test_hadamard_rerotate_vs_oracle(env, r, neox, d, Hkv):
    # head_dim 128 runs the two-lanes-per-row kernels (half rows when the turn stays in dims < 64), other
    # head dims the general one; with 3 or 5 KV heads a 128-row chunk starts and ends inside a position,
    # and the second chunk of each layer is partial; 10 layers span two groups of layers
    R, torch, dev = env
    L, T = (10 if Hkv == 5 else 2), 48
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=262144, neox=neox)
    cb = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.625, orig_max_pos=262144, neox=neox)
    pos0 = 300007
    c0, s0 = seeded_int8_rows((L, T, Hkv, d), 1300 + r + d, r, 127)
    s0[1, 7, Hkv - 1] = 0.0  # an all-zero row stays all zero with scale 0
    c0[1, 7, Hkv - 1] = 0
    codes = torch.from_numpy(c0).to(dev)
    scale = torch.from_numpy(s0).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, codes, capacity=T, pos0=pos0, k_scale=scale, err_word=err,
                      k_int8_mode=R.I8_HADAMARD)
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    c1, s1 = codes.cpu().numpy(), scale.cpu().numpy()
    pos = np.repeat(np.arange(pos0, pos0 + T), Hkv)
    for layer in range(L):
        cl, sl = c0[layer].reshape(-1, d), s0[layer].reshape(-1)
        wc, ws_ = O.rerotate_int8_hadamard_rows(cl, sl, pos, oracle_cfg(ca), oracle_cfg(cb))
        np.testing.assert_allclose(s1[layer].reshape(-1), ws_, rtol=1e-5)
        quot = int8_turn_quotients("i8_hadamard", cl, sl, pos, oracle_cfg(ca), oracle_cfg(cb), ws_)
        assert_int8_codes_valid(c1[layer].reshape(-1, d), wc, quot, EPS_TURN_HADAMARD)
    assert s1[1, 7, Hkv - 1] == 0 and np.all(c1[1, 7, Hkv - 1] == 0)


@pytest.mark.parametrize("neox,r", [(True, 64), (False, 64), (True, 128)])
def test_hadamard_rerotate_identity(env, neox, r):
    # A -> A over Hadamard rows as the quantiser leaves them (a row's largest code +-127): the turn is
    # the identity, so the codes come back bit for bit and the scale within one float32 rounding;
    # the oracle's turn is the identity too
    R, torch, dev = env
    L, T, Hkv, d = 2, 40, 4, 128
    ca = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.375, orig_max_pos=262144, neox=neox)
    oa = oracle_cfg(ca)
    pos0 = 250001
    raw = synth.normal((L, T, Hkv, d), 1350 + r + neox)
    angles = np.outer(np.arange(pos0, pos0 + T), O.inv_freq(oa))[:, None, :]
    key = np.stack([O.rotate_by_angle(raw[l], angles, r, neox, O.mscale(oa)) for l in range(L)])
    c0, s0 = O.quant_int8_hadamard_rows(key)
    s0 = np.asarray(s0, dtype=np.float32)
    codes, scale = torch.from_numpy(c0).to(dev), torch.from_numpy(s0).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, codes, capacity=T, pos0=pos0, k_scale=scale, err_word=err,
                      k_int8_mode=R.I8_HADAMARD)
    R.rerotate(ca, ca, desc, L)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert np.array_equal(codes.cpu().numpy(), c0)
    np.testing.assert_allclose(scale.cpu().numpy(), s0, rtol=2.0 ** -23, atol=0)
    pos = np.repeat(np.arange(pos0, pos0 + T), Hkv)
    wc, ws_ = O.rerotate_int8_hadamard_rows(c0[0].reshape(-1, d), s0[0].reshape(-1), pos, oa, oa)
    assert np.array_equal(wc, c0[0].reshape(-1, d))
    np.testing.assert_allclose(ws_, s0[0].reshape(-1), rtol=1e-12)


def test_hadamard_rerotate_bounds_from_append(env):
    # raw keys written at A by apply_append into Hadamard-rotated int8 rows, turned to B, compared with
    # the fp64 key at B in the H domain; the key written directly at B, as the oracle's Hadamard
    # quantiser stores it, is the yardstick
    R, torch, dev = env
    L, T, Hkv, d, r = 2, 256, 8, 128, 64
    kw = dict(rope_theta=5e5, orig_max_pos=262144)
    P = 524288
    for fa, fb in ((1.0, 2.0), (2.0, 1.0)):
        ca, cb = R.rope_cfg(d, r, yarn_factor=fa, **kw), R.rope_cfg(d, r, yarn_factor=fb, **kw)
        ta = torch.empty(P, r, dtype=torch.float32, device=dev)
        R.build_table(ca, P, ta)
        pos0 = 262144 - T // 2
        raw = torch.from_numpy(synth.normal((L, T, Hkv, d), 1400)).to(dev, torch.float16)
        ka = torch.zeros(L, T, Hkv, d, dtype=torch.int8, device=dev)
        sa = torch.zeros(L, T, Hkv, dtype=torch.float32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        pos_d = torch.arange(pos0, pos0 + T, dtype=torch.int32, device=dev)
        for layer in range(L):
            dl = R.kv_cache(R.CONTIG, R.I8, Hkv, d, ka[layer], capacity=T, pos0=pos0, k_scale=sa[layer],
                            err_word=err, k_int8_mode=R.I8_HADAMARD)
            R.apply_append(ca, ta, P, None, 0, raw[layer].clone(), None, R.F16, T, pos_d, None, dl)
        torch.cuda.synchronize()
        assert err.item() == 0
        desc_a = R.kv_cache(R.CONTIG, R.I8, Hkv, d, ka, capacity=T, pos0=pos0, k_scale=sa, err_word=err,
                            k_int8_mode=R.I8_HADAMARD)
        rawn = to_np64(raw)
        pos = np.arange(pos0, pos0 + T)
        oa, ob = oracle_cfg(ca), oracle_cfg(cb)

        def key_at(o):
            return np.stack([O.rotate_by_angle(rawn[l], np.outer(pos, O.inv_freq(o))[:, None, :], r, True, O.mscale(o))
                             for l in range(L)])

        # the append's rows against the oracle's Hadamard quantiser of the fp64 key at A
        key_a = key_at(oa)
        wc, ws_ = O.quant_int8_hadamard_rows(key_a)
        assert_int8_codes_valid(ka.cpu().numpy(), wc, O.row_quotients(O.hadamard(key_a), ws_), EPS_TURN_HADAMARD)
        np.testing.assert_allclose(sa.cpu().numpy(), ws_, rtol=1e-5)
        R.rerotate(ca, cb, desc_a, L)
        torch.cuda.synchronize()
        assert err.item() == 0
        key_b = key_at(ob)
        truth = O.hadamard(key_b)
        written, unit = oracle_written("i8_hadamard", key_b)  # H domain
        turned = decode_int8(ka.cpu().numpy(), sa.cpu().numpy())
        et, ew = turned - truth, written - truth
        ratio = float(np.sqrt(np.mean(et * et)) / np.sqrt(np.mean(ew * ew)))
        worst = float(np.max(np.abs(et) / unit))
        assert ratio <= 1.6 and worst <= 3.0, (fa, fb, ratio, worst)


@pytest.mark.parametrize("n_rep,d", [(4, 128), (8, 64)])
def test_hadamard_decode_paged(env, n_rep, d):
    # seeded codes standing for H k: decode must score with H q, i.e. equal attention over the plain keys
    R, torch, dev = env
    Hkv, S, W = 4, 4, 100
    Hq = Hkv * n_rep
    lens = [1, 16, 33, 150, 700]
    B = len(lens)
    max_blocks = 48
    num_blocks = B * max_blocks + 3
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 1500 + d)
    cache = DevPaged(R, torch, dev, torch.int8, B, Hkv, d, S, W, table, num_blocks)
    synth.device_int8_codes_(cache.k, 1501)
    synth.device_int8_codes_(cache.v, 1502)
    synth.device_uniform_(cache.k_scale, 0.5 / 127, 3.0 / 127, 1503)
    synth.device_uniform_(cache.v_scale, 0.5 / 127, 3.0 / 127, 1504)
    cache.desc.k_int8_mode = R.I8_HADAMARD
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    q = synth.device_normal_(torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev), 1505)
    out = torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kd = O.hadamard(O.dequant_int8_rows(cache.k.cpu().numpy(), cache.k_scale.cpu().numpy()))  # plain keys
    vd = O.dequant_int8_rows(cache.v.cpu().numpy(), cache.v_scale.cpu().numpy())
    qq, got = to_np64(q), to_np64(out)
    for b, n in enumerate(lens):
        ref = bf16_attention_ref(got[b], O.decode_attention, qq[b], lambda j, b=b: kd[table[b, j // 16], :, j % 16],
                                 lambda j, b=b: vd[table[b, j // 16], :, j % 16], n, S, W, Hkv)


def test_hadamard_paged_append_then_decode(env):
    # bf16 activations appended into Hadamard-rotated int8 keys, then decode, against the oracle's storage
    R, torch, dev = env
    B, Hq, Hkv, d, S, W = 2, 16, 4, 128, 4, 40
    n_tok, bs = 90, 16
    max_blocks = n_tok // bs + 1
    num_blocks = B * max_blocks
    table = synth.block_table_permutation(B, max_blocks, num_blocks, 1600)
    cfg = R.rope_cfg(d, d, rope_theta=5e5)
    gtab = torch.empty(n_tok, d, dtype=torch.float32, device=dev)
    R.build_table(cfg, n_tok, gtab)
    otab = O.build_table(oracle_cfg(cfg), n_tok)
    cache = DevPaged(R, torch, dev, torch.int8, B, Hkv, d, S, W, table, num_blocks)
    cache.desc.k_int8_mode = R.I8_HADAMARD
    bf = torch.bfloat16
    qall = to_np64(torch.from_numpy(synth.normal((B, n_tok, Hq, d), 1601)).to(bf))
    kall = to_np64(torch.from_numpy(synth.normal((B, n_tok, Hkv, d), 1602)).to(bf))
    vall = to_np64(torch.from_numpy(synth.normal((B, n_tok, Hkv, d), 1603)).to(bf))
    krot = np.stack([O.rope_apply(kall[b], np.arange(n_tok), otab, d, True) for b in range(B)])
    qrot = np.stack([O.rope_apply(qall[b], np.arange(n_tok), otab, d, True) for b in range(B)])
    kc_want, ks_want = O.quant_int8_hadamard_rows(krot)
    kplain = O.hadamard(O.dequant_int8_rows(kc_want, ks_want))
    vc_want, vs_want = O.quant_int8_rows(vall)
    vdeq = O.dequant_int8_rows(vc_want, vs_want)
    # whole prompts in one call (positions 0 .. n_tok - 1 of both sequences)
    toks = [(b, p) for b in range(B) for p in range(n_tok)]
    q = torch.from_numpy(np.stack([qall[b, p] for b, p in toks])).to(dev, bf)
    k = torch.from_numpy(np.stack([kall[b, p] for b, p in toks])).to(dev, bf)
    v = torch.from_numpy(np.stack([vall[b, p] for b, p in toks])).to(dev, bf)
    pos = torch.tensor([p for _, p in toks], dtype=torch.int32, device=dev)
    seq = torch.tensor([b for b, _ in toks], dtype=torch.int32, device=dev)
    R.apply_append(cfg, gtab, n_tok, q, Hq, k, v, R.BF16, len(toks), pos, seq, cache.desc)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    kc, ks = cache.k.cpu().numpy(), cache.k_scale.cpu().numpy()
    got_c = np.stack([kc[table[b, p // bs], :, p % bs] for b, p in toks]).reshape(B, n_tok, Hkv, d)
    got_s = np.stack([ks[table[b, p // bs], :, p % bs] for b, p in toks]).reshape(B, n_tok, Hkv)
    assert_int8_codes_valid(got_c, kc_want, O.row_quotients(O.hadamard(krot), ks_want), EPS_TURN_HADAMARD)
    np.testing.assert_allclose(got_s, ks_want, rtol=1e-5)
    qd = torch.from_numpy(qrot[:, n_tok - 1]).to(dev, bf)
    out = torch.empty(B, Hq, d, dtype=bf, device=dev)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(qd, B, Hq, cache.desc, 0.0, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    got, qused = to_np64(out), to_np64(qd)
    for b in range(B):
        ref = bf16_attention_ref(got[b], O.decode_attention, qused[b], lambda j, b=b: kplain[b, j], lambda j, b=b: vdeq[b, j], n_tok, S, W, Hkv)
