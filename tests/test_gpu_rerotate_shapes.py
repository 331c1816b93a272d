"""Re-rotation ([DYN] "What it does": turn cached keys from factor A to factor B; rotation of rotated
keys, R_a R_b = R_{a+b}) over head shapes beyond the 128-dim rows of the benchmark: each of the
kernel paths the shape selects, against the fp64 oracle.

Float keys: A -> A leaves the cache bit for bit; A -> B is one rounding of the oracle's turn of the
stored values, the tail bit for bit.  int8 keys: codes valid against the oracle's exact quotients
(a code may differ from rne only where the quotient sits within EPS_TURN_I8 of a rounding edge),
new scales within 5e-6; keep-scale rows checked against the branch the kernel took.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (EPS_TURN_I8, assert_int8_codes_valid, assert_rounded_once, check_keep_scale_rows,
                            int8_turn_quotients, oracle_cfg, seeded_int8_rows, to_np64, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    return R, torch, dev


def _cfgs(R, d, r, neox):
    a = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.0, orig_max_pos=4096, neox=neox)
    b = R.rope_cfg(d, r, rope_theta=5e5, yarn_factor=1.75, orig_max_pos=4096, neox=neox)
    return a, b


FLOAT_SHAPES = [
    # dtype, d, r, neox
    ("f16", 64, 64, True),      # 8 16-byte chunks per rotary slice (chunk kernel)
    ("bf16", 256, 256, False),  # 32 chunks, the chunk kernel's largest
    ("f16", 512, 512, False),   # 64 chunks: 8-element vectors per thread
    ("f32", 512, 512, True),    # 4-element vectors, the largest head
    ("bf16", 128, 96, True),    # 12 chunks, not a power of two: 8-element vectors
    ("f16", 128, 36, True),     # half 18: one pair per thread
    ("f32", 34, 18, False),     # half 9, odd head dim
    ("f32", 2, 2, True),        # a single pair
    ("f16", 36, 16, True),      # 72-byte rows: not on 16-byte boundaries, so element by element
    ("f32", 34, 16, False),     # 136-byte rows, likewise
    ("bf16", 100, 64, True),    # 200-byte rows, likewise
]


@pytest.mark.parametrize("dtype_name,d,r,neox", FLOAT_SHAPES)
def test_rerotate_float_head_shapes(env, dtype_name, d, r, neox):
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype_name]
    kvdt = {"f32": R.F32, "bf16": R.BF16, "f16": R.F16}[dtype_name]
    L, T, Hkv, pos0 = 2, 40, 3, 300001
    ca, cb = _cfgs(R, d, r, neox)
    k = torch.from_numpy(synth.normal((L, T, Hkv, d), 700 + d + r)).to(dev, dtype)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, kvdt, Hkv, d, k, capacity=T, pos0=pos0, err_word=err)
    before = k.clone()
    R.rerotate(ca, ca, desc, L)
    torch.cuda.synchronize()
    assert torch.equal(k, before)  # A -> A: the identity, bit for bit
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    assert err.item() == 0
    b0, got = to_np64(before), to_np64(k)
    pos = np.arange(pos0, pos0 + T)
    for layer in range(L):
        want = O.rerotate_rows(b0[layer], pos, oracle_cfg(ca), oracle_cfg(cb))
        assert_rounded_once(got[layer], want, dtype_name)
        assert np.array_equal(got[layer][..., r:], b0[layer][..., r:])
    assert not np.array_equal(got[..., :r], b0[..., :r])


INT8_SHAPES = [
    # d, r, neox, keep the scale
    (64, 64, True, False),     # chunk kernel, 4 lanes per row
    (256, 128, True, False),   # chunk kernel, 16 lanes per row
    (512, 256, True, False),   # lane-local NeoX pairs, 32 lanes per row (the largest head)
    (512, 256, False, False),  # lane-local GPT-J pairs, 32 lanes per row
    (256, 128, True, True),    # keep-scale, rotary slice half the row, 16 lanes per row
    (64, 32, False, True),     # keep-scale chunk kernel, 4 lanes per row
    (512, 128, False, True),   # keep-scale lane-local pairs, 2 pairs per lane
    (512, 512, True, True),    # keep-scale lane-local pairs, 8 per lane, no tail (the largest head)
]


@pytest.mark.parametrize("d,r,neox,keep", INT8_SHAPES)
def test_rerotate_int8_head_shapes(env, d, r, neox, keep):
    R, torch, dev = env
    L, T, Hkv, pos0 = 2, 40, 3, 300007
    ca, cb = _cfgs(R, d, r, neox)
    c0, s0 = seeded_int8_rows((L, T, Hkv, d), 800 + d + r, r, 80 if keep else 127)
    s0[0, 3, 1] = 0.0  # an all-zero row
    c0[0, 3, 1] = 0
    codes = torch.from_numpy(c0).to(dev)
    scale = torch.from_numpy(s0).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, R.I8, Hkv, d, codes, capacity=T, pos0=pos0, k_scale=scale, err_word=err,
                      k_int8_mode=R.I8_KEEP_SCALE if keep else 0)
    R.rerotate(ca, cb, desc, L)
    torch.cuda.synchronize()
    assert err.item() == 0
    c1, s1 = codes.cpu().numpy(), scale.cpu().numpy()
    pos = np.repeat(np.arange(pos0, pos0 + T), Hkv)
    oa, ob = oracle_cfg(ca), oracle_cfg(cb)
    n_keep = n_over = 0
    for layer in range(L):
        cl, sl = c0[layer].reshape(-1, d), s0[layer].reshape(-1)
        got_c, got_s = c1[layer].reshape(-1, d), s1[layer].reshape(-1)
        if keep:
            k_, o_ = check_keep_scale_rows(cl, sl, got_c, got_s, pos, oa, ob)
            n_keep += k_
            n_over += o_
        else:
            wc, ws_ = O.rerotate_int8_rows(cl, sl, pos, oa, ob)
            np.testing.assert_allclose(got_s, ws_, rtol=5e-6)
            quot = int8_turn_quotients("i8", cl, sl, pos, oa, ob, ws_)
            assert_int8_codes_valid(got_c, wc, quot, EPS_TURN_I8)
    if keep:
        assert n_keep > 10 and n_over > 10  # both branches taken
    assert s1[0, 3, 1] == 0 and np.all(c1[0, 3, 1] == 0)


SHIFT_SHAPES = [
    # dtype, d, r, neox, delta
    ("f16", 128, 64, True, -1),   # 16-byte vectors (8 pairs per thread)
    ("f32", 512, 512, False, 3),  # 16-byte vectors (4 pairs), the largest head
    ("bf16", 96, 24, True, -2),   # r / 2 = 12: one pair per thread
    ("f32", 34, 16, True, 5),     # 136-byte rows: element by element
    ("bf16", 100, 64, False, -1), # 200-byte rows: element by element
]


@pytest.mark.parametrize("dtype_name,d,r,neox,delta", SHIFT_SHAPES)
def test_shift_keys_contig_head_shapes(env, dtype_name, d, r, neox, delta):
    # a contiguous cache of 3 layers: every row turns by delta positions ([SINK] "RoPE: absolute
    # positions and local rerotation", R_a R_b = R_{a+b}), one rounding of the oracle's shift, the
    # tail bit for bit
    R, torch, dev = env
    dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype_name]
    kvdt = {"f32": R.F32, "bf16": R.BF16, "f16": R.F16}[dtype_name]
    L, T, Hkv = 3, 24, 2
    cfg = R.rope_cfg(d, r, rope_theta=1e4, neox=neox)
    k = torch.from_numpy(synth.normal((L, T, Hkv, d), 900 + d + r)).to(dev, dtype)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    desc = R.kv_cache(R.CONTIG, kvdt, Hkv, d, k, capacity=T, err_word=err)
    before = to_np64(k)
    R.shift_keys(cfg, desc, delta, L)
    torch.cuda.synchronize()
    assert err.item() == 0
    got = to_np64(k)
    want = O.shift_keys(before.reshape(-1, d), delta, oracle_cfg(cfg)).reshape(before.shape)
    assert_rounded_once(got, want, dtype_name)
    assert np.array_equal(got[..., r:], before[..., r:])
