"""The allocation-free decode entry point against the workspace one.

ropekv_decode_attn_noalloc keeps its split-K partials in the library's own
per-GPU device array instead of a caller workspace; it runs the same plan and
kernels, so its output must equal ropekv_decode_attn's bit for bit.  Two calls
in a row, the second on a smaller input, show that a call does not depend on
what the previous one left in the shared array.  A plan whose partials exceed
the array is refused before any launch.
"""
import ctypes

import numpy as np
import pytest

from sliding_window_kv_amd import synth
from tests.gpu_util import DevPaged, DevRing, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R

    return R, torch, dev


def _both(R, torch, dev, q, B, Hq, cache, sinks=None):
    out_ws = torch.empty_like(q)
    out_na = torch.full_like(q, float("nan")) if q.is_floating_point() else torch.empty_like(q)
    ws = torch.empty(R.decode_workspace_size(B, Hq, cache.desc) // 4 + 1, dtype=torch.float32, device=dev)
    R.decode_attn(q, B, Hq, cache.desc, 0.0, out_ws, ws, ws.numel() * 4, sink_logits=sinks)
    R.decode_attn_noalloc(q, B, Hq, cache.desc, 0.0, out_na, sink_logits=sinks)
    torch.cuda.synchronize()
    assert cache.err.item() == 0
    return out_ws, out_na


def _paged(R, torch, dev, tdt, B, Hkv, d, S, W, lens, seed):
    max_blocks = max(lens) // 16 + 2
    num_blocks = B * max_blocks + 3
    table = synth.block_table_permutation(B, max_blocks, num_blocks, seed)
    cache = DevPaged(R, torch, dev, tdt, B, Hkv, d, S, W, table, num_blocks)
    if tdt == torch.int8:
        synth.device_int8_codes_(cache.k, seed + 1)
        synth.device_int8_codes_(cache.v, seed + 2)
        synth.device_uniform_(cache.k_scale, 1.0 / 127, 3.0 / 127, seed + 3)
        synth.device_uniform_(cache.v_scale, 1.0 / 127, 3.0 / 127, seed + 4)
    else:
        synth.device_normal_(cache.k, seed + 1)
        synth.device_normal_(cache.v, seed + 2)
    cache.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
    return cache


@pytest.mark.parametrize("kind", ["bf16", "f32", "i8"])
def test_noalloc_equals_workspace_decode_twice(env, kind):
    R, torch, dev = env
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "i8": torch.int8}[kind]
    qdt = torch.float32 if kind == "f32" else torch.bfloat16
    Hkv, n_rep, d = 8, 4, 128
    Hq = Hkv * n_rep
    # first call: a sink + window paged layer with ragged lengths, many splits per sequence
    lens = [1, 17, 300, 4100, 9000, 20000]
    cache = _paged(R, torch, dev, tdt, len(lens), Hkv, d, 4, 4096, lens, 71)
    q = torch.empty(len(lens), Hq, d, dtype=qdt, device=dev)
    synth.device_normal_(q, 72)
    sinks = torch.empty(Hq, dtype=torch.float32, device=dev)
    synth.device_normal_(sinks, 73)
    a, b = _both(R, torch, dev, q, len(lens), Hq, cache, sinks)
    assert torch.equal(a, b)
    assert bool(torch.isfinite(b.float()).all())
    # second call, smaller: fewer sequences, shorter, full attention, no sink logits
    lens2 = [40, 700]
    cache2 = _paged(R, torch, dev, tdt, len(lens2), Hkv, d, 0, 0, lens2, 81)
    q2 = torch.empty(len(lens2), Hq, d, dtype=qdt, device=dev)
    synth.device_normal_(q2, 82)
    a2, b2 = _both(R, torch, dev, q2, len(lens2), Hq, cache2)
    assert torch.equal(a2, b2)


def test_noalloc_ring_after_paged(env):
    # a ring layer (head at a random offset) right after a larger paged call
    R, torch, dev = env
    Hkv, n_rep, d, S, W = 8, 8, 128, 4, 1000
    Hq = Hkv * n_rep
    big = _paged(R, torch, dev, torch.bfloat16, 16, Hkv, d, 0, 0, [30000] * 16, 91)
    qb = torch.empty(16, Hq, d, dtype=torch.bfloat16, device=dev)
    synth.device_normal_(qb, 92)
    a, b = _both(R, torch, dev, qb, 16, Hq, big)
    assert torch.equal(a, b)
    B = 3
    ring = DevRing(R, torch, dev, torch.bfloat16, B, Hkv, d, S, W)
    synth.device_normal_(ring.k, 93)
    synth.device_normal_(ring.v, 94)
    ring.head.copy_(torch.from_numpy(synth.uniform_ints(B, 0, W, 95)))
    ring.count.fill_(W)
    ring.seq_len.copy_(torch.tensor([5000, 131072, 1004], dtype=torch.int32))
    q = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    synth.device_normal_(q, 96)
    a, b = _both(R, torch, dev, q, B, Hq, ring)
    assert torch.equal(a, b)


def test_noalloc_direct_plan(env):
    # 256 (sequence, KV head) units with short runs: a plan without partials (each unit's workgroup
    # writes its output); the allocation-free call takes it too
    R, torch, dev = env
    B, Hkv, n_rep, d, S, W = 32, 8, 4, 128, 4, 500
    Hq = Hkv * n_rep
    ring = DevRing(R, torch, dev, torch.bfloat16, B, Hkv, d, S, W)
    synth.device_normal_(ring.k, 101)
    synth.device_normal_(ring.v, 102)
    ring.head.copy_(torch.from_numpy(synth.uniform_ints(B, 0, W, 103)))
    ring.count.fill_(W)
    ring.seq_len.copy_(torch.from_numpy(synth.uniform_ints(B, W + S, 200000, 104)))
    assert R.decode_workspace_size(B, Hq, ring.desc) == 0
    q = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    synth.device_normal_(q, 105)
    a, b = _both(R, torch, dev, q, B, Hq, ring)
    assert torch.equal(a, b)
    assert bool(torch.isfinite(b.float()).all())


def test_noalloc_refuses_plans_beyond_its_array(env):
    # 256 sequences of a full-attention layer of 8192 blocks need 32 splits x 256 x 8 KV heads x
    # 4 heads x 130 floats = 136 MB of partials, more than the 64 MiB array: refused, nothing launched
    R, torch, dev = env
    Hkv, d = 8, 128
    fake = 0x1000
    desc = R.kv_cache(R.PAGED, R.BF16, Hkv, d, fake, fake, batch=256, block_size=16, max_blocks=8192,
                      num_blocks=1 << 21, block_table=fake, seq_len=fake, err_word=fake)
    need = R.decode_workspace_size(256, 32, desc)
    assert need > 64 << 20
    f = R.raw("ropekv_decode_attn_noalloc")
    rc = f(fake, 256, 32, ctypes.byref(desc), ctypes.c_float(0.0), None, fake, None)
    assert rc == R.ENOSPACE
    assert "scratch" in R.last_error()
    # a plan that fits is accepted by the same check (a real call, small)
    lens = [33]
    cache = _paged(R, torch, dev, torch.bfloat16, 1, Hkv, d, 0, 0, lens, 97)
    q = torch.empty(1, 32, d, dtype=torch.bfloat16, device=dev)
    synth.device_normal_(q, 98)
    a, b = _both(R, torch, dev, q, 1, 32, cache)
    assert torch.equal(a, b)
    assert np.isfinite(b.float().cpu().numpy()).all()
