"""A decode step (rope + append of one token per sequence, then split-K decode)
captured in a HIP graph and replayed: every replay must give the eager step's
outputs bit for bit (same kernels, same inputs), with eager work and
synchronisations between the replays, and the oracle must agree with both.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from tests.gpu_util import bf16_attention_ref, bf16_round, assert_bf16_close, assert_bf16_rounded, oracle_cfg, to_np64, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R
    from sliding_window_kv_amd import workloads as WL

    return R, torch, dev, WL


@pytest.mark.parametrize("kv8", [None, "i8"])
def test_graph_replays_match_eager_step(env, kv8):
    R, torch, dev, WL = env
    wl = WL.PagedDecode(R, torch, dev, B=6, Hq=16, Hkv=4, d=128, ctx=531, seed=7100, kv8=kv8)
    q0, k0, v0 = wl.q.clone(), wl.k_new.clone(), wl.v_new.clone()

    def step():
        # fresh activations each time: the append rotates q in place
        wl.q.copy_(q0)
        wl.k_new.copy_(k0)
        wl.v_new.copy_(v0)
        wl.step()

    step()
    torch.cuda.synchronize()
    assert wl.err.item() == 0
    eager_out = wl.out.clone()
    eager_q = wl.q.clone()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream once
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        wl.out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device=dev)  # unrelated eager work between replays
        scratch.mul_(2.0).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert wl.err.item() == 0
        assert torch.equal(wl.out, eager_out), f"replay {rep} differs from the eager step"
        assert torch.equal(wl.q, eager_q)

    if kv8 is None:
        # the eager (and replayed) output against the oracle on two sequences
        otab = O.build_table(oracle_cfg(wl.cfg), wl.ctx)
        q_rot = to_np64(eager_q)
        out = to_np64(eager_out)
        p = wl.ctx - 1
        for b in (0, wl.B - 1):
            k, v = wl.kv_of(b)
            want_k = O.rope_apply(to_np64(k0)[b:b + 1], [p], otab, wl.d, True)[0]
            want_q = O.rope_apply(to_np64(q0)[b:b + 1], [p], otab, wl.d, True)[0]
            assert_bf16_rounded(k[p], want_k)
            assert_bf16_rounded(q_rot[b], want_q)
            # the attention over the oracle's own rotated q and new key (as bf16 holds them), the seeded
            # new value and the seeded cache rows before them
            assert np.array_equal(v[p], to_np64(v0)[b])
            k_ref, v_ref = k.copy(), v.copy()
            k_ref[p], v_ref[p] = bf16_round(want_k), to_np64(v0)[b]
            bf16_attention_ref(out[b], O.decode_attention, bf16_round(want_q), lambda j: k_ref[j], lambda j: v_ref[j],
                               wl.ctx, 0, 0, wl.Hkv)
