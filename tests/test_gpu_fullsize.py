"""Parity at the benchmark's full sizes, in the launch configuration bench.py times.

Sampled outputs are checked one by one against the fp64 oracle: whole
sequences for decode, single query rows for prefill, random rows for the
re-rotation.  Inputs are the seeded device buffers of the workload (filled by
torch's generator), read back to the host for the oracle.
"""
import numpy as np
import pytest

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import synth
from tests.gpu_util import (EPS_APPEND_FP8, EPS_APPEND_I8, EPS_TURN_HADAMARD, EPS_TURN_I8, assert_bf16_close,
                            assert_fp8_codes_valid, assert_int8_codes_valid, check_keep_scale_rows,
                            int8_turn_quotients, oracle_cfg, to_np64, torch_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch

    dev = torch_dev()
    from sliding_window_kv_amd import ropekv as R
    from sliding_window_kv_amd import workloads as WL

    return R, torch, dev, WL


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
        assert_bf16_close(q_rot[b], want_q, atol=1e-2, rtol=1e-2)
        k, v = wl.kv_of(b)
        want_k = O.rope_apply(k_raw[b:b + 1], [p], otab_row, wl.d, True)[0]
        assert_bf16_close(k[p], want_k, atol=1e-2, rtol=1e-2)
        assert np.array_equal(v[p], v_raw[b])
        ref = O.decode_attention(q_rot[b], lambda j: k[j], lambda j: v[j], wl.ctx, 0, 0, wl.Hkv)
        assert_bf16_close(out[b], ref)


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
        k = dequant(kc, ks)
        v = dequant(vc, vs)
        ref = O.decode_attention(q_rot[b], lambda j: k[j], lambda j: v[j], wl.ctx, 0, 0, wl.Hkv)
        assert_bf16_close(out[b], ref)


def test_ring_decode_128k(env):
    R, torch, dev, WL = env
    r = WL.RingDecode(R, torch, dev)
    r.decode()
    torch.cuda.synchronize()
    assert r.err.item() == 0
    heads = r.head.cpu().numpy()
    out = to_np64(r.out)
    q = to_np64(r.q)
    for b in (0, 17, 31):
        kc = to_np64(r.k[b])
        vc = to_np64(r.v[b])
        ring = O.RingSeq(sinks=r.S, window=r.W, head=int(heads[b]), count=r.W, seq_len=r.n)
        slot_of = dict(zip(O.visible_positions(r.n - 1, r.S, r.W), ring.chronological_slots()))
        ref = O.decode_attention(q[b], lambda j: kc[:, slot_of[j]], lambda j: vc[:, slot_of[j]], r.n, r.S, r.W,
                                 r.Hkv)
        assert_bf16_close(out[b], ref)


def test_windowed_paged_decode_b256(env):
    R, torch, dev, WL = env
    wd = WL.WindowedPagedDecode(R, torch, dev)
    wd.decode()
    torch.cuda.synchronize()
    assert wd.err.item() == 0
    out, q = to_np64(wd.out), to_np64(wd.q)
    kp, vp = wd.k, wd.v
    for b in (0, 100, 255):
        n = int(wd.lens[b])
        row = wd.table_host[b]
        vis = O.visible_positions(n - 1, wd.S, wd.W)
        blocks = sorted({row[j // 16] for j in vis})
        idx = torch.tensor(blocks, dtype=torch.long, device=kp.device)
        kb = dict(zip(blocks, to_np64(kp[idx])))
        vb = dict(zip(blocks, to_np64(vp[idx])))
        ref = O.decode_attention(q[b], lambda j: kb[row[j // 16]][:, j % 16], lambda j: vb[row[j // 16]][:, j % 16],
                                 n, wd.S, wd.W, wd.Hkv)
        assert_bf16_close(out[b], ref)


def test_prefill_t8192_sampled_rows(env):
    R, torch, dev, WL = env
    pf = WL.Prefill(R, torch, dev)
    pf.run()
    torch.cuda.synchronize()
    assert pf.int_state[3].item() == 0
    q, k, v, out = to_np64(pf.q), to_np64(pf.k), to_np64(pf.v), to_np64(pf.out)
    for t in (0, 1, 15, 16, 63, 64, 4095, 4099, 4100, 4101, 5000, 8191):
        ref = O.decode_attention(q[t], lambda j: k[j], lambda j: v[j], t + 1, pf.S, pf.W, pf.Hkv)
        assert_bf16_close(out[t], ref)


@pytest.mark.parametrize("kind", ["f16", "i8", "i8_keep", "i8_hadamard"])
def test_rerotate_l64_t524288_sampled_rows(env, kind):
    R, torch, dev, WL = env
    rr = WL.Rerotate(R, torch, dev, kind=kind)
    rows = synth.rng(77).integers(0, rr.L * rr.T * rr.Hkv, 512)
    flat = rr.k.view(-1, rr.d)
    idx = torch.from_numpy(rows).to(dev)
    before = flat[idx].cpu().numpy()
    sc_before = rr.scale.view(-1)[idx].cpu().numpy() if kind != "f16" else None
    rr.run(1.0, 1.125)
    torch.cuda.synchronize()
    after = flat[idx].cpu().numpy()
    positions = (rows // rr.Hkv) % rr.T
    ca, cb = oracle_cfg(rr.cfg(1.0)), oracle_cfg(rr.cfg(1.125))
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
