"""Host-side checks of the C ABI (CPU only, no kernel launches).

The library loads, exports every entry point include/ropekv.h declares, the
ctypes structures match the C layout, and every argument check returns its
error code before anything reaches the GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ropekv.h")
LIB = os.path.join(ROOT, "sliding_window_kv_amd", "libropekv.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libropekv.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ropekv_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ropekv_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    from sliding_window_kv_amd import ropekv

    assert sorted(ropekv.EXPORTS) == names


def test_struct_layout_matches_c(tmp_path):
    from sliding_window_kv_amd import ropekv as R

    fields_rc = [f for f, _ in R.RopeCfg._fields_]
    fields_kv = [f for f, _ in R.KVCache._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "ropekv.h"', "int main(void){"]
    prog.append('printf("%zu\\n", sizeof(ropekv_rope_cfg));')
    for f in fields_rc:
        prog.append(f'printf("%zu\\n", offsetof(ropekv_rope_cfg, {f}));')
    prog.append('printf("%zu\\n", sizeof(ropekv_kv_cache));')
    for f in fields_kv:
        prog.append(f'printf("%zu\\n", offsetof(ropekv_kv_cache, {f}));')
    prog.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(R.RopeCfg)] + [getattr(R.RopeCfg, f).offset for f in fields_rc]
    want += [ctypes.sizeof(R.KVCache)] + [getattr(R.KVCache, f).offset for f in fields_kv]
    assert got == want


FAKE = 0x1000  # a non-null pointer value; validation fails before anything dereferences it


def _ring(**kw):
    from sliding_window_kv_amd import ropekv as R

    args = dict(batch=1, capacity=16, sinks=4, window=12, k=FAKE, v=FAKE, ring_head=FAKE, ring_count=FAKE,
                seq_len=FAKE, err_word=FAKE)
    args.update(kw)
    return R.kv_cache(args.pop("layout", R.RING), args.pop("kv_dtype", R.F32), args.pop("num_kv_heads", 4),
                      args.pop("head_dim", 64), **args)


def test_build_table_argument_errors():
    from sliding_window_kv_amd import ropekv as R

    f = R.raw("ropekv_build_table")
    bad = [R.rope_cfg(64, 63), R.rope_cfg(64, 0), R.rope_cfg(32, 64), R.rope_cfg(64, 64, rope_theta=1.0),
           R.rope_cfg(64, 64, yarn_factor=2.0, orig_max_pos=0)]
    for cfg in bad:
        assert f(ctypes.byref(cfg), 16, FAKE, None, None) == R.EINVAL
        assert R.last_error() != ""
    bad2 = [R.rope_cfg(64, 64, rope_type=9), R.rope_cfg(64, 64, pruned_pairs=33),
            R.rope_cfg(64, 64, rope_type=R.ROPE_DYNAMIC_NTK, yarn_factor=8.0, served_len=10, orig_max_pos=4096),
            R.rope_cfg(64, 64, rope_type=R.ROPE_LLAMA3, yarn_factor=8.0, low_freq_factor=4.0, high_freq_factor=1.0),
            R.rope_cfg(64, 64, rope_type=R.ROPE_LINEAR, yarn_factor=0.0)]
    for cfg in bad2:
        assert f(ctypes.byref(cfg), 16, FAKE, None, None) == R.EINVAL, R.last_error()
    good = R.rope_cfg(64, 64)
    assert f(ctypes.byref(good), 0, FAKE, None, None) == R.EINVAL
    assert f(ctypes.byref(good), 16, None, None, None) == R.EINVAL
    assert f(None, 16, FAKE, None, None) == R.EINVAL


def test_apply_append_argument_errors():
    from sliding_window_kv_amd import ropekv as R

    f = R.raw("ropekv_apply_append")
    cfg = R.rope_cfg(64, 64)

    def call(cache, **kw):
        a = dict(table=FAKE, table_len=100, q=FAKE, nq=8, k=FAKE, v=FAKE, act=R.F32, n=4, pos=FAKE, seq=FAKE,
                 freed=None, cap=0, nfreed=None)
        a.update(kw)
        return f(ctypes.byref(cfg), a["table"], a["table_len"], a["q"], a["nq"], a["k"], a["v"], a["act"], a["n"],
                 a["pos"], a["seq"], ctypes.byref(cache) if cache is not None else None, a["freed"], a["cap"],
                 a["nfreed"], None)

    assert call(_ring(capacity=15)) == R.EINVAL               # C != S + W
    assert call(_ring(window=0, capacity=4)) == R.EINVAL      # ring without a window
    assert call(_ring(kv_dtype=R.BF16)) == R.EDTYPE           # act != kv dtype
    assert call(_ring(), act=R.I8) == R.EDTYPE
    assert call(_ring(head_dim=128)) == R.EINVAL              # cfg / cache head_dim mismatch
    assert call(_ring(), q=None) == R.EINVAL                  # q missing with n_q_heads > 0
    assert call(_ring(), seq=None) == R.EINVAL
    assert call(_ring(), table_len=0) == R.EINVAL
    assert call(_ring(err_word=None)) == R.EINVAL
    assert call(_ring(layout=7)) == R.ELAYOUT
    assert call(None) == R.EINVAL
    assert call(_ring(), freed=FAKE, nfreed=None) == R.EINVAL
    assert call(_ring(), n=0) == R.OK                         # nothing to do, nothing launched
    assert call(_ring(kv_dtype=R.I8)) == R.EINVAL             # int8 cache without scales
    assert call(_ring(kv_dtype=R.I8, k_scale=FAKE)) == R.EINVAL  # int8 cache without value scales
    assert call(_ring(kv_dtype=R.I8, k_scale=FAKE, v_scale=FAKE), n=0) == R.OK
    assert call(_ring(k_int8_mode=R.I8_HADAMARD)) == R.EINVAL  # int8 key modes need an I8 cache
    i8 = dict(kv_dtype=R.I8, k_scale=FAKE, v_scale=FAKE)
    assert call(_ring(k_int8_mode=4, **i8)) == R.EINVAL       # unknown mode bit
    assert call(_ring(k_int8_mode=R.I8_HADAMARD | R.I8_KEEP_SCALE, **i8)) == R.EINVAL
    assert call(_ring(k_int8_mode=R.I8_HADAMARD, head_dim=96, **i8)) == R.ERANGE  # H needs d = 2^k
    assert call(_ring(k=FAKE + 8)) == R.EINVAL                # cache pools must be 16-byte aligned
    assert call(_ring(kv_dtype=R.I8, k_scale=FAKE, v_scale=FAKE + 4)) == R.EINVAL
    # E4M3 caches: the same scale rules as int8, no int8 key modes
    assert call(_ring(kv_dtype=R.FP8)) == R.EINVAL
    assert call(_ring(kv_dtype=R.FP8, k_scale=FAKE)) == R.EINVAL
    assert call(_ring(kv_dtype=R.FP8, k_scale=FAKE, v_scale=FAKE), n=0) == R.OK
    assert call(_ring(kv_dtype=R.FP8, k_scale=FAKE, v_scale=FAKE, k_int8_mode=R.I8_KEEP_SCALE)) == R.EINVAL
    assert call(_ring(), act=R.FP8) == R.EDTYPE               # activations are never 8-bit
    assert call(_ring(kv_dtype=5, k_scale=FAKE, v_scale=FAKE)) == R.EDTYPE


def test_attention_argument_errors():
    from sliding_window_kv_amd import ropekv as R

    dec = R.raw("ropekv_decode_attn")
    pre = R.raw("ropekv_prefill_attn")
    c = _ring()
    assert dec(FAKE, 1, 6, ctypes.byref(c), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.EINVAL   # 6 % 4
    assert dec(FAKE, 1, 64, ctypes.byref(c), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.ERANGE  # n_rep 16
    assert dec(FAKE, 2, 8, ctypes.byref(c), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.EINVAL   # batch > cache batch
    assert dec(FAKE, 1, 8, ctypes.byref(c), 0.0, None, FAKE, FAKE, 1, None) == R.ENOSPACE       # workspace
    assert dec(FAKE, 1, 8, ctypes.byref(c), float("nan"), None, FAKE, FAKE, 1 << 30, None) == R.EINVAL
    c2 = _ring(head_dim=96)
    assert dec(FAKE, 1, 8, ctypes.byref(c2), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.ERANGE
    c3 = _ring(kv_dtype=R.F16)
    assert dec(FAKE, 1, 8, ctypes.byref(c3), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.EDTYPE
    assert dec(FAKE + 2, 1, 8, ctypes.byref(c), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.EINVAL  # q alignment
    assert pre(FAKE, FAKE, FAKE, 8, 0, 8, ctypes.byref(c), 0, 0.0, None, FAKE + 4, None) == R.EINVAL  # out alignment
    c4 = _ring(kv_dtype=R.I8, k_scale=FAKE, v_scale=FAKE)
    assert dec(FAKE, 1, 8, ctypes.byref(c4), 0.0, None, FAKE, FAKE, 1, None) == R.ENOSPACE      # int8 accepted
    assert pre(FAKE, FAKE, FAKE, 8, 5, 8, ctypes.byref(c4), 0, 0.0, None, FAKE, None) == R.EDTYPE  # prefill: no int8
    c5 = _ring(kv_dtype=R.FP8, k_scale=FAKE, v_scale=FAKE)
    assert dec(FAKE, 1, 8, ctypes.byref(c5), 0.0, None, FAKE, FAKE, 1, None) == R.ENOSPACE      # E4M3 accepted
    assert pre(FAKE, FAKE, FAKE, 8, 5, 8, ctypes.byref(c5), 0, 0.0, None, FAKE, None) == R.EDTYPE
    contig = R.kv_cache(R.CONTIG, R.F32, 4, 64, FAKE, capacity=10, err_word=FAKE)
    assert dec(FAKE, 1, 8, ctypes.byref(contig), 0.0, None, FAKE, FAKE, 1 << 30, None) == R.ELAYOUT
    assert pre(FAKE, FAKE, FAKE, 8, 5, 8, ctypes.byref(contig), 0, 0.0, None, FAKE, None) == R.ELAYOUT  # prefix needs cache
    assert pre(FAKE, FAKE, FAKE, 8, 5, 8, ctypes.byref(c), 3, 0.0, None, FAKE, None) == R.EINVAL        # seq outside batch
    assert pre(FAKE, FAKE, FAKE, -1, 0, 8, ctypes.byref(c), 0, 0.0, None, FAKE, None) == R.EINVAL
    assert pre(FAKE, FAKE, FAKE, 0, 0, 8, ctypes.byref(c), 0, 0.0, None, FAKE, None) == R.OK


def test_decode_noalloc_argument_errors():
    # the allocation-free decode shares the workspace call's checks and refuses plans whose
    # split-K partials exceed its fixed 64 MiB array, all before any launch
    from sliding_window_kv_amd import ropekv as R

    f = R.raw("ropekv_decode_attn_noalloc")
    c = _ring()
    assert f(FAKE, 1, 6, ctypes.byref(c), 0.0, None, FAKE, None) == R.EINVAL      # 6 % 4
    assert f(FAKE, 1, 64, ctypes.byref(c), 0.0, None, FAKE, None) == R.ERANGE     # n_rep 16
    assert f(FAKE, 2, 8, ctypes.byref(c), 0.0, None, FAKE, None) == R.EINVAL      # batch > cache batch
    assert f(FAKE + 2, 1, 8, ctypes.byref(c), 0.0, None, FAKE, None) == R.EINVAL  # q alignment
    assert f(FAKE, 1, 8, ctypes.byref(c), float("inf"), None, FAKE, None) == R.EINVAL
    assert f(FAKE, 1, 8, ctypes.byref(c), 0.0, None, None, None) == R.EINVAL      # out missing
    contig = R.kv_cache(R.CONTIG, R.F32, 4, 64, FAKE, capacity=10, err_word=FAKE)
    assert f(FAKE, 1, 8, ctypes.byref(contig), 0.0, None, FAKE, None) == R.ELAYOUT
    big = R.kv_cache(R.PAGED, R.BF16, 8, 128, FAKE, FAKE, batch=256, max_blocks=8192, num_blocks=1 << 21,
                     block_table=FAKE, seq_len=FAKE, err_word=FAKE)
    assert R.decode_workspace_size(256, 32, big) > 64 << 20
    assert f(FAKE, 256, 32, ctypes.byref(big), 0.0, None, FAKE, None) == R.ENOSPACE
    assert "scratch" in R.last_error()


def test_workspace_size_formula():
    from sliding_window_kv_amd import ropekv as R

    paged = R.kv_cache(R.PAGED, R.BF16, 8, 128, FAKE, FAKE, batch=64, max_blocks=2048, num_blocks=131072,
                       block_table=FAKE, seq_len=FAKE, err_word=FAKE)
    ws = R.decode_workspace_size(64, 32, paged)
    # [B, Hkv, splits, n_rep, d + 2] fp32; 2048 tiles split into 8..256 splits
    unit = 64 * 8 * 4 * 130 * 4
    assert ws % unit == 0 and 8 <= ws // unit <= 256
    assert R.decode_workspace_size(64, 30, paged) == 0


def test_rerotate_argument_errors():
    from sliding_window_kv_amd import ropekv as R

    f = R.raw("ropekv_rerotate")
    a = R.rope_cfg(128, 64, rope_theta=5e5)
    b = R.rope_cfg(128, 64, rope_theta=5e5, yarn_factor=2.0, orig_max_pos=262144)
    contig = R.kv_cache(R.CONTIG, R.F16, 8, 128, FAKE, capacity=100, err_word=FAKE)
    ring = _ring()
    assert f(ctypes.byref(a), ctypes.byref(b), ctypes.byref(ring), 1, None) == R.ELAYOUT
    assert f(ctypes.byref(a), ctypes.byref(b), ctypes.byref(contig), 0, None) == R.EINVAL
    c = R.rope_cfg(128, 32, rope_theta=5e5)
    assert f(ctypes.byref(a), ctypes.byref(c), ctypes.byref(contig), 1, None) == R.EINVAL
    i8 = R.kv_cache(R.CONTIG, R.I8, 8, 128, FAKE, capacity=100, err_word=FAKE)  # no scale
    assert f(ctypes.byref(a), ctypes.byref(b), ctypes.byref(i8), 1, None) == R.EINVAL
    i8b = R.kv_cache(R.CONTIG, R.I8, 8, 128, FAKE, capacity=100, err_word=FAKE, k_scale=FAKE)
    d = R.rope_cfg(128, 48, rope_theta=5e5)
    e = R.rope_cfg(128, 48, rope_theta=5e5, yarn_factor=2.0, orig_max_pos=262144)
    assert f(ctypes.byref(d), ctypes.byref(e), ctypes.byref(i8b), 1, None) == R.ERANGE
    i8h = R.kv_cache(R.CONTIG, R.I8, 8, 128, FAKE, capacity=100, err_word=FAKE, k_scale=FAKE,
                     k_int8_mode=R.I8_HADAMARD)
    g = R.rope_cfg(128, 96, rope_theta=5e5)
    h = R.rope_cfg(128, 96, rope_theta=5e5, yarn_factor=2.0, orig_max_pos=262144)
    assert f(ctypes.byref(g), ctypes.byref(h), ctypes.byref(i8h), 1, None) == R.ERANGE  # H + NeoX: r = 2^k
    f8 = R.kv_cache(R.CONTIG, R.FP8, 8, 128, FAKE, capacity=100, err_word=FAKE, k_scale=FAKE)
    assert f(ctypes.byref(a), ctypes.byref(b), ctypes.byref(f8), 1, None) == R.EDTYPE    # no E4M3 re-rotation
