"""Thin ctypes binding of libropekv.so (argument marshalling only).

Every function here forwards to the C ABI in include/ropekv.h with the same
name minus the ``ropekv_`` prefix.  Tensors are torch tensors on the GPU; only
their data pointers cross the boundary.  There is no fallback path: if the
library is not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libropekv.so")

F32, BF16, F16, I8, FP8 = 0, 1, 2, 3, 4
RING, PAGED, CONTIG = 0, 1, 2
I8_KEEP_SCALE, I8_HADAMARD = 1, 2

DEV_TABLE_RANGE = 1
DEV_POSITION = 2
DEV_NULL_BLOCK = 4
DEV_BLOCK_RANGE = 8
DEV_SEQ_RANGE = 16
DEV_PREFIX_LOST = 32
DEV_FREE_OVERFLOW = 64

OK, EINVAL, EDTYPE, ERANGE, ELAYOUT, ENOSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6

EXPORTS = [
    "ropekv_build_table",
    "ropekv_apply_append",
    "ropekv_decode_workspace_size",
    "ropekv_decode_attn",
    "ropekv_decode_attn_noalloc",
    "ropekv_prefill_attn",
    "ropekv_rerotate",
    "ropekv_shift_keys",
    "ropekv_visible_slots",
    "ropekv_last_error",
]


class RopeCfg(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("neox", ctypes.c_int32),
        ("orig_max_pos", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("yarn_factor", ctypes.c_double),
        ("beta_fast", ctypes.c_double),
        ("beta_slow", ctypes.c_double),
        ("extrapolation_factor", ctypes.c_double),
        ("rope_type", ctypes.c_int32),
        ("pruned_pairs", ctypes.c_int32),
        ("served_len", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
    ]


class KVCache(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("sinks", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("pos0", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("ring_head", ctypes.c_void_p),
        ("ring_count", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_len", ctypes.c_void_p),
        ("err_word", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("k_int8_mode", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class RopeKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ropekv error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sliding_window_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    RC, KC = ctypes.POINTER(RopeCfg), ctypes.POINTER(KVCache)
    lib.ropekv_build_table.argtypes = [RC, I32, P, P, P]
    lib.ropekv_apply_append.argtypes = [RC, P, I32, P, I32, P, P, I32, I32, P, P, KC, P, I32, P, P]
    lib.ropekv_decode_workspace_size.argtypes = [I32, I32, KC]
    lib.ropekv_decode_workspace_size.restype = SZ
    lib.ropekv_decode_attn.argtypes = [P, I32, I32, KC, ctypes.c_float, P, P, P, SZ, P]
    lib.ropekv_decode_attn_noalloc.argtypes = [P, I32, I32, KC, ctypes.c_float, P, P, P]
    lib.ropekv_prefill_attn.argtypes = [P, P, P, I32, I32, I32, KC, I32, ctypes.c_float, P, P, P]
    lib.ropekv_rerotate.argtypes = [RC, RC, KC, I32, P]
    lib.ropekv_shift_keys.argtypes = [RC, KC, I32, I32, P]
    lib.ropekv_visible_slots.argtypes = [KC, I32, P, P, I32, P, P]
    lib.ropekv_last_error.argtypes = []
    lib.ropekv_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "ropekv_decode_workspace_size" and name != "ropekv_last_error":
            getattr(lib, name).restype = ctypes.c_int
    return lib


LIB = _load()


def last_error() -> str:
    return LIB.ropekv_last_error().decode()


def _check(rc: int) -> int:
    if rc != OK:
        raise RopeKVError(rc, last_error())
    return rc


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


ROPE_YARN, ROPE_LINEAR, ROPE_NTK, ROPE_DYNAMIC_NTK, ROPE_LLAMA3 = 0, 1, 2, 3, 4


def rope_cfg(head_dim, rotary_dim, rope_theta=10000.0, yarn_factor=1.0, orig_max_pos=4096, neox=True,
             beta_fast=32.0, beta_slow=1.0, extrapolation_factor=1.0, rope_type=ROPE_YARN, pruned_pairs=0,
             served_len=0, low_freq_factor=1.0, high_freq_factor=4.0) -> RopeCfg:
    return RopeCfg(head_dim=head_dim, rotary_dim=rotary_dim, neox=1 if neox else 0, orig_max_pos=orig_max_pos,
                   rope_theta=rope_theta, yarn_factor=yarn_factor, beta_fast=beta_fast, beta_slow=beta_slow,
                   extrapolation_factor=extrapolation_factor, rope_type=rope_type, pruned_pairs=pruned_pairs,
                   served_len=served_len, reserved=0, low_freq_factor=low_freq_factor,
                   high_freq_factor=high_freq_factor)


def kv_cache(layout, kv_dtype, num_kv_heads, head_dim, k, v=None, *, batch=0, capacity=0, sinks=0, window=0,
             block_size=16, max_blocks=0, num_blocks=0, pos0=0, k_scale=None, ring_head=None, ring_count=None,
             block_table=None, seq_len=None, err_word=None, v_scale=None, k_int8_mode=0) -> KVCache:
    return KVCache(layout=layout, kv_dtype=kv_dtype, num_kv_heads=num_kv_heads, head_dim=head_dim, batch=batch,
                   capacity=capacity, sinks=sinks, window=window, block_size=block_size, max_blocks=max_blocks,
                   num_blocks=num_blocks, pos0=pos0, k=_ptr(k), v=_ptr(v), k_scale=_ptr(k_scale),
                   ring_head=_ptr(ring_head), ring_count=_ptr(ring_count), block_table=_ptr(block_table),
                   seq_len=_ptr(seq_len), err_word=_ptr(err_word), v_scale=_ptr(v_scale),
                   k_int8_mode=k_int8_mode, reserved=0)


def build_table(cfg: RopeCfg, max_pos: int, cos_sin, mscale=None, stream=None) -> int:
    return _check(LIB.ropekv_build_table(ctypes.byref(cfg), max_pos, _ptr(cos_sin), _ptr(mscale), _stream(stream)))


def apply_append(cfg: RopeCfg, cos_sin, table_len: int, q, n_q_heads: int, k, v, act_dtype: int, n_tokens: int,
                 positions, seq_ids, cache: KVCache, freed_blocks=None, freed_capacity: int = 0, n_freed=None,
                 stream=None) -> int:
    return _check(LIB.ropekv_apply_append(ctypes.byref(cfg), _ptr(cos_sin), table_len, _ptr(q), n_q_heads, _ptr(k),
                                          _ptr(v), act_dtype, n_tokens, _ptr(positions), _ptr(seq_ids),
                                          ctypes.byref(cache), _ptr(freed_blocks), freed_capacity, _ptr(n_freed),
                                          _stream(stream)))


def decode_workspace_size(batch: int, n_q_heads: int, cache: KVCache) -> int:
    return int(LIB.ropekv_decode_workspace_size(batch, n_q_heads, ctypes.byref(cache)))


def decode_attn(q, batch: int, n_q_heads: int, cache: KVCache, scale: float, out, ws, ws_bytes: int,
                stream=None, sink_logits=None) -> int:
    return _check(LIB.ropekv_decode_attn(_ptr(q), batch, n_q_heads, ctypes.byref(cache), scale, _ptr(sink_logits),
                                         _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def decode_attn_noalloc(q, batch: int, n_q_heads: int, cache: KVCache, scale: float, out, stream=None,
                       sink_logits=None) -> int:
    return _check(LIB.ropekv_decode_attn_noalloc(_ptr(q), batch, n_q_heads, ctypes.byref(cache), scale,
                                                 _ptr(sink_logits), _ptr(out), _stream(stream)))


def prefill_attn(q, k, v, T: int, pos0: int, n_q_heads: int, cache: KVCache, seq_id: int, scale: float, out,
                 stream=None, sink_logits=None) -> int:
    return _check(LIB.ropekv_prefill_attn(_ptr(q), _ptr(k), _ptr(v), T, pos0, n_q_heads, ctypes.byref(cache),
                                          seq_id, scale, _ptr(sink_logits), _ptr(out), _stream(stream)))


def rerotate(cfg_from: RopeCfg, cfg_to: RopeCfg, cache: KVCache, n_layers: int, stream=None) -> int:
    return _check(LIB.ropekv_rerotate(ctypes.byref(cfg_from), ctypes.byref(cfg_to), ctypes.byref(cache), n_layers,
                                      _stream(stream)))


def shift_keys(cfg: RopeCfg, cache: KVCache, delta: int, n_layers: int = 1, stream=None) -> int:
    return _check(LIB.ropekv_shift_keys(ctypes.byref(cfg), ctypes.byref(cache), delta, n_layers, _stream(stream)))


def visible_slots(cache: KVCache, seq: int, positions_out, offsets_out, max_out: int, n_out, stream=None) -> int:
    return _check(LIB.ropekv_visible_slots(ctypes.byref(cache), seq, _ptr(positions_out), _ptr(offsets_out), max_out,
                                           _ptr(n_out), _stream(stream)))


def raw(fn_name: str):
    """The raw C function (for tests that check return codes without raising)."""
    return getattr(LIB, fn_name)
