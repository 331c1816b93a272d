"""Helpers for the GPU parity tests: device buffers, comparisons, oracle glue."""
from __future__ import annotations

import numpy as np

from oracle import ropekv_oracle as O


def torch_dev():
    import torch

    if not torch.cuda.is_available():
        import pytest

        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_np64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """x rounded to the nearest bf16 on the host (what a bf16 tensor holds for the exact value x),
    back in fp64: the oracle's rotated q and k as the bf16 activations and cache store them."""
    import torch

    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def normwise(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over the whole tensor."""
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(gpu - ref))) / (den if den > 0 else 1.0)


def rowwise(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis) of max |gpu - ref| / max |ref| of that row."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    den = np.maximum(np.max(np.abs(r), axis=1), 1e-30)
    return float(np.max(np.max(np.abs(g - r), axis=1) / den))


def assert_bf16_rounded(gpu: np.ndarray, ref: np.ndarray, rel_fp32=1e-6):
    """gpu is the exact value ref, computed in fp32 and rounded once to bf16 (round to nearest):
    |gpu - ref| <= ulp(gpu) / 2 + e, with ulp(g) = 2^(floor(log2 |g|) - 7) (8 significant bits) and
    e = rel_fp32 * (the row's largest |ref|) a bound on the fp32 arithmetic before the rounding (a
    few fp32 roundings of products of the inputs and the cos / sin table, ~1e-7).  A value one
    bf16 step off fails unless ref lies within e of the midpoint between the two."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    e = rel_fp32 * np.max(np.abs(r), axis=1, keepdims=True)
    _, ex = np.frexp(g)  # g = m 2^ex, 0.5 <= |m| < 1: ulp = 2^(ex - 8)
    half = np.where(g == 0, 0.0, np.ldexp(1.0, ex - 9))
    excess = np.abs(g - r) - (half + e)
    assert float(np.max(excess)) <= 0.0, (
        f"max excess {float(np.max(excess)):.3e} over half a bf16 ulp, max abs err {float(np.max(np.abs(g - r))):.3e}")


def assert_f16_rounded(gpu: np.ndarray, ref: np.ndarray, rel_fp32=1e-6):
    """gpu is the exact value ref, computed in fp32 and rounded once to IEEE half (round to
    nearest): |gpu - ref| <= ulp / 2 + e, with ulp = 2^(max(floor(log2 |g|), -14) - 10) (11
    significant bits, subnormals below 2^-14 on the fixed 2^-24 grid), and e as for bf16."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    e = rel_fp32 * np.max(np.abs(r), axis=1, keepdims=True)
    _, ex = np.frexp(g)  # floor(log2 |g|) = ex - 1
    half = np.ldexp(1.0, np.maximum(ex - 1, -14) - 11)
    excess = np.abs(g - r) - (half + e)
    assert float(np.max(excess)) <= 0.0, (
        f"max excess {float(np.max(excess)):.3e} over half an fp16 ulp, max abs err {float(np.max(np.abs(g - r))):.3e}")


def assert_rounded_once(gpu: np.ndarray, ref: np.ndarray, dtype_name: str, rel_fp32=1e-6):
    """One rounding of the exact value to the stored dtype ("f32", "bf16", "f16"); fp32 stores the
    fp32 arithmetic itself, within rel_fp32 of the row's largest |ref|."""
    if dtype_name == "bf16":
        assert_bf16_rounded(gpu, ref, rel_fp32)
    elif dtype_name == "f16":
        assert_f16_rounded(gpu, ref, rel_fp32)
    else:
        assert rowwise(gpu, ref) <= rel_fp32, f"fp32 row error {rowwise(gpu, ref):.3e}"


def assert_bf16_close(gpu: np.ndarray, ref: np.ndarray, atol=2e-2, rtol=1e-2):
    err = np.abs(gpu - ref) - (atol + rtol * np.abs(ref))
    assert float(np.max(err)) <= 0.0, f"max excess {float(np.max(err)):.3e}, max abs err {float(np.max(np.abs(gpu-ref))):.3e}"


def assert_bf16_attention(gpu: np.ndarray, ref: np.ndarray, ref_abs: np.ndarray):
    """The bound a bf16 attention output's own roundings imply.  The kernels round each weight P_j
    once to bf16 (relative error <= 2^-8) and sum in fp32, which moves the weighted average by at
    most 2^-8 (A + |out|), A = sum_j w_j |v_j| (the same attention over |V|, ref_abs); the output's
    rounding to bf16 adds half an ulp <= 2^-8 |out|.  The 5 % and 1e-5 A margins cover the fp32
    score and exp2 arithmetic (relative ~1e-4 at the needle rows' scores)."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    a = ref_abs.reshape(-1, ref_abs.shape[-1])
    bound = 1.05 * 2.0 ** -8 * (a + 2.0 * np.abs(r)) + 1e-5 * np.max(a, axis=1, keepdims=True)
    excess_ = np.abs(g - r) - bound
    assert float(np.max(excess_)) <= 0.0, (
        f"max excess {float(np.max(excess_)):.3e} over the bf16 rounding bound (max abs err "
        f"{float(np.max(np.abs(g - r))):.3e})")


def bf16_attention_ref(gpu: np.ndarray, attention, q, kfn, vfn, *args, **kw):
    """ref = attention(q, kfn, vfn, *args, **kw), an oracle attention; gpu is checked against it at
    the stated bf16 tolerance (2e-2 + 1e-2 |ref|) and at the tighter bound of its roundings
    (assert_bf16_attention, with the same attention over |V|).  Returns ref."""
    ref = attention(q, kfn, vfn, *args, **kw)
    ref_abs = attention(q, kfn, lambda j: np.abs(vfn(j)), *args, **kw)
    assert_bf16_close(gpu, ref)
    assert_bf16_attention(gpu, ref, ref_abs)
    return ref


def oracle_cfg(cfg) -> O.RopeCfg:
    """The oracle's view of a ctypes RopeCfg (same numbers)."""
    types = {0: "yarn", 1: "linear", 2: "ntk", 3: "dynamic_ntk", 4: "llama3"}
    return O.RopeCfg(head_dim=cfg.head_dim, rotary_dim=cfg.rotary_dim, rope_theta=cfg.rope_theta,
                     yarn_factor=cfg.yarn_factor, orig_max_pos=cfg.orig_max_pos, beta_fast=cfg.beta_fast,
                     beta_slow=cfg.beta_slow, extrapolation_factor=cfg.extrapolation_factor, neox=bool(cfg.neox),
                     rope_type=types[cfg.rope_type], pruned_pairs=cfg.pruned_pairs, served_len=cfg.served_len,
                     low_freq_factor=cfg.low_freq_factor, high_freq_factor=cfg.high_freq_factor)


def _kv_kind(R, torch, dtype):
    """(kv_dtype, torch storage dtype, has row scales) of a cache dtype: a torch dtype, or
    "fp8" for E4M3 codes held as raw bytes (uint8)."""
    if dtype == "fp8":
        return R.FP8, torch.uint8, True
    kvdt = {torch.float32: R.F32, torch.bfloat16: R.BF16, torch.float16: R.F16, torch.int8: R.I8}[dtype]
    return kvdt, dtype, dtype == torch.int8


class DevRing:
    """A RING cache in device memory (torch) plus its descriptor."""

    def __init__(self, R, torch, dev, dtype, B, Hkv, d, S, W):
        self.C = S + W
        kvdt, store, coded = _kv_kind(R, torch, dtype)
        self.k = torch.zeros(B, Hkv, self.C, d, dtype=store, device=dev)
        self.v = torch.zeros_like(self.k)
        self.head = torch.zeros(B, dtype=torch.int32, device=dev)
        self.count = torch.zeros(B, dtype=torch.int32, device=dev)
        self.seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        # 8-bit caches: one fp32 scale per cached row, K and V
        self.k_scale = torch.zeros(B, Hkv, self.C, dtype=torch.float32, device=dev) if coded else None
        self.v_scale = torch.zeros_like(self.k_scale) if coded else None
        self.desc = R.kv_cache(R.RING, kvdt, Hkv, d, self.k, self.v, batch=B, capacity=self.C, sinks=S, window=W,
                               ring_head=self.head, ring_count=self.count, seq_len=self.seq_len, err_word=self.err,
                               k_scale=self.k_scale, v_scale=self.v_scale)


class DevPaged:
    """A PAGED cache (pool + block table) in device memory plus its descriptor."""

    def __init__(self, R, torch, dev, dtype, B, Hkv, d, S, W, table: np.ndarray, num_blocks: int, bs: int = 16):
        kvdt, store, coded = _kv_kind(R, torch, dtype)
        self.k = torch.zeros(num_blocks, Hkv, bs, d, dtype=store, device=dev)
        self.v = torch.zeros_like(self.k)
        self.table = torch.from_numpy(np.ascontiguousarray(table.astype(np.int32))).to(dev)
        self.seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.k_scale = torch.zeros(num_blocks, Hkv, bs, dtype=torch.float32, device=dev) if coded else None
        self.v_scale = torch.zeros_like(self.k_scale) if coded else None
        self.desc = R.kv_cache(R.PAGED, kvdt, Hkv, d, self.k, self.v, batch=B, sinks=S, window=W, block_size=bs,
                               max_blocks=table.shape[1], num_blocks=num_blocks, block_table=self.table,
                               seq_len=self.seq_len, err_word=self.err, k_scale=self.k_scale, v_scale=self.v_scale)


# ------------------------------------------------------------------ 8-bit codes: rounding-edge validity
#
# A kernel and the oracle decide an 8-bit code from the same quotient x / scale but by different
# float32 arithmetic: the kernels rotate in float32 with a float32 table (the oracle in fp64) and
# re-quantise turned rows by a product with the correctly rounded reciprocal 127 / max (the oracle
# divides).  So a kernel code may land on the other side of a rounding boundary.  It may differ from
# the oracle's code only by one step, and only where the oracle's exact fp64 quotient lies within
# eps of the boundary between the two codes.  Values that are never rotated (the appended V rows)
# go through the same IEEE float32 division on both sides and are compared bit for bit instead.
#
# eps, in quotient units (code steps for int8):
#   append of a rotated key: float32 table entries (2^-24 relative each) and three float32
#     roundings of a pair, |pair| <= sqrt(2) max|x|, scaled by 127 / max|x|:
#     127 (2 + 3 sqrt(2)) 2^-24 ~ 4.7e-5 for int8; 448 x the same ~ 1.7e-4 for E4M3.
#     eps = 2.5e-4 (int8), 1e-3 (E4M3): about 5x margin.
#   re-rotation of int8 rows in code units: cos / sin of the reduced angle within 5e-7 (the
#     re-rotation's stated accuracy), gain <= 1.1, |c| <= 127, three float32 roundings, then the
#     new unit 127 / max|y| <= sqrt(2) per old unit: sqrt(2) (127 * 2 * 5e-7 * 1.1 + 3 * 127 * 2^-24)
#     ~ 2.3e-4.  eps = 1e-3.
#   Hadamard rows: the second transform of the turned row runs in float32 (7 butterfly levels over
#     values up to sqrt(128) * 127): about 1e-3 code steps at worst.  eps = 4e-3.
EPS_APPEND_I8 = 2.5e-4
EPS_APPEND_FP8 = 1e-3
EPS_TURN_I8 = 1e-3
EPS_TURN_HADAMARD = 4e-3


def assert_int8_codes_valid(got, want, quot, eps):
    """got, want: int8 codes; quot: the oracle's exact quotients (same shape).  Returns the number
    of codes that differ (each one step, at a rounding edge)."""
    g = np.asarray(got).astype(np.int32)
    w = np.asarray(want).astype(np.int32)
    diff = g - w
    assert int(np.max(np.abs(diff), initial=0)) <= 1, "a code differs by more than one step"
    bad = diff != 0
    if bad.any():
        edge = (g[bad] + w[bad]) / 2.0
        dist = np.abs(np.asarray(quot, dtype=np.float64)[bad] - edge)
        assert float(dist.max()) <= eps, (
            f"{int(bad.sum())} codes differ; worst is {float(dist.max()):.3e} from its rounding edge (eps {eps})")
    return int(bad.sum())


def decode_int8(codes, scale) -> np.ndarray:
    """Rows of an int8 cache read back for comparison: codes x the row's fp32 scale, float64
    (Hadamard rows stay in the transformed domain their codes live in)."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scale).astype(np.float64)[..., None]


def decode_e4m3(codes) -> np.ndarray:
    """E4M3 bytes read back for comparison, decoded by torch's float8_e4m3fn (bias 7, no
    infinities, largest finite 448), float64."""
    import torch

    u8 = np.ascontiguousarray(np.asarray(codes).view(np.uint8))
    return torch.from_numpy(u8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def oracle_written(kind, key):
    """A key as a cache written directly at its factor holds it, by the oracle's storage: fp16
    rounding to nearest ("f16"), or the oracle's row quantiser ("i8", "i8_keep"; for "i8_hadamard"
    the codes of H key, and the values stay in the H domain).  Returns (values, unit): the unit is an
    fp16 ulp of the row's largest stored value, or the row's quantisation step."""
    key = np.asarray(key, dtype=np.float64)
    if kind == "f16":
        vals = key.astype(np.float16).astype(np.float64)
        rowmax = np.max(np.abs(vals), axis=-1, keepdims=True)
        return vals, np.spacing(rowmax.astype(np.float16)).astype(np.float64)
    codes, scale = O.quant_int8_hadamard_rows(key) if kind == "i8_hadamard" else O.quant_int8_rows(key)
    return O.dequant_int8_rows(codes, scale), np.asarray(scale, dtype=np.float64)[..., None]


def _e4m3_ordinal(codes):
    u = np.asarray(codes).view(np.uint8).astype(np.int32)
    return np.where(u & 0x80, -(u & 0x7F), u)


def assert_fp8_codes_valid(got, want, quot, eps):
    """As assert_int8_codes_valid for E4M3 bytes: neighbouring values (ordinal step one), the
    oracle's quotient within eps of the midpoint of the two values (+0 and -0 count as equal)."""
    og, ow = _e4m3_ordinal(got), _e4m3_ordinal(want)
    diff = og - ow
    assert int(np.max(np.abs(diff), initial=0)) <= 1, "an E4M3 code differs by more than one step"
    bad = diff != 0
    if bad.any():
        mid = (decode_e4m3(np.asarray(got)[bad]) + decode_e4m3(np.asarray(want)[bad])) / 2.0
        q = np.clip(np.asarray(quot, dtype=np.float64)[bad], -O.E4M3_MAX, O.E4M3_MAX)
        dist = np.abs(q - mid)
        assert float(dist.max()) <= eps, (
            f"{int(bad.sum())} codes differ; worst is {float(dist.max()):.3e} from its rounding edge (eps {eps})")
    return int(bad.sum())


def int8_turn_quotients(kind, codes, scale, positions, cfg_from, cfg_to, new_scale, kept=None):
    """The oracle's exact quotients behind re-rotated int8 codes: the fp64 turned row (in the H
    domain for Hadamard rows) over the scale the codes are taken against (the new one, or the
    old one for rows that keep their scale)."""
    x = O.dequant_int8_rows(codes, scale)
    if kind == "i8_hadamard":
        y = O.hadamard(O.rerotate_rows(O.hadamard(x), positions, cfg_from, cfg_to))
    else:
        y = O.rerotate_rows(x, positions, cfg_from, cfg_to)
    s = np.asarray(new_scale, dtype=np.float32)
    if kept is not None:
        s = np.where(kept, np.asarray(scale, dtype=np.float32), s)
    return O.row_quotients(y, s)


def seeded_int8_rows(shape, seed, rot_dims, rot_amp):
    """int8 rows: rotary dims uniform in [-rot_amp, rot_amp], the rest in [-127, 127]; scales U(0.01, 0.03).
    Odd rows use the full range in the rotary dims too (those rows tend to overflow a turn)."""
    from sliding_window_kv_amd import synth

    rng = synth.rng(seed)
    codes = rng.integers(-127, 128, size=shape).astype(np.int8)
    small = rng.integers(-rot_amp, rot_amp + 1, size=shape[:-1] + (rot_dims,)).astype(np.int8)
    rows = codes.reshape(-1, shape[-1])
    srows = small.reshape(-1, rot_dims)
    rows[0::2, :rot_dims] = srows[0::2]
    scale = (rng.random(shape[:-1], dtype=np.float32) * 0.02 + 0.01).astype(np.float32)
    return codes, scale


def check_keep_scale_rows(before, sc_before, after, sc_after, positions, cfg_from, cfg_to):
    """Keep-scale re-rotation of int8 rows, checked row by row against the branch the kernel took.

    A row the kernel kept (scale unchanged) must have its tail codes bit for bit and rotary codes
    valid against rne(y / old scale); a row it re-quantised must match the oracle's whole-row
    quantiser of y (scale to 5e-6, codes valid).  The kernel's decision may differ from the
    oracle's only where the row's largest turned rotary quotient at the old scale sits at the
    re-coding edge 127.5.  Returns (rows kept, rows re-quantised)."""
    r = cfg_to.rotary_dim
    codes_o, scale_o, over_o = O.rerotate_int8_keep_scale_rows(before, sc_before, positions, cfg_from, cfg_to)
    y = O.rerotate_rows(O.dequant_int8_rows(before, sc_before), positions, cfg_from, cfg_to)
    kept = np.asarray(sc_after) == np.asarray(sc_before)
    q_old = O.row_quotients(y[:, :r], sc_before)
    dis = kept == over_o
    if dis.any():
        edge = np.max(np.abs(q_old[dis]), axis=1)
        assert np.all(np.abs(edge - 127.5) <= EPS_TURN_I8), edge
    if kept.any():
        assert np.array_equal(after[kept, r:], before[kept, r:])
        want = np.rint(q_old[kept].astype(np.float32)).astype(np.int32)
        assert_int8_codes_valid(after[kept, :r], want, q_old[kept], EPS_TURN_I8)
    req = ~kept
    if req.any():
        full_c, full_s = O.quant_int8_rows(y[req])
        np.testing.assert_allclose(sc_after[req], full_s, rtol=5e-6)
        assert_int8_codes_valid(after[req], full_c, O.row_quotients(y[req], full_s), EPS_TURN_I8)
    return int(kept.sum()), int(req.sum())


# ------------------------------------------------------------------ needles: full-size attention parity with power
#
# With N(0, 1) queries, keys and values, an attention output over n keys is a mean of ~n / e
# values and only ~1/sqrt(n) in size: at full size it sits below the bf16 tolerance
# 2e-2 + 1e-2 |ref|, so a dropped sink, an off-by-one window edge or a wrong block would pass.
# These helpers plant needles.  The tested queries get a component beta * u_g along a unit
# direction u_g of their KV head g (beta = sqrt(d)), and keys at chosen positions are set to
# alpha * u_g: a needle scores alpha (1 + N(0, 1) / sqrt(d)) ~ 16 nats, the background keys
# N(0, 2), so the visible needles carry > 99 % of the softmax mass even over 131072 keys.  Their
# values are distinct N(0, gamma^2) rows (gamma 4), so the output is about the mean of the visible
# needles' values and a needle wrongly dropped or admitted moves it by O(1).  Each test also checks
# that the oracle over a wrong visible set (shifted window, no sinks, a dropped block...) fails the
# same tolerance: the comparison has the power to see that mistake.
NEEDLE_ALPHA = 16.0
NEEDLE_GAMMA = 4.0


def needle_dirs(Hkv, d, seed):
    """One unit direction per KV head, float64 [Hkv, d]."""
    from sliding_window_kv_amd import synth

    u = synth.normal((Hkv, d), seed).astype(np.float64)
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def plant_queries_(torch, q, u):
    """q: device tensor [..., Hq, d]; adds sqrt(d) u_g to every query head of KV head g, in place."""
    Hq, d = q.shape[-2], q.shape[-1]
    n_rep = Hq // u.shape[0]
    add = torch.from_numpy(np.repeat(u, n_rep, axis=0) * np.sqrt(d)).to(q.device, torch.float32)
    q.copy_((q.float() + add).to(q.dtype))


def needle_kv(u, n, seed):
    """n needle rows: keys alpha u_g, values N(0, gamma^2); float64 [n, Hkv, d] each."""
    from sliding_window_kv_amd import synth

    K = np.broadcast_to(NEEDLE_ALPHA * u, (n,) + u.shape).copy()
    V = NEEDLE_GAMMA * synth.normal((n,) + u.shape, seed).astype(np.float64)
    return K, V


def excess(gpu, ref, atol=2e-2, rtol=1e-2):
    """max(|gpu - ref| - (atol + rtol |ref|)): > 0 means the bf16 comparison fails."""
    return float(np.max(np.abs(gpu - ref) - (atol + rtol * np.abs(ref))))


def attend_set(q, K, V, idx, Hkv):
    """The oracle's attention of q [Hq, d] over the rows idx of K, V [n, Hkv, d] (a wrong visible
    set for a negative control, or the true one)."""
    import math

    Hq, d = q.shape
    n_rep = Hq // Hkv
    idx = np.asarray(idx)
    out = np.empty((Hq, d))
    for g in range(Hkv):
        Kg, Vg = K[idx, g], V[idx, g]
        for h in range(g * n_rep, (g + 1) * n_rep):
            out[h] = O.attend(q[h], Kg, Vg, 1.0 / math.sqrt(d))
    return out
