"""Plain fp64 CPU oracle for RoPE/YaRN + sink/sliding-window KV caching.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
module.  The product path (the HIP library and its Python binding) never
imports or calls it, and this module imports nothing from the product path.

Everything here is written for a reader to check against the pages by eye:
no blocking, no fusion, no reordering beyond what each definition states.
All floating point is numpy float64 unless a function says otherwise.  The
8-bit quantisers take their integer decisions in float32 (the stored scales
are float32 and the pages fix no other precision), by the plain definition
code = rne(x / scale) with the quotient rounded once to float32.

Sources (cited by page title and section):
  [RoPE]   "RoPE, scaling, sliding window, attention sinks" (mlinterviewnotes,
           positional encoding and long context)
  [GOSS]   "Inference & 128K Long Context" (GPT-OSS-Lite docs, inference)
  [DYN]    "#2961 rope: --rope-scaling dynamic" (strata pull request)
  [SINK]   "Attention Sink 与 Streaming KV Cache" (llm-glossary, attention-sink)
  [VLLM]   "vLLM, from the inside out"

Parity status: every function below is pinned by a CPU test against values
the pages print, closed forms, invariants or brute force (tests/test_oracle_*.py);
none is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Configuration
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class RopeCfg:
    """The rope parameters the pages use ([RoPE] notation section, "YaRN, precisely").

    head_dim d_h, rotary_dim r <= d_h (leading slice, tail passes through),
    rope_theta b, yarn_factor s (s <= 1 means plain RoPE), orig_max_pos L0,
    beta_fast / beta_slow (defaults 32 / 1), extrapolation_factor (used in the
    blend; the pages give no default, 1.0 is taken), neox pairing flag.
    """

    head_dim: int
    rotary_dim: int
    rope_theta: float = 10000.0
    yarn_factor: float = 1.0          # the scaling factor s of every scheme below
    orig_max_pos: int = 4096          # L0, the trained context
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    extrapolation_factor: float = 1.0
    neox: bool = True
    rope_type: str = "yarn"           # "yarn" (plain when s <= 1), "linear", "ntk", "dynamic_ntk", "llama3"
    pruned_pairs: int = 0             # leading pairs kept unrotated (identity)
    served_len: int = 0               # dynamic NTK: the served length P
    low_freq_factor: float = 1.0      # Llama-3 blend
    high_freq_factor: float = 4.0


# --------------------------------------------------------------------------
# Frequencies, YaRN band, mscale   ([RoPE] frequency definition; "YaRN, precisely")
# --------------------------------------------------------------------------


def plain_inv_freq(rotary_dim: int, base: float) -> np.ndarray:
    """omega_i = 1 / b^(2i/r) for pair i = 0 .. r/2-1 ([RoPE] the inverse-frequency code)."""
    i2 = np.arange(0, rotary_dim, 2, dtype=np.float64)
    return 1.0 / (float(base) ** (i2 / rotary_dim))


def yarn_correction_dim(num_rotations: float, rotary_dim: int, base: float, orig_max_pos: int) -> float:
    """Pair index at which a pair turns `num_rotations` times within L0 ([RoPE] "YaRN, precisely")."""
    return (rotary_dim * math.log(orig_max_pos / (num_rotations * 2 * math.pi))) / (2 * math.log(base))


def yarn_correction_range(beta_fast, beta_slow, rotary_dim, base, orig_max_pos):
    """(low, high): floor of d(beta_fast) and ceil of d(beta_slow), clamped to [0, r-1].

    The body is not printed on the pages; this is the truncating reading the
    worked script in [RoPE] ("See the YaRN band for your own config") uses.
    """
    low = math.floor(yarn_correction_dim(beta_fast, rotary_dim, base, orig_max_pos))
    high = math.ceil(yarn_correction_dim(beta_slow, rotary_dim, base, orig_max_pos))
    return max(low, 0), min(high, rotary_dim - 1)


def yarn_ramp(low: float, high: float, n: int) -> np.ndarray:
    """Linear ramp clamped to [0, 1], with the +0.001 singularity guard ([RoPE] "YaRN, precisely")."""
    if low == high:
        high += 0.001
    x = (np.arange(n, dtype=np.float64) - low) / (high - low)
    return np.clip(x, 0.0, 1.0)


def yarn_mscale(scale: float) -> float:
    """mu = 0.1 ln s + 1 for s > 1, else 1 ([RoPE] "YaRN, precisely")."""
    if scale <= 1.0:
        return 1.0
    return 0.1 * math.log(scale) + 1.0


def yarn_inv_freq(cfg: RopeCfg) -> np.ndarray:
    """Per-pair angular frequency of the (possibly YaRN-scaled) rotation.

    Plain RoPE when s <= 1.  Otherwise the extrapolated set 1/b^(2i/r) and
    the interpolated set 1/(s b^(2i/r)) are blended by mask = (1 - ramp) *
    extrapolation_factor: mask 1 keeps the original frequency (fast pairs,
    below `low`), mask 0 divides it by s (slow pairs, above `high`)
    ([RoPE] "YaRN, precisely", the _compute_inv_freq excerpt).
    """
    r, b = cfg.rotary_dim, float(cfg.rope_theta)
    pos_freqs = b ** (np.arange(0, r, 2, dtype=np.float64) / r)
    extrap = 1.0 / pos_freqs
    s = float(cfg.yarn_factor)
    if s <= 1.0:
        return extrap
    interp = 1.0 / (s * pos_freqs)
    low, high = yarn_correction_range(cfg.beta_fast, cfg.beta_slow, r, b, cfg.orig_max_pos)
    mask = (1.0 - yarn_ramp(low, high, r // 2)) * cfg.extrapolation_factor
    return interp * (1.0 - mask) + extrap * mask


def ntk_base(base: float, factor: float, rotary_dim: int) -> float:
    """NTK-aware base: b * s^(r / (r - 2)) (the scheme edits the base, [RoPE] the four families)."""
    return base * factor ** (rotary_dim / (rotary_dim - 2))


def dynamic_ntk_base(base: float, factor: float, served: int, trained: int, rotary_dim: int) -> float:
    """Dynamic NTK: b * (s * P / L0 - (s - 1))^(r / (r - 2)) ([RoPE] the printed dynamic-NTK excerpt)."""
    return base * ((factor * served / trained) - (factor - 1)) ** (rotary_dim / (rotary_dim - 2))


def llama3_inv_freq(cfg: RopeCfg) -> np.ndarray:
    """Llama-3 blend ([RoPE] the four families): pairs whose wavelength is below L0 / high_freq_factor
    keep their frequency, pairs above L0 / low_freq_factor are divided by s, and between the two the
    frequency moves linearly in L0 / wavelength from one to the other."""
    w = plain_inv_freq(cfg.rotary_dim, cfg.rope_theta)
    s, L0 = float(cfg.yarn_factor), float(cfg.orig_max_pos)
    lo, hi = float(cfg.low_freq_factor), float(cfg.high_freq_factor)
    out = np.empty_like(w)
    for i, wi in enumerate(w):
        wavelen = 2 * math.pi / wi
        if wavelen < L0 / hi:
            out[i] = wi
        elif wavelen > L0 / lo:
            out[i] = wi / s
        else:
            smooth = (L0 / wavelen - lo) / (hi - lo)
            out[i] = (1 - smooth) * wi / s + smooth * wi
    return out


def inv_freq(cfg: RopeCfg) -> np.ndarray:
    """Per-pair angular frequency under cfg.rope_type, with the first pruned_pairs pairs at 0.

    "linear" is position interpolation: angles of position m / s ([RoPE] the PI
    note), i.e. every frequency divided by s.  "ntk" / "dynamic_ntk" recompute the
    base.  Pruned pairs rotate by nothing ([GOSS] pruned RoPE: cos 1, sin 0).
    """
    t = cfg.rope_type
    r, b, s = cfg.rotary_dim, float(cfg.rope_theta), float(cfg.yarn_factor)
    if t == "yarn":
        w = yarn_inv_freq(cfg)
    elif t == "linear":
        w = plain_inv_freq(r, b) / s
    elif t == "ntk":
        w = plain_inv_freq(r, ntk_base(b, s, r))
    elif t == "dynamic_ntk":
        w = plain_inv_freq(r, dynamic_ntk_base(b, s, cfg.served_len, cfg.orig_max_pos, r))
    elif t == "llama3":
        w = llama3_inv_freq(cfg)
    else:
        raise ValueError(f"unknown rope_type {t}")
    w = np.array(w, dtype=np.float64)
    w[: cfg.pruned_pairs] = 0.0
    return w


def mscale(cfg: RopeCfg) -> float:
    """The YaRN attention-temperature factor; the other schemes leave magnitudes alone."""
    return yarn_mscale(cfg.yarn_factor) if cfg.rope_type == "yarn" else 1.0


def build_table(cfg: RopeCfg, max_pos: int) -> np.ndarray:
    """cos/sin table [max_pos, r]: cos(m w_i) * mu in the first r/2 columns, sin in the rest.

    Angles are m * w_i in float64 ([RoPE] _compute_cos_sin_cache, scaled by
    mscale as in the YaRN variant).  Returns float64; a device table is this
    rounded once to float32.
    """
    w = inv_freq(cfg)
    m = np.arange(max_pos, dtype=np.float64)
    ang = np.outer(m, w)
    mu = mscale(cfg)
    return np.concatenate([np.cos(ang) * mu, np.sin(ang) * mu], axis=1)


# --------------------------------------------------------------------------
# Rotation   ([RoPE] the rotation excerpt and the NeoX / GPT-J pairing note)
# --------------------------------------------------------------------------


def pair_index(rotary_dim: int, neox: bool):
    """(first, second) element index of each rotary pair.

    NeoX pairs j with j + r/2; GPT-J pairs 2j with 2j + 1 ([RoPE] the
    is_neox_style branch).
    """
    half = rotary_dim // 2
    j = np.arange(half)
    if neox:
        return j, j + half
    return 2 * j, 2 * j + 1


def rope_apply(x: np.ndarray, positions: np.ndarray, table: np.ndarray, rotary_dim: int, neox: bool) -> np.ndarray:
    """Rotate the leading r dims of x[..., d] by the table row of each position.

    x has shape [N, ..., d]; positions has shape [N].  For each pair (a, c):
    (a cos - c sin, c cos + a sin); dims r..d-1 pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    half = rotary_dim // 2
    rows = table[np.asarray(positions, dtype=np.int64)]
    cos = rows[:, :half]
    sin = rows[:, half:]
    extra = x.ndim - 2
    cos = cos.reshape(cos.shape[0], *([1] * extra), half)
    sin = sin.reshape(sin.shape[0], *([1] * extra), half)
    i1, i2 = pair_index(rotary_dim, neox)
    out = x.copy()
    a = x[..., i1]
    c = x[..., i2]
    out[..., i1] = a * cos - c * sin
    out[..., i2] = c * cos + a * sin
    return out


def rotate_by_angle(x: np.ndarray, angles: np.ndarray, rotary_dim: int, neox: bool, gain: float = 1.0) -> np.ndarray:
    """Rotate each pair i of rows x[n, d] by angles[n, i] and multiply the pair by `gain`."""
    x = np.asarray(x, dtype=np.float64)
    i1, i2 = pair_index(rotary_dim, neox)
    c, s = np.cos(angles), np.sin(angles)
    out = x.copy()
    a = x[..., i1]
    b = x[..., i2]
    out[..., i1] = (a * c - b * s) * gain
    out[..., i2] = (b * c + a * s) * gain
    return out


# --------------------------------------------------------------------------
# Visible set   ([SINK] "可见集合与容量定义" and the C=6, S=2, T=10 table)
# --------------------------------------------------------------------------


def visible_positions(p: int, sinks: int, window: int) -> list[int]:
    """Logical positions visible to the query at absolute position p.

    sinks S, recent window W = C - S counting the current token.  A key j <= p
    is visible iff j < S or p - j < W.  window == 0 means full causal attention.
    """
    if window == 0:
        return list(range(p + 1))
    return [j for j in range(p + 1) if j < sinks or p - j < window]


# --------------------------------------------------------------------------
# Quantisers   ([DYN] "What it does": cached K is dequantised, turned and
# requantised; the 64-layer re-rotated caches keep one fp32 scale per row)
# --------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) via float32; returns float64 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_f16(x: np.ndarray) -> np.ndarray:
    """Round to IEEE half (nearest, ties to even); returns float64 values."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _row_scale(x: np.ndarray, qmax: float) -> np.ndarray:
    """scale = max|x| / qmax over the last axis, rounded once to float32 (the stored precision)."""
    amax = np.max(np.abs(np.asarray(x, dtype=np.float64)), axis=-1)
    return (amax / qmax).astype(np.float32)


def _quotients32(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x / scale per row, rounded once to float32; rows with scale 0 give 0.  For float32
    operands this is the IEEE float32 quotient (a float64 quotient rounded to float32 is
    correctly rounded)."""
    s = np.asarray(scale, dtype=np.float64)
    safe = np.where(s > 0, s, 1.0)
    q = (np.asarray(x, dtype=np.float64) / safe[..., None]).astype(np.float32)
    return np.where(s[..., None] > 0, q, np.float32(0.0)).astype(np.float32)


def quant_int8_rows(x: np.ndarray):
    """Per-row symmetric int8: scale = max|x| / 127, code = clamp(rne(x / scale), -127, 127).

    One scale per row of d dims (a per-row fp32 scale, as the re-rotated int8 caches keep).  The scale is
    max|x| / 127 rounded to float32, the precision it is stored in; each code
    rounds (to nearest, ties to even) the quotient x / scale taken against that
    stored scale and rounded to float32: the code whose multiple of the stored
    scale is nearest to x.  An all-zero row gets scale 0 and codes 0.
    Returns (codes int8 [..., d], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    scale = _row_scale(x, 127.0)
    q = np.clip(np.rint(_quotients32(x, scale)), -127, 127)
    return q.astype(np.int8), scale


def row_quotients(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x / scale per row in float64: the exact value a code rounds, for locating rounding edges."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64)
    safe = np.where(s > 0, s, 1.0)
    return np.where(s[..., None] > 0, x / safe[..., None], 0.0)


def dequant_int8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return codes.astype(np.float64) * scale.astype(np.float64)[..., None]


# 8-bit float E4M3 ([VLLM] memory levers: the KV cache itself stored as FP8).
# The pages name no FP8 layout; the reading taken is the OCP E4M3 "fn" format
# (the one this chip converts natively) with the same per-row absmax scale as
# the int8 rows, 448 (the largest E4M3 value) taking the place of 127.

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of each E4M3 byte: bit 7 the sign, bits 6..3 the exponent e (bias 7), bits 2..0
    the mantissa m.  e = 0 is subnormal, m / 8 * 2^-6; otherwise (1 + m / 8) * 2^(e - 7).
    S.1111.111 is NaN; there are no infinities, so the largest value is 1.75 * 2^8 = 448."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def round_e4m3(y) -> np.ndarray:
    """The E4M3 byte nearest to each value of y, ties to the byte with an even mantissa (the
    IEEE rule), magnitudes beyond 448 saturating to 448; the sign of a zero is kept.
    Non-negative finite bytes 0 .. 126 have increasing values, so the nearest one is found by
    bisection among them."""
    y = np.asarray(y, dtype=np.float64)
    mags = e4m3_value(np.arange(127))  # 0x00 .. 0x7e
    a = np.minimum(np.abs(y), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag_code = np.where(pick_hi, hi, lo)
    return (mag_code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quant_fp8_rows(x: np.ndarray):
    """Per-row E4M3: scale = max|x| / 448, code = round_e4m3(x / scale).

    The same reading as the int8 rows with 448, the largest E4M3 value, in place
    of 127: scale and quotient rounded once to float32, the quotient clamped to
    [-448, 448] and rounded to the nearest E4M3 value (ties to the even
    mantissa).  An all-zero row gets scale 0 (its
    codes are zeros).
    Returns (codes uint8 [..., d], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    scale = _row_scale(x, E4M3_MAX)
    y = np.clip(_quotients32(x, scale), np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return round_e4m3(y.astype(np.float64)), scale


def dequant_fp8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return e4m3_value(codes) * scale.astype(np.float64)[..., None]


# --------------------------------------------------------------------------
# Ring-buffer state   ([GOSS] "Windowed layers — ring buffer", "5.2 append", "5.3 get")
# --------------------------------------------------------------------------


@dataclass
class RingSeq:
    """One sequence of a sink + ring cache: S sink slots then a W-slot ring.

    Slot p holds the sink token at position p < S; non-sink tokens go to ring
    index `head` (slot S + head).  seq_len counts tokens appended so far.
    """

    sinks: int
    window: int
    head: int = 0
    count: int = 0
    seq_len: int = 0
    slot_pos: dict = field(default_factory=dict)  # slot -> position held (for tests)

    def append(self, n_new: int) -> dict:
        """Append positions seq_len .. seq_len+n_new-1; return {position: slot} of the writes kept.

        A chunk holding k >= W non-sink tokens written into an empty ring
        keeps its last W tokens in order and sets head 0, count W (the first
        prompt write).  Otherwise each non-sink token is written at head, head
        advances mod W and count saturates at W; only the last write to a slot
        survives.
        """
        S, W = self.sinks, self.window
        start = self.seq_len
        positions = list(range(start, start + n_new))
        writes: dict[int, int] = {}
        nonsink = []
        for p in positions:
            if p < S:
                writes[p] = p
            else:
                nonsink.append(p)
        k = len(nonsink)
        if k > 0 and self.count == 0 and k >= W:
            for i, p in enumerate(nonsink[-W:]):
                writes[p] = S + i
            self.head = 0
            self.count = W
        else:
            for p in nonsink:
                writes[p] = S + self.head
                self.head = (self.head + 1) % W
                self.count = min(W, self.count + 1)
        # drop writes overwritten later in the same chunk
        last_for_slot = {}
        for p in positions:
            if p in writes:
                last_for_slot[writes[p]] = p
        kept = {p: s for s, p in last_for_slot.items()}
        for s, p in last_for_slot.items():
            self.slot_pos[s] = p
        self.seq_len = start + n_new
        return kept

    def chronological_slots(self) -> list[int]:
        """Sinks in order, then the ring from its oldest entry: (head - count) mod W onward."""
        S, W = self.sinks, self.window
        sinks = list(range(min(S, self.seq_len)))
        first = (self.head - self.count) % W
        ring = [S + (first + j) % W for j in range(self.count)]
        return sinks + ring


# --------------------------------------------------------------------------
# Paged state   ([RoPE] the SlidingWindowSpec bound, the null-block freeing loop
#               and the window edge; [VLLM] block tables of 16-token blocks)
# --------------------------------------------------------------------------


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def sliding_window_max_blocks(window: int, block_size: int, extra: int = 0, in_flight: int = 0,
                              max_model_len: int | None = None) -> int:
    """Block bound of a windowed layer: cdiv(W - 1 + extra + in_flight, bs) + 1."""
    num_tokens = window - 1 + extra + in_flight
    if max_model_len is not None:
        num_tokens = min(num_tokens, max_model_len)
    return cdiv(num_tokens, block_size) + 1


def paged_slot(block_table_row, p: int, block_size: int) -> tuple[int, int]:
    """(physical block, offset) of logical position p: table[p // bs], p % bs."""
    return int(block_table_row[p // block_size]), p % block_size


def paged_free_expired(block_table_row: list[int], n_before: int, sinks: int, window: int,
                       block_size: int) -> list[int]:
    """Null the blocks that no present or future query can see; return freed ids.

    The edge is e = max(0, n_before - W + 1) with n_before the tokens cached
    before the call, so the call's first query (at position n_before) keeps
    its whole window.  Blocks wholly below e that hold no sink are replaced by
    -1, scanning backwards and stopping at the first null already present;
    freed ids come out in that (descending) order.  W == 0 frees nothing.
    """
    if window == 0:
        return []
    edge = max(0, n_before - window + 1)
    last_block = min(edge // block_size, len(block_table_row))
    first_block = cdiv(sinks, block_size)
    freed = []
    for j in range(last_block - 1, first_block - 1, -1):
        if block_table_row[j] == -1:
            break
        freed.append(block_table_row[j])
        block_table_row[j] = -1
    return freed


# --------------------------------------------------------------------------
# Attention   ([SINK] the runnable experiment; [GOSS] 4.4 GQA and 5.5 mask alignment)
# --------------------------------------------------------------------------


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, sink_logit: float | None = None) -> np.ndarray:
    """softmax(q . K^T * scale) V for one query vector over the rows of K, V (float64).

    With a learned sink ([RoPE] the learned-sink excerpt: a trained per-head
    logit in the softmax denominator that costs no cache; [GOSS] the sink
    bias), the normaliser gains exp(sink_logit) and no value is added:
    out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink}).  The logit is in the
    units of the scaled scores.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = (K @ q) * scale
    m = np.max(s)
    if sink_logit is not None:
        m = max(m, float(sink_logit))
    w = np.exp(s - m)
    den = np.sum(w)
    if sink_logit is not None:
        den += math.exp(float(sink_logit) - m)
    return (w @ V) / den


def decode_attention(q: np.ndarray, k_by_pos, v_by_pos, n: int, sinks: int, window: int,
                     n_kv_heads: int, scale: float | None = None, sink_logits=None) -> np.ndarray:
    """Decode output for one sequence: q [Hq, d] at position n-1 over the visible keys.

    k_by_pos(j) / v_by_pos(j) return the [Hkv, d] key / value rows at logical
    position j.  Query head h reads KV head h // (Hq / Hkv) (repeat-free GQA).
    sink_logits: optional [Hq] learned sink logits (see attend).
    """
    Hq, d = q.shape
    n_rep = Hq // n_kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    vis = visible_positions(n - 1, sinks, window)
    K = np.stack([np.asarray(k_by_pos(j), dtype=np.float64) for j in vis])  # [nv, Hkv, d]
    V = np.stack([np.asarray(v_by_pos(j), dtype=np.float64) for j in vis])
    out = np.empty((Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = h // n_rep
        sl = None if sink_logits is None else float(sink_logits[h])
        out[h] = attend(q[h], K[:, g, :], V[:, g, :], scale, sl)
    return out


def prefill_attention(q: np.ndarray, k_by_pos, v_by_pos, pos0: int, sinks: int, window: int,
                      n_kv_heads: int, scale: float | None = None, sink_logits=None) -> np.ndarray:
    """Chunk of T queries at positions pos0 .. pos0+T-1; q [T, Hq, d].

    Query t sits at absolute position pos0 + t (the idx_q = arange(T_q) + (T_k - T_q)
    alignment of [GOSS] 5.5) and sees visible_positions(pos0 + t).
    """
    T, Hq, d = q.shape
    out = np.empty((T, Hq, d), dtype=np.float64)
    for t in range(T):
        out[t] = decode_attention(q[t], k_by_pos, v_by_pos, pos0 + t + 1, sinks, window, n_kv_heads, scale,
                                  sink_logits)
    return out


def dense_sink_attention(q, k, v, capacity: int, sinks: int):
    """Dense masked form over a whole sequence: q, k, v [t, d] (the [SINK] experiment's dense path).

    The mask comes from the capacity form: query p sees all of 0..p while
    p < C, else the S sinks and the last C - S positions.
    """
    t, d = q.shape
    scores = (q @ k.T) / math.sqrt(d)
    mask = np.zeros((t, t), dtype=bool)
    for p in range(t):
        if p < capacity:
            mask[p, : p + 1] = True
        else:
            recent = capacity - sinks
            mask[p, :sinks] = True
            mask[p, max(sinks, p - recent + 1): p + 1] = True
    scores = np.where(mask, scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v, mask


def full_causal_attention(q, k, v):
    t, d = q.shape
    scores = (q @ k.T) / math.sqrt(d)
    mask = np.tril(np.ones((t, t), dtype=bool))
    scores = np.where(mask, scores, -np.inf)
    scores = scores - scores.max(axis=1, keepdims=True)
    w = np.exp(scores)
    return (w / w.sum(axis=1, keepdims=True)) @ v


# --------------------------------------------------------------------------
# Re-rotation of cached keys   ([DYN] "What it does": the cached keys follow a
# change; [SINK] R_a R_b = R_{a+b})
# --------------------------------------------------------------------------


def rerotate_rows(k_rot: np.ndarray, positions: np.ndarray, cfg_from: RopeCfg, cfg_to: RopeCfg) -> np.ndarray:
    """Turn keys rotated under cfg_from into keys rotated under cfg_to.

    Each pair i of the row at position p rotates by p (w_to,i - w_from,i) and
    is scaled by mscale_to / mscale_from; dims r..d-1 are untouched.
    k_rot has shape [N, d] (or [N, ..., d]), positions [N].
    """
    w_a = inv_freq(cfg_from)
    w_b = inv_freq(cfg_to)
    p = np.asarray(positions, dtype=np.float64)
    ang = np.outer(p, w_b - w_a)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    extra = k_rot.ndim - 2
    ang = ang.reshape(ang.shape[0], *([1] * extra), ang.shape[1])
    gain = mscale(cfg_to) / mscale(cfg_from)
    return rotate_by_angle(k_rot, ang, cfg_to.rotary_dim, cfg_to.neox, gain)


def shift_keys(k_rot: np.ndarray, delta: int, cfg: RopeCfg) -> np.ndarray:
    """Move rotated keys by `delta` positions: every pair turns by delta * w_i, gain 1.

    The local-position implementation of [SINK] ("RoPE: absolute positions and
    local rerotation"): when attention re-maps the window to positions
    [0, C-1], each recent key moves from p to p + delta (delta = -1 per slide)
    without recovering the raw key, because R_a R_b = R_{a+b}; sink keys keep
    their local positions (the caller shifts only the recent rows).
    """
    k_rot = np.asarray(k_rot, dtype=np.float64)
    ang = float(delta) * inv_freq(cfg)
    ang = np.broadcast_to(ang, k_rot.shape[:-1] + ang.shape)
    return rotate_by_angle(k_rot, ang, cfg.rotary_dim, cfg.neox, 1.0)


def rerotate_int8_rows(codes: np.ndarray, scale: np.ndarray, positions: np.ndarray,
                       cfg_from: RopeCfg, cfg_to: RopeCfg):
    """int8 rows: dequantise, turn as rerotate_rows, requantise the whole row."""
    x = dequant_int8_rows(codes, scale)
    y = rerotate_rows(x, positions, cfg_from, cfg_to)
    return quant_int8_rows(y)


def rerotate_int8_keep_scale_rows(codes: np.ndarray, scale: np.ndarray, positions: np.ndarray,
                                  cfg_from: RopeCfg, cfg_to: RopeCfg):
    """int8 rows, keeping each row's scale unless a turned code overflows.

    [DYN] "Measured on this branch" notes that, without the Hadamard, a turn
    leaves the dims past the rotary slice (codes and scales) bitwise as they
    were written.  With one scale per row that holds only if the scale stays:
    dequantise, turn the rotary pairs, and re-code the rotary dims with the old
    scale (code = rne(y / scale), the quotient rounded to float32 as in
    quant_int8_rows); the tail codes and the scale are kept.  If any re-coded
    value leaves [-127, 127] (the turn can grow a pair's larger component up to
    sqrt(2) times, and the gain mscale_to / mscale_from may exceed 1), the row
    is re-quantised whole as in rerotate_int8_rows.  A zero scale (all-zero
    row) stays zero.
    Returns (codes, scale, overflow) with overflow True for the re-quantised rows.
    """
    codes = np.asarray(codes)
    scale = np.asarray(scale, dtype=np.float32)
    x = dequant_int8_rows(codes, scale)
    y = rerotate_rows(x, positions, cfg_from, cfg_to)
    r = cfg_to.rotary_dim
    cand = np.rint(_quotients32(y[..., :r], scale))
    overflow = np.any(np.abs(cand) > 127, axis=-1)
    out_codes = codes.astype(np.int8).copy()
    out_scale = scale.copy()
    keep = ~overflow
    out_codes[keep, :r] = cand[keep].astype(np.int8)
    full_codes, full_scale = quant_int8_rows(y)
    out_codes[overflow] = full_codes[overflow]
    out_scale[overflow] = full_scale[overflow]
    return out_codes, out_scale, overflow


# --------------------------------------------------------------------------
# Hadamard-rotated int8 keys   ([DYN] "What it does": K with the Hadamard)
# --------------------------------------------------------------------------


def hadamard(x: np.ndarray) -> np.ndarray:
    """Orthonormal Walsh-Hadamard transform over the last axis (length n = 2^k).

    H_n = H_2 (x) ... (x) H_2 / sqrt(n) with H_2 = [[1, 1], [1, -1]]
    (Sylvester order: H[i, j] = (-1)^popcount(i & j) / sqrt(n)).  H is
    symmetric and orthogonal, so it is its own inverse.  Written as the k
    butterfly passes over pairs (j, j + h), h = 1, 2, 4, ...
    """
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    if n < 1 or n & (n - 1):
        raise ValueError("length must be a power of two")
    h = 1
    while h < n:
        for start in range(0, n, 2 * h):
            a = y[..., start:start + h].copy()
            b = y[..., start + h:start + 2 * h].copy()
            y[..., start:start + h] = a + b
            y[..., start + h:start + 2 * h] = a - b
        h *= 2
    return y / math.sqrt(n)


def quant_int8_hadamard_rows(k_rot: np.ndarray):
    """Store a rotated key as int8 codes of H k (per-row scale over the transformed row)."""
    return quant_int8_rows(hadamard(k_rot))


def rerotate_int8_hadamard_rows(codes: np.ndarray, scale: np.ndarray, positions: np.ndarray,
                                cfg_from: RopeCfg, cfg_to: RopeCfg):
    """Hadamard-rotated int8 rows: dequantise, H (back to the rotated key), turn the
    rotary pairs as rerotate_rows, H, requantise the row ([DYN] "What it does")."""
    k = hadamard(dequant_int8_rows(codes, scale))
    y = rerotate_rows(k, positions, cfg_from, cfg_to)
    return quant_int8_rows(hadamard(y))


# --------------------------------------------------------------------------
# The dynamic factor policy   ([DYN] "What it does": the factor)
# --------------------------------------------------------------------------


def dynamic_factor(length: int, trained: int, step: float = 0.125, cap: float = 2.0) -> float:
    """None (1.0) inside the trained range; above it length / trained rounded up to `step`, capped."""
    if length <= trained:
        return 1.0
    f = math.ceil((length / trained) / step) * step
    return min(f, cap)
