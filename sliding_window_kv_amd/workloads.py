"""Device-resident synthetic workloads at full size (shared by bench.py and the full-size tests).

Each class allocates its buffers with torch, fills them from seeded
generators, and exposes the calls the hot path makes.  Nothing here computes
any part of the method: positions, slots, visibility and attention all run in
libropekv.so.  Byte and FLOP counts are the algorithmic work of each call
(what the method must move or compute, not what a dense kernel would).
"""
from __future__ import annotations

import numpy as np

from . import synth

BLOCK = 16


def visible_count(p: int, sinks: int, window: int) -> int:
    """Number of keys the query at position p sees (window 0 = causal)."""
    if window == 0 or p + 1 <= window:
        return p + 1
    return window + min(sinks, p + 1 - window)


class PagedDecode:
    """Full-attention paged decode of one layer (Llama-3-8B-shaped by default).

    B sequences of ctx tokens after the step's append, Hq / Hkv heads, d dims,
    bf16, 16-token blocks, block table = a seeded random permutation of the
    pool.  kv8 "i8" or "fp8" holds the cache as 8-bit codes (int8 or E4M3)
    with one fp32 scale per row instead of bf16.  A step appends each sequence's new token at position ctx - 1
    (rotating q and k, writing k and v into the pool) and runs decode.
    """

    def __init__(self, R, torch, dev, B=64, Hq=32, Hkv=8, d=128, ctx=32768, theta=5e5, seed=2000, kv8=None):
        self.R, self.torch, self.dev = R, torch, dev
        self.B, self.Hq, self.Hkv, self.d, self.ctx = B, Hq, Hkv, d, ctx
        if kv8 not in (None, "i8", "fp8"):
            raise ValueError(f"kv8 must be None, 'i8' or 'fp8', not {kv8!r}")
        self.kv8 = kv8
        self.max_blocks = (ctx + BLOCK - 1) // BLOCK
        self.num_blocks = B * self.max_blocks
        table = synth.block_table_permutation(B, self.max_blocks, self.num_blocks, seed)
        self.table_host = table
        bf = torch.bfloat16
        pool = (self.num_blocks, Hkv, BLOCK, d)
        if kv8:
            # 8-bit codes (int8 uniform in [-127, 127]; E4M3 uniform over its finite bytes) with
            # per-row scales that put the largest code near 2 .. 3.5: rows of magnitude ~ N(0, 1) data
            fill = synth.device_int8_codes_ if kv8 == "i8" else synth.device_fp8_codes_
            store = torch.int8 if kv8 == "i8" else torch.uint8
            qmax = 127.0 if kv8 == "i8" else 448.0
            self.k = fill(torch.empty(pool, dtype=store, device=dev), seed + 1)
            self.v = fill(torch.empty(pool, dtype=store, device=dev), seed + 2)
            self.k_scale = synth.device_uniform_(torch.empty(pool[:3], dtype=torch.float32, device=dev),
                                                 2.0 / qmax, 3.5 / qmax, seed + 6)
            self.v_scale = synth.device_uniform_(torch.empty(pool[:3], dtype=torch.float32, device=dev),
                                                 2.0 / qmax, 3.5 / qmax, seed + 7)
        else:
            self.k = synth.device_normal_(torch.empty(pool, dtype=bf, device=dev), seed + 1)
            self.v = synth.device_normal_(torch.empty(pool, dtype=bf, device=dev), seed + 2)
            self.k_scale = self.v_scale = None
        self.table = torch.from_numpy(table).to(dev)
        self.seq_len = torch.full((B,), ctx - 1, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.desc = R.kv_cache(R.PAGED, {None: R.BF16, "i8": R.I8, "fp8": R.FP8}[kv8], Hkv, d, self.k, self.v, batch=B, sinks=0,
                               window=0, block_size=BLOCK, max_blocks=self.max_blocks, num_blocks=self.num_blocks,
                               block_table=self.table, seq_len=self.seq_len, err_word=self.err,
                               k_scale=self.k_scale, v_scale=self.v_scale)
        self.cfg = R.rope_cfg(d, d, rope_theta=theta)
        self.rope_table = torch.empty(ctx, d, dtype=torch.float32, device=dev)
        R.build_table(self.cfg, ctx, self.rope_table)
        self.q = synth.device_normal_(torch.empty(B, Hq, d, dtype=bf, device=dev), seed + 3)
        self.k_new = synth.device_normal_(torch.empty(B, Hkv, d, dtype=bf, device=dev), seed + 4)
        self.v_new = synth.device_normal_(torch.empty(B, Hkv, d, dtype=bf, device=dev), seed + 5)
        self.pos = torch.full((B,), ctx - 1, dtype=torch.int32, device=dev)
        self.seq_ids = torch.arange(B, dtype=torch.int32, device=dev)
        self.out = torch.empty(B, Hq, d, dtype=bf, device=dev)
        self.ws_bytes = R.decode_workspace_size(B, Hq, self.desc)
        self.ws = torch.empty(self.ws_bytes // 4 + 1, dtype=torch.float32, device=dev)

    def step(self):
        """One decode step: reset to ctx-1 cached tokens, rope + append the new token, decode."""
        self.seq_len.fill_(self.ctx - 1)
        self.append()
        self.decode()

    def append(self):
        R = self.R
        R.apply_append(self.cfg, self.rope_table, self.ctx, self.q, self.Hq, self.k_new, self.v_new, R.BF16, self.B,
                       self.pos, self.seq_ids, self.desc)

    def decode(self):
        self.R.decode_attn(self.q, self.B, self.Hq, self.desc, 0.0, self.out, self.ws, self.ws_bytes)

    def decode_bytes(self) -> int:
        """K + V of the visible keys once per KV head (8-bit: codes + one fp32 scale per row),
        plus q, out and the block-table entries read."""
        row = self.d + 4 if self.kv8 else 2 * self.d
        kv = 2 * self.B * self.Hkv * self.ctx * row
        qo = 2 * self.B * self.Hq * self.d * 2
        bt = self.B * self.max_blocks * 4
        return kv + qo + bt

    def kv_of(self, b: int):
        """Keys / values of sequence b by position, as host float64 [ctx, Hkv, d] (for the oracle)."""
        if self.kv8:
            raise ValueError("8-bit cache: use codes_of")
        rows = self.table[b]
        k = self.k[rows].permute(0, 2, 1, 3).reshape(-1, self.Hkv, self.d)[: self.ctx]
        v = self.v[rows].permute(0, 2, 1, 3).reshape(-1, self.Hkv, self.d)[: self.ctx]
        return (k.float().cpu().numpy().astype(np.float64), v.float().cpu().numpy().astype(np.float64))

    def codes_of(self, b: int):
        """8-bit cache: (k codes, k scales, v codes, v scales) of sequence b by position, host arrays
        [ctx, Hkv, d] int8 / uint8 and [ctx, Hkv] float32."""
        rows = self.table[b]

        def by_pos(t, tail):
            return t[rows].permute(0, 2, 1, *tail).reshape(-1, self.Hkv, *([self.d] if tail else []))[: self.ctx]

        return (by_pos(self.k, (3,)).cpu().numpy(), by_pos(self.k_scale, ()).cpu().numpy(),
                by_pos(self.v, (3,)).cpu().numpy(), by_pos(self.v_scale, ()).cpu().numpy())


class RingDecode:
    """Windowed decode of one ring layer: full ring (count = W), head at a seeded random offset."""

    def __init__(self, R, torch, dev, B=32, Hq=32, Hkv=8, d=128, S=4, W=4096, n=131072, seed=3000):
        self.R, self.torch = R, torch
        self.B, self.Hq, self.Hkv, self.d, self.S, self.W, self.n = B, Hq, Hkv, d, S, W, n
        self.C = S + W
        bf = torch.bfloat16
        self.k = synth.device_normal_(torch.empty(B, Hkv, self.C, d, dtype=bf, device=dev), seed + 1)
        self.v = synth.device_normal_(torch.empty(B, Hkv, self.C, d, dtype=bf, device=dev), seed + 2)
        self.head = torch.from_numpy(synth.uniform_ints(B, 0, W, seed + 3)).to(dev)
        self.count = torch.full((B,), W, dtype=torch.int32, device=dev)
        self.seq_len = torch.full((B,), n, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.desc = R.kv_cache(R.RING, R.BF16, Hkv, d, self.k, self.v, batch=B, capacity=self.C, sinks=S, window=W,
                               ring_head=self.head, ring_count=self.count, seq_len=self.seq_len, err_word=self.err)
        self.q = synth.device_normal_(torch.empty(B, Hq, d, dtype=bf, device=dev), seed + 4)
        self.out = torch.empty_like(self.q)
        self.ws_bytes = R.decode_workspace_size(B, Hq, self.desc)
        self.ws = torch.empty(self.ws_bytes // 4 + 1, dtype=torch.float32, device=dev)

    def decode(self):
        self.R.decode_attn(self.q, self.B, self.Hq, self.desc, 0.0, self.out, self.ws, self.ws_bytes)

    def decode_bytes(self) -> int:
        vis = min(self.n, self.S + self.W)
        return 2 * self.B * self.Hkv * vis * self.d * 2 + 2 * self.B * self.Hq * self.d * 2


class WindowedPagedDecode:
    """Sink + window paged decode with ragged lengths; only live blocks are allocated, the rest are null."""

    def __init__(self, R, torch, dev, B=256, Hq=64, Hkv=8, d=128, S=4, W=4096, lo=1024, hi=131072, seed=5000):
        self.R, self.torch = R, torch
        self.B, self.Hq, self.Hkv, self.d, self.S, self.W = B, Hq, Hkv, d, S, W
        self.lens = synth.uniform_lengths(B, lo, hi, seed)
        self.max_blocks = (int(self.lens.max()) + BLOCK - 1) // BLOCK
        table = np.full((B, self.max_blocks), -1, dtype=np.int64)
        nxt = 0
        for b, n in enumerate(self.lens):
            live = set(range((min(S, n) + BLOCK - 1) // BLOCK))
            first = max(0, n - W) // BLOCK
            live |= set(range(first, (n - 1) // BLOCK + 1))
            for j in sorted(live):
                table[b, j] = nxt
                nxt += 1
        self.num_blocks = nxt
        perm = synth.rng(seed + 9).permutation(nxt)  # scatter the live blocks over the pool
        table = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
        self.table_host = table
        bf = torch.bfloat16
        self.k = synth.device_normal_(torch.empty(nxt, Hkv, BLOCK, d, dtype=bf, device=dev), seed + 1)
        self.v = synth.device_normal_(torch.empty(nxt, Hkv, BLOCK, d, dtype=bf, device=dev), seed + 2)
        self.table = torch.from_numpy(table).to(dev)
        self.seq_len = torch.from_numpy(self.lens.astype(np.int32)).to(dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.desc = R.kv_cache(R.PAGED, R.BF16, Hkv, d, self.k, self.v, batch=B, sinks=S, window=W, block_size=BLOCK,
                               max_blocks=self.max_blocks, num_blocks=nxt, block_table=self.table,
                               seq_len=self.seq_len, err_word=self.err)
        self.q = synth.device_normal_(torch.empty(B, Hq, d, dtype=bf, device=dev), seed + 4)
        self.out = torch.empty_like(self.q)
        self.ws_bytes = R.decode_workspace_size(B, Hq, self.desc)
        self.ws = torch.empty(self.ws_bytes // 4 + 1, dtype=torch.float32, device=dev)

    def decode(self, stream=None):
        self.R.decode_attn(self.q, self.B, self.Hq, self.desc, 0.0, self.out, self.ws, self.ws_bytes, stream=stream)

    def decode_bytes(self) -> int:
        vis = sum(visible_count(int(n) - 1, self.S, self.W) for n in self.lens)
        blocks = int((self.table_host >= 0).sum())
        return 2 * vis * self.Hkv * self.d * 2 + 2 * self.B * self.Hq * self.d * 2 + blocks * 4


class Prefill:
    """One prompt chunk of T tokens at pos0 = 0 over the sink + window mask, bf16."""

    def __init__(self, R, torch, dev, T=8192, Hq=64, Hkv=8, d=128, S=4, W=4096, seed=6000):
        self.R, self.torch = R, torch
        self.T, self.Hq, self.Hkv, self.d, self.S, self.W = T, Hq, Hkv, d, S, W
        bf = torch.bfloat16
        self.q = synth.device_normal_(torch.empty(T, Hq, d, dtype=bf, device=dev), seed + 1)
        self.k = synth.device_normal_(torch.empty(T, Hkv, d, dtype=bf, device=dev), seed + 2)
        self.v = synth.device_normal_(torch.empty(T, Hkv, d, dtype=bf, device=dev), seed + 3)
        self.out = torch.empty_like(self.q)
        # the chunk starts at position 0; its rope + append writes the survivors into a ring layer
        self.kc = torch.zeros(1, Hkv, S + W, d, dtype=bf, device=dev)
        self.vc = torch.zeros(1, Hkv, S + W, d, dtype=bf, device=dev)
        self.int_state = torch.zeros(4, dtype=torch.int32, device=dev)
        st = self.int_state
        self.desc = R.kv_cache(R.RING, R.BF16, Hkv, d, self.kc, self.vc, batch=1, capacity=S + W, sinks=S, window=W,
                               ring_head=st[0:1], ring_count=st[1:2], seq_len=st[2:3], err_word=st[3:4])
        self.cfg = R.rope_cfg(d, d, rope_theta=5e5)
        self.rope_table = torch.empty(T, d, dtype=torch.float32, device=dev)
        R.build_table(self.cfg, T, self.rope_table)
        self.pos = torch.arange(T, dtype=torch.int32, device=dev)
        self.seq_ids = torch.zeros(T, dtype=torch.int32, device=dev)

    def run(self, stream=None):
        self.R.prefill_attn(self.q, self.k, self.v, self.T, 0, self.Hq, self.desc, 0, 0.0, self.out, stream=stream)

    def append(self):
        """Rope + append of the whole chunk into an empty ring (state reset first)."""
        self.int_state[0:3].zero_()
        self.R.apply_append(self.cfg, self.rope_table, self.T, self.q, self.Hq, self.k, self.v, self.R.BF16, self.T,
                            self.pos, self.seq_ids, self.desc)

    def append_bytes(self) -> int:
        """q and k read and written in place, v read, and the C surviving rows of k and v written."""
        qb = self.T * self.Hq * self.d * 2
        kb = self.T * self.Hkv * self.d * 2
        written = min(self.T, self.S + self.W) * self.Hkv * self.d * 2
        return 2 * qb + 2 * kb + kb + 2 * written

    def flops(self) -> int:
        vis = sum(visible_count(p, self.S, self.W) for p in range(self.T))
        return 4 * self.d * self.Hq * vis


class Rerotate:
    """Cached keys of L layers x T positions x Hkv heads, fp16 or int8 + per-row fp32 scale, turned in place.

    kind "f16" and "i8": seeded N(0, 1) fp16 keys / uniform int8 codes with U(0.01, 0.03) scales.
    "i8_keep" (keep the row scale unless a code overflows) and "i8_hadamard" (rows hold codes of H k):
    seeded N(0, 1) raw keys written at factor 1 by apply_append, so rows look like quantised keys.
    """

    def __init__(self, R, torch, dev, kind="f16", L=64, T=524288, Hkv=8, d=128, r=64, theta=5e5, L0=262144, pos0=0,
                 seed=4000):
        self.R, self.torch = R, torch
        self.kind, self.L, self.T, self.Hkv, self.d, self.r = kind, L, T, Hkv, d, r
        self.theta, self.L0 = theta, L0
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        mode = {"i8_keep": R.I8_KEEP_SCALE, "i8_hadamard": R.I8_HADAMARD}.get(kind, 0)
        if kind == "f16":
            self.k = synth.device_normal_(torch.empty(L, T, Hkv, d, dtype=torch.float16, device=dev), seed)
            self.scale = None
            dt = R.F16
        elif kind == "i8":
            g = torch.Generator(device=dev)
            g.manual_seed(seed)
            self.k = torch.randint(-127, 128, (L, T, Hkv, d), dtype=torch.int8, device=dev, generator=g)
            self.scale = torch.rand(L, T, Hkv, dtype=torch.float32, device=dev, generator=g) * 0.02 + 0.01
            dt = R.I8
        else:
            self.k = torch.empty(L, T, Hkv, d, dtype=torch.int8, device=dev)
            self.scale = torch.empty(L, T, Hkv, dtype=torch.float32, device=dev)
            dt = R.I8
            cfg = self.cfg(1.0)
            table = torch.empty(pos0 + T, r, dtype=torch.float32, device=dev)
            R.build_table(cfg, pos0 + T, table)
            pos = torch.arange(pos0, pos0 + T, dtype=torch.int32, device=dev)
            raw = torch.empty(T, Hkv, d, dtype=torch.float16, device=dev)
            for layer in range(L):
                synth.device_normal_(raw, seed + layer)
                dl = R.kv_cache(R.CONTIG, dt, Hkv, d, self.k[layer], capacity=T, pos0=pos0,
                                k_scale=self.scale[layer], err_word=self.err, k_int8_mode=mode)
                R.apply_append(cfg, table, pos0 + T, None, 0, raw, None, R.F16, T, pos, None, dl)
            del raw, table
        self.desc = R.kv_cache(R.CONTIG, dt, Hkv, d, self.k, capacity=T, pos0=pos0, k_scale=self.scale,
                               err_word=self.err, k_int8_mode=mode)

    def cfg(self, s: float):
        return self.R.rope_cfg(self.d, self.r, rope_theta=self.theta, yarn_factor=s, orig_max_pos=self.L0)

    def run(self, s_from: float, s_to: float):
        self.R.rerotate(self.cfg(s_from), self.cfg(s_to), self.desc, self.L)

    def bytes(self, kept_fraction=None) -> int:
        """fp16: the rotary slice read and written.  int8: the row and its scale read and written.
        Keep-scale: every row and scale read; a row that keeps its scale writes its rotary codes,
        one that overflows writes the whole row and its scale (kept_fraction: the measured share of
        rows that kept their scale; None counts every row as kept)."""
        rows = self.L * self.T * self.Hkv
        if self.kind == "f16":
            return 2 * rows * self.r * 2
        if self.kind == "i8_keep":
            kept = rows if kept_fraction is None else int(round(rows * kept_fraction))
            return rows * (self.d + 4) + kept * self.r + (rows - kept) * (self.d + 4)
        return 2 * rows * (self.d + 4)
