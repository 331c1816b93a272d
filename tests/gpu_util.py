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


def assert_bf16_close(gpu: np.ndarray, ref: np.ndarray, atol=2e-2, rtol=1e-2):
    err = np.abs(gpu - ref) - (atol + rtol * np.abs(ref))
    assert float(np.max(err)) <= 0.0, f"max excess {float(np.max(err)):.3e}, max abs err {float(np.max(np.abs(gpu-ref))):.3e}"


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
