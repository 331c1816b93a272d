"""The algorithmic work bench.py divides by time (the roofline's `achieved`), pinned on the CPU to the
counts derived from the workload shapes and to the oracle's visible set (no GPU, no kernel)."""
from types import SimpleNamespace

from oracle import ropekv_oracle as O
from sliding_window_kv_amd import workloads as WL


def test_visible_count_matches_the_oracle_set():
    for S, W in ((4, 4096), (0, 12), (3, 1), (4, 0)):
        for p in list(range(0, 40)) + [4094, 4095, 4096, 4097, 4099, 4100, 5000, 8191]:
            assert WL.visible_count(p, S, W) == len(O.visible_positions(p, S, W)), (p, S, W)


def test_prefill_flops_of_the_8192_token_chunk():
    # 25,184,250 visible (query, key) pairs per head: 4096 causal rows 0..4095 (sum 1..4096 = 8,390,656),
    # then 4096 rows of 4096 window keys plus the sinks not already in the window (4 from row 4099 on,
    # 1, 2, 3 at rows 4096..4098); 4 d FLOP per pair and head
    pf = SimpleNamespace(T=8192, S=4, W=4096, d=128, Hq=64)
    pairs = sum(WL.visible_count(p, 4, 4096) for p in range(8192))
    assert pairs == 4096 * 4097 // 2 + 4096 * 4100 - (3 + 2 + 1) == 25_184_250
    assert WL.Prefill.flops(pf) == 4 * 128 * 64 * 25_184_250 == 825_237_504_000


def test_decode_bytes_of_the_timed_rows():
    # batch 64 x 32768 paged: K + V once per KV head, q and out, the block-table entries
    pd = SimpleNamespace(B=64, Hkv=8, Hq=32, d=128, ctx=32768, kv8=None, max_blocks=2048)
    assert WL.PagedDecode.decode_bytes(pd) == 2 * 64 * 8 * 32768 * 256 + 2 * 64 * 32 * 128 * 2 + 64 * 2048 * 4
    assert WL.PagedDecode.decode_bytes(pd) == 8_591_507_456
    # the same over an 8-bit cache: codes plus one fp32 scale per row
    pd.kv8 = "i8"
    assert WL.PagedDecode.decode_bytes(pd) == 2 * 64 * 8 * 32768 * 132 + 2 * 64 * 32 * 128 * 2 + 64 * 2048 * 4
    # one ring layer at position 131071: S + W = 4100 visible keys per sequence and KV head
    rd = SimpleNamespace(B=32, Hkv=8, Hq=32, d=128, S=4, W=4096, n=131072)
    assert WL.RingDecode.decode_bytes(rd) == 2 * 32 * 8 * 4100 * 256 + 2 * 32 * 32 * 128 * 2 == 537_919_488


def test_rerotate_bytes_of_the_64_layer_switch():
    rows = 64 * 524288 * 8
    f16 = SimpleNamespace(kind="f16", L=64, T=524288, Hkv=8, d=128, r=64)
    i8 = SimpleNamespace(kind="i8", L=64, T=524288, Hkv=8, d=128, r=64)
    assert WL.Rerotate.bytes(f16) == 2 * rows * 64 * 2 == 68_719_476_736
    assert WL.Rerotate.bytes(i8) == 2 * rows * (128 + 4) == 70_866_960_384
    keep = SimpleNamespace(kind="i8_keep", L=64, T=524288, Hkv=8, d=128, r=64)
    # every row and scale read; kept rows write 64 rotary codes, the others the row and its scale
    assert WL.Rerotate.bytes(keep, 0.5) == rows * 132 + rows // 2 * 64 + rows // 2 * 132
