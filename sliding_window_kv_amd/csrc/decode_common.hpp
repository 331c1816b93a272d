// Shared pieces of the split-K decode kernels (16-bit / fp32 and int8 caches):
// the tile walk over a sequence's visible cache rows, fragment loads, and the
// launch that merges the split partials.
#pragma once

#include "kernels.hpp"

namespace ropekv {
namespace decode_detail {
namespace {  // each decode source gets its own copies of these kernels and helpers

constexpr int kTile = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// Tiles of one sequence and how a tile maps to cache rows.
struct SeqTiles {
  int n;       // tokens in the sequence (query at n - 1)
  int ntiles;  // tiles to visit
  int ns, rs;  // PAGED: positions < ns (sinks) and [rs, n) are visible
  int nsb, fr; // PAGED: sink tiles are blocks 0..nsb-1; then blocks fr, fr+1, ...
  int oldest, count;  // RING: valid ring indices are oldest .. oldest+count-1 (mod W)
};

__device__ __forceinline__ int imod(int x, int m) {
  int r = x % m;
  return r < 0 ? r + m : r;
}

__device__ inline SeqTiles seq_tiles(const ropekv_kv_cache &c, int b) {
  SeqTiles st;
  st.n = c.seq_len[b];
  st.ntiles = 0;
  st.ns = st.rs = st.nsb = st.fr = st.oldest = st.count = 0;
  const int n = st.n;
  if (n <= 0) return st;
  if (c.layout == ROPEKV_PAGED) {
    if (c.window == 0) {
      st.ns = n;
      st.rs = n;
      st.nsb = (n + kTile - 1) / kTile;
      st.fr = st.nsb;
      st.ntiles = st.nsb;
    } else {
      const int ns = min(c.sinks, n);
      const int rs = max(ns, n - c.window);
      const int nsb = (ns + kTile - 1) / kTile;
      const int fr = max(rs / kTile, nsb);
      const int lastb = (n - 1) / kTile;
      st.ns = ns;
      st.rs = rs;
      st.nsb = nsb;
      st.fr = fr;
      st.ntiles = nsb + max(0, lastb - fr + 1);
    }
  } else {  // RING
    const int S = c.sinks, W = c.window, C = c.capacity;
    const int cnt = min(max(c.ring_count[b], 0), W);
    const int hb = imod(c.ring_head[b], W);
    const int oldest = imod(hb - cnt, W);
    const int limit = (cnt < W && oldest + cnt <= W) ? S + oldest + cnt : C;
    st.ns = min(S, n);
    st.oldest = oldest;
    st.count = cnt;
    st.ntiles = (limit + kTile - 1) / kTile;
  }
  return st;
}

template <int NB>
__device__ __forceinline__ void load_bytes(uint32_t *dst, const void *src) {
  static_assert(NB % 8 == 0, "fragment size");
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)src + i);
      dst[4 * i + 0] = v.x;
      dst[4 * i + 1] = v.y;
      dst[4 * i + 2] = v.z;
      dst[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const uint2 v = ((const uint2 *)src)[i];
      dst[2 * i + 0] = v.x;
      dst[2 * i + 1] = v.y;
    }
  }
}

// A lane's share of one K (or Q) row for the 16x16 MFMAs: QB bytes as 16-byte
// pieces, piece i taken from byte offset (4 i + grp) * 16 of the row.  The four
// lane groups of a row thus read 64 contiguous bytes per load instruction.
// Any fixed assignment of row chunks to (piece, group) is valid because the
// d-reduction is order-free, as long as K and Q use the same one.
// K and V are streamed once per decode: nontemporal loads keep them from
// displacing reusable lines in the caches.
__device__ __forceinline__ void stream16(uint32_t *dst, const void *p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
  dst[0] = v.x;
  dst[1] = v.y;
  dst[2] = v.z;
  dst[3] = v.w;
}

template <int QB>
__device__ __forceinline__ void load_pieces(uint32_t *dst, const char *row, int grp) {
  static_assert(QB % 16 == 0, "pieces are 16 bytes");
#pragma unroll
  for (int i = 0; i < QB / 16; ++i) stream16(dst + 4 * i, row + (4 * i + grp) * 16);
}

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float get(const uint32_t *w, int i) { return __uint_as_float(w[i]); }
  static __device__ __forceinline__ void put(void *p, long i, float v) { ((float *)p)[i] = v; }
};
template <>
struct ElemTraits<bf16_t> {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float get(const uint32_t *w, int i) {
    const uint32_t x = w[i >> 1];
    return __uint_as_float((i & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  static __device__ __forceinline__ void put(void *p, long i, float v) { ((uint16_t *)p)[i] = f_to_bf16(v); }
};

constexpr int kMaxTps = 256;  // tiles per split of a split plan
constexpr int kMaxDirectTiles = 512;  // tiles of a direct-plan workgroup (block-table entries staged in LDS)
constexpr int kDirectWaves = 8;       // waves of a direct-plan workgroup, 16-bit caches (2 per SIMD; windowed batch-256 and ring layer: 4: +1 % / +7 %, 6: -3 %, 8: -3 %, 16: +40 % against 12)
constexpr int kDirectWavesF32 = 8;    // fp32 caches run at 2 waves per SIMD

// Merge the split partials of one (sequence, KV head) for its n_rep query heads:
// one wave per query head finds the global maximum and the split weights
// exp2(m_s - m) (into LDS) and the total weight l, then all threads make one
// coalesced pass over the partial rows.
constexpr int kMaxSplits = 1024;

template <typename T, int D, int NREP>
__global__ __launch_bounds__(256) void decode_combine_kernel(ropekv_kv_cache c, const float *__restrict__ ws,
                                                             const float *__restrict__ sinks, void *__restrict__ out,
                                                             int tps, int splits) {
  __shared__ float s_w[NREP][kMaxSplits];
  __shared__ float s_inv[NREP];
  const int g = blockIdx.x, b = blockIdx.y;
  const int Hkv = c.num_kv_heads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const SeqTiles st = seq_tiles(c, b);
  const int used = min(min((st.ntiles + tps - 1) / tps, splits), kMaxSplits);
  const float *src = ws + ((long)(b * Hkv + g) * splits) * NREP * (D + 2);  // [split][n_rep][D + 2]
  const long sstride = (long)NREP * (D + 2);
  for (int hh = wave; hh < NREP; hh += 4) {
    const float *sh = src + hh * (D + 2);
    float m = kNegBig;
    for (int s = lane; s < used; s += 64) m = fmaxf(m, sh[s * sstride + D]);
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    // a learned sink logit joins the normaliser (log2 units like the partial maxima)
    const float sink2 = sinks ? sinks[g * NREP + hh] * kLog2e : -INFINITY;
    if (used > 0) m = fmaxf(m, sink2);
    float l = 0.f;
    for (int s = lane; s < used; s += 64) {
      const float w = exp2f(sh[s * sstride + D] - m);
      s_w[hh][s] = w;
      l += w * sh[s * sstride + D + 1];
    }
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    if (sinks && used > 0) l += exp2f(sink2 - m);
    if (lane == 0) s_inv[hh] = l > 0.f ? 1.f / l : 0.f;
  }
  __syncthreads();
  const long obase = ((long)b * Hkv + g) * NREP * D;
  for (int idx = threadIdx.x; idx < NREP * D; idx += 256) {
    const int hh = idx / D, dd = idx - hh * D;
    const float *sh = src + hh * (D + 2) + dd;
    float a = 0.f;
    for (int s = 0; s < used; ++s) a = fmaf(s_w[hh][s], sh[s * sstride], a);
    ElemTraits<T>::put(out, obase + idx, a * s_inv[hh]);
  }
}

}  // namespace
}  // namespace decode_detail
}  // namespace ropekv
