// Split-K decode attention over the sink + recent visible set.
//
// "Attention Sink 与 Streaming KV Cache" (visible set; the incremental cache
// of the runnable experiment) and "Inference & 128K Long Context" (4.3 decode
// is memory bound, 4.4 GQA): one query per sequence and query head attends
// to the keys visible at position n - 1, reading the cache in place.  The
// n_rep query heads of a KV head share every K/V byte loaded (repeat-free
// GQA, h -> h / n_rep).
//
// Work unit: a "tile" = 16 consecutive cache rows (one 16-token paged block,
// or 16 ring slots) of one KV head.  A workgroup (4 waves) owns a contiguous
// run of tiles of one (sequence, KV head); each wave takes every 4th tile and
// keeps its own online-softmax state; the waves are merged in LDS and one
// fp32 partial (acc, m, l) per split goes to the workspace.  A second launch
// merges the splits.
//
// Per tile and wave:  S^T[16 keys x 16 cols] = K . Q^T on MFMA (the n_rep
// query heads fill the first columns, the rest are zero), scores scaled into
// the log2 domain, masked, online softmax per query head; P and the
// correction factors go through a small per-wave LDS slot to the layout in
// which each lane holds 4 keys x (d/16) dims of V, and O += P V in fp32.
#include <stdlib.h>

#include "kernels.hpp"

namespace ropekv {

namespace {

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

// Row r (< 16) of tile `tile` for (b, g): element offset of the row in k/v
// (clamped in bounds) and whether the key there is visible.
struct TileRows {
  long base;  // element offset of row 0 of the tile (PAGED) or of slot 0 of (b, g) (RING)
  int slot0;  // RING: first slot of the tile
  int pos0;   // PAGED: position of row 0
  bool ok;    // the tile maps to allocated memory
};

__device__ __forceinline__ TileRows tile_rows(const ropekv_kv_cache &c, const SeqTiles &st, int b, int g,
                                             int tile, int D) {
  TileRows tr;
  tr.ok = true;
  tr.slot0 = 0;
  tr.pos0 = 0;
  if (c.layout == ROPEKV_PAGED) {
    const int blk = tile < st.nsb ? tile : st.fr + (tile - st.nsb);
    const int bid = (blk < c.max_blocks) ? c.block_table[(long)b * c.max_blocks + blk] : -1;
    tr.pos0 = blk * kTile;
    if (bid < 0 || bid >= c.num_blocks) {
      tr.ok = false;
      tr.base = 0;
    } else {
      tr.base = ((long)bid * c.num_kv_heads + g) * kTile * D;
    }
  } else {
    tr.slot0 = tile * kTile;
    tr.base = ((long)b * c.num_kv_heads + g) * (long)c.capacity * D;
  }
  return tr;
}

__device__ __forceinline__ long row_offset(const ropekv_kv_cache &c, const TileRows &tr, int r, int D) {
  if (c.layout == ROPEKV_PAGED) return tr.base + (long)r * D;
  const int slot = min(tr.slot0 + r, c.capacity - 1);
  return tr.base + (long)slot * D;
}

__device__ __forceinline__ bool row_visible(const ropekv_kv_cache &c, const SeqTiles &st, const TileRows &tr,
                                            int r) {
  if (!tr.ok) return false;
  if (c.layout == ROPEKV_PAGED) {
    const int pos = tr.pos0 + r;
    return pos < st.ns || (pos >= st.rs && pos < st.n);
  }
  const int slot = tr.slot0 + r;
  if (slot >= c.capacity) return false;
  if (slot < c.sinks) return slot < st.ns;
  const int i = slot - c.sinks;
  return imod(i - st.oldest, c.window) < st.count;
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

// S^T (16 keys x 16 columns) += K (16 x D) . Q^T (D x 16), lane-distributed
// as: kw / qw = the lane's share (load_pieces) of K row lane%16 / of Q column
// lane%16.  The reduction over d is order-free, so lanes feed their shares
// to consecutive MFMAs in the same element order on both sides.
template <typename T, int D>
__device__ __forceinline__ f32x4 qk_tile(const uint32_t *kw, const uint32_t *qw) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      short8 a, bq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = (short)(kw[4 * t + e] & 0xffff);
        a[2 * e + 1] = (short)(kw[4 * t + e] >> 16);
        bq[2 * e] = (short)(qw[4 * t + e] & 0xffff);
        bq[2 * e + 1] = (short)(qw[4 * t + e] >> 16);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, bq),
                                                    acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int t = 0; t < D / 4; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[t]), __uint_as_float(qw[t]), acc, 0, 0, 0);
  }
  return acc;
}

// K and V pieces of one tile held by one lane, plus which of its 4 V keys are visible.
template <int QB, int VB>
struct TileFrag {
  uint32_t kw[QB / 4];
  uint32_t vw[4][VB / 4];
  bool vis[4];
};

constexpr int kMaxTps = 256;  // tiles per split (block-table entries staged in LDS)

template <typename T, int D, int NREP>
__global__ __launch_bounds__(256) void decode_split_kernel(const void *__restrict__ qp, ropekv_kv_cache c,
                                                           float sl2, float *__restrict__ ws, int tps, int splits) {
  using TR = ElemTraits<T>;
  constexpr int QB = (D / 4) * TR::kBytes;   // bytes of a lane's K / Q quarter-row
  constexpr int E = D / 16;                  // V dims per lane per key
  constexpr int VB = E * TR::kBytes;         // bytes of a lane's V piece per key
  using Frag = TileFrag<QB, VB>;
  __shared__ float s_p[4][NREP][kTile];
  __shared__ float s_corr[4][NREP];
  __shared__ float s_m[4][NREP], s_l[4][NREP];
  __shared__ float s_acc[4][NREP][D];
  __shared__ int s_bid[kMaxTps];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = c.num_kv_heads;
  const SeqTiles st = seq_tiles(c, b);
  // a length the planned splits cannot cover (table too short for seq_len) is flagged, not read
  if (split == splits - 1 && threadIdx.x == 0 && st.ntiles > splits * tps) dev_error(c.err_word, ROPEKV_DEV_BLOCK_RANGE);
  const int t_begin = split * tps;
  if (t_begin >= st.ntiles) return;
  const int t_end = min(st.ntiles, t_begin + tps);

  // stage this split's block ids (paged) so no tile waits on a dependent table load
  if (c.layout == ROPEKV_PAGED) {
    for (int i = threadIdx.x; i < t_end - t_begin; i += 256) {
      const int tile = t_begin + i;
      const int blk = tile < st.nsb ? tile : st.fr + (tile - st.nsb);
      s_bid[i] = (blk < c.max_blocks) ? c.block_table[(long)b * c.max_blocks + blk] : -1;
    }
  }

  // Q^T fragment: column `col` = query head g * NREP + col (zero beyond NREP)
  uint32_t qw[QB / 4];
  if (col < NREP) {
    const char *qrow = (const char *)qp + ((long)(b * Hkv * NREP + g * NREP + col) * D) * TR::kBytes;
    load_pieces<QB>(qw, qrow, grp);
  } else {
#pragma unroll
    for (int i = 0; i < QB / 4; ++i) qw[i] = 0u;
  }
  __syncthreads();

  const char *kbase = (const char *)c.k;
  const char *vbase = (const char *)c.v;
  const long head_base = ((long)b * Hkv + g) * (long)c.capacity * D;  // RING: slot 0 of (b, g)

  // Issue the loads of one tile (all in flight until first use).  Returns false for a null block.
  auto load_tile = [&](Frag &f, int tile) -> bool {
    long base;
    int pos0 = 0, slot0 = 0;
    bool ok = true;
    if (c.layout == ROPEKV_PAGED) {
      const int bid = s_bid[tile - t_begin];
      const int blk = tile < st.nsb ? tile : st.fr + (tile - st.nsb);
      pos0 = blk * kTile;
      ok = bid >= 0 && bid < c.num_blocks;
      base = ok ? ((long)bid * Hkv + g) * kTile * D : 0;
    } else {
      slot0 = tile * kTile;
      base = head_base;
    }
    auto roff = [&](int r) -> long {
      if (c.layout == ROPEKV_PAGED) return base + (long)r * D;
      return base + (long)min(slot0 + r, c.capacity - 1) * D;
    };
    auto visible = [&](int r) -> bool {
      if (!ok) return false;
      if (c.layout == ROPEKV_PAGED) {
        const int pos = pos0 + r;
        return pos < st.ns || (pos >= st.rs && pos < st.n);
      }
      const int slot = slot0 + r;
      if (slot >= c.capacity) return false;
      if (slot < c.sinks) return slot < st.ns;
      return imod(slot - c.sinks - st.oldest, c.window) < st.count;
    };
    if (ok) {
      load_pieces<QB>(f.kw, kbase + roff(col) * TR::kBytes, grp);
#pragma unroll
      for (int j = 0; j < 4; ++j) load_bytes<VB>(f.vw[j], vbase + roff(4 * grp + j) * TR::kBytes + col * VB);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) f.vis[j] = visible(4 * grp + j);
    return ok;
  };

  float m_run = kNegBig, l_run = 0.f;
  float acc[NREP][E];
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;

  bool bad_tile = false;
  int tile = t_begin + wave;
  Frag cur, nxt;
  bool cur_ok = tile < t_end ? load_tile(cur, tile) : false;
  for (; tile < t_end; tile += 4) {
    bool nxt_ok = false;
    if (tile + 4 < t_end) nxt_ok = load_tile(nxt, tile + 4);
    if (!cur_ok) {
      bad_tile = true;
    } else {
      const f32x4 sacc = qk_tile<T, D>(cur.kw, qw);
      float s[4];
      float mx = kNegBig;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[j] = cur.vis[j] ? sacc[j] * sl2 : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2f(m_run - m_new);
      float psum = 0.f;
      float pj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pj[j] = exp2f(s[j] - m_new);
        psum += pj[j];
      }
      l_run = l_run * corr + psum;
      m_run = m_new;
      if (col < NREP) {
        *(float4 *)&s_p[wave][col][4 * grp] = make_float4(pj[0], pj[1], pj[2], pj[3]);
        if (grp == 0) s_corr[wave][col] = corr;
      }
      // invisible keys have p = 0, but their rows may hold anything: zero them once
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!cur.vis[j]) {
#pragma unroll
          for (int w = 0; w < VB / 4; ++w) cur.vw[j][w] = 0u;
        }
      float vf[4][E];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < E; ++e) vf[j][e] = TR::get(cur.vw[j], e);
      wave_lds_sync();
      // V layout: this lane holds keys 4*grp + j, dims [col*E, col*E + E)
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        const float ch = s_corr[wave][h];  // the same value in every lane: a uniform branch
        const float4 ph = *(const float4 *)&s_p[wave][h][4 * grp];
        if (ch != 1.f) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= ch;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float a = acc[h][e];
          a = fmaf(ph.x, vf[0][e], a);
          a = fmaf(ph.y, vf[1][e], a);
          a = fmaf(ph.z, vf[2][e], a);
          a = fmaf(ph.w, vf[3][e], a);
          acc[h][e] = a;
        }
      }
      wave_lds_sync();
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }
  if (bad_tile && lane == 0) dev_error(c.err_word, ROPEKV_DEV_NULL_BLOCK);

  // merge the 4 lane groups of this wave (they share m per query head)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int h = 0; h < NREP; ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = acc[h][e];
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[h][e] = a;
    }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < NREP; ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][h][col * E + e] = acc[h][e];
    if (col < NREP) {
      s_m[wave][col] = m_run;
      s_l[wave][col] = l_run;
    }
  }
  __syncthreads();
  // merge the 4 waves and write this split's partial
  const int nwaves = min(4, t_end - t_begin);
  float *dst = ws + (((long)(b * Hkv + g) * splits + split) * NREP) * (D + 2);
  for (int idx = threadIdx.x; idx < NREP * D; idx += 256) {
    const int h = idx / D, dd = idx % D;
    float m = kNegBig;
    for (int w = 0; w < nwaves; ++w) m = fmaxf(m, s_m[w][h]);
    float a = 0.f, l = 0.f;
    for (int w = 0; w < nwaves; ++w) {
      const float f = exp2f(s_m[w][h] - m);
      a += f * s_acc[w][h][dd];
      l += f * s_l[w][h];
    }
    float *o = dst + (long)h * (D + 2);
    o[dd] = a;
    if (dd == 0) {
      o[D] = m;
      o[D + 1] = l;
    }
  }
}

// ---- int8 KV (codes + one fp32 scale per cached row) ----
//
// K and V rows are int8 codes c with a per-row scale sc (x ~ c * sc, the row
// quantizer of the append).  |c| <= 127 is exact in bf16, so both products run
// on bf16 MFMAs with the codes converted in registers:
//   S^T = Kc . Q^T (16x16x32), then s = S^T * k_scale(key) in the log2 domain;
//   O  += (P * v_scale(key)) . Vc (16x16x16, one MFMA per V column block).
// The S^T fragment a lane holds (head `col`, keys 4 grp + j) is exactly the A
// operand of the second MFMA, so P never leaves registers.  The V operand of
// MFMA e is column dim col * (D / 16) + e, keys 4 grp + j.  Output row
// 4 grp + j of MFMA e is query head 4 grp + j, dim col * (D / 16) + e.
//
// An int8 tile is half the bytes of a bf16 one, so a wave needs more tiles in
// flight to keep HBM busy.  Tiles are staged through LDS with direct
// global -> LDS loads (no registers held while in flight): each wave keeps a
// ring of NST tile stages and runs NST - 1 tiles ahead, waiting on the vector
// memory counter for the oldest.  Key rows are stored with their 16-byte
// chunks XOR-swizzled by row so the MFMA operand reads hit distinct banks.
// Direct global -> LDS loads: 64 lanes x N bytes land at LDS [m0 + N * lane].  Issued as
// inline assembly so the only waits on them are the explicit vmcnt waits of the
// pipeline (the stage being read is never the one being filled).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void dma16(const void *gsrc, const void *lds_base) {
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_offset(lds_base))
                   : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *gsrc, const void *lds_base) {
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(lds_offset(lds_base))
                   : "memory", "m0");
}

__device__ __forceinline__ float code_f(uint32_t w, int byte) { return (float)(int8_t)(w >> (8 * byte)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// two floats -> one packed bf16 word (round to nearest even; exact for codes)
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
  __asm__ volatile("" ::: "memory");
}

template <int D>
struct I8Stage {
  uint8_t k[16 * D];  // 16-byte chunk c of row r at chunk slot r * (D / 16) + (c ^ swz(r))
  uint8_t v[16 * D];  // row-major
  float sc[32];       // key scales of rows 0..15, then value scales
};

template <int D>
__device__ __forceinline__ int kswz(int row) {
  constexpr int CPR = D / 16;
  return (row * CPR / 8) % CPR;
}

template <int D, int NREP, int LAYOUT, int NST>
__global__ __launch_bounds__(256) void decode_split_i8_kernel(const void *__restrict__ qp, ropekv_kv_cache c,
                                                              float sl2, float *__restrict__ ws, int tps,
                                                              int splits) {
  constexpr int QB = D / 4;         // key-code bytes per lane per tile
  constexpr int E = D / 16;         // value-code bytes per lane per key = PV MFMAs per tile
  constexpr int CPR = D / 16;       // 16-byte chunks per cached row
  constexpr int KI = 16 * D / 1024; // 1 KB direct loads per tile for K (and for V)
  constexpr int NI = 2 * KI + 1;    // direct loads per stage (K, V, scales)
  constexpr bool kPaged = LAYOUT == ROPEKV_PAGED;
  static_assert(4 * NST * sizeof(I8Stage<D>) >= 4 * NREP * D * sizeof(float), "merge buffer aliases the stages");
  static_assert(NST >= 2 && NST <= 4, "stages per wave");
  __shared__ __attribute__((aligned(16))) I8Stage<D> s_st[4][NST];
  __shared__ float s_m[4][NREP], s_l[4][NREP];
  __shared__ int s_bid[kMaxTps];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the pipeline branches are scalar
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = c.num_kv_heads;
  const SeqTiles st = seq_tiles(c, b);
  if (split == splits - 1 && threadIdx.x == 0 && st.ntiles > splits * tps) dev_error(c.err_word, ROPEKV_DEV_BLOCK_RANGE);
  const int t_begin = split * tps;
  if (t_begin >= st.ntiles) return;
  const int t_end = min(st.ntiles, t_begin + tps);

  if (kPaged) {
    for (int i = threadIdx.x; i < t_end - t_begin; i += 256) {
      const int tile = t_begin + i;
      const int blk = tile < st.nsb ? tile : st.fr + (tile - st.nsb);
      s_bid[i] = (blk < c.max_blocks) ? c.block_table[(long)b * c.max_blocks + blk] : -1;
    }
  }

  // Q^T fragment (bf16): local element u of this lane is d = (4 (u / 16) + grp) * 16 + u % 16,
  // the same d as the key bytes of piece u / 16 the lane reads.
  uint32_t qw[D / 8];
  if (col < NREP) {
    const char *qrow = (const char *)qp + (long)(b * Hkv * NREP + g * NREP + col) * D * 2;
#pragma unroll
    for (int i = 0; i < QB / 16; ++i) load_bytes<32>(qw + 8 * i, qrow + (4 * i + grp) * 32);
  } else {
#pragma unroll
    for (int i = 0; i < D / 8; ++i) qw[i] = 0u;
  }
  wait_vmcnt<0>();
  if (c.k_int8_mode & ROPEKV_I8_HADAMARD) {
    // Keys hold codes of H k: score with H q (H orthonormal, so (H q).(H k) = q.k).  The lane's
    // local index u covers the bits of d other than the two lane-group bits (d = (4 (u / 16) + grp) * 16
    // + u % 16), so the butterflies over u stay in the lane and the other two are lane-group exchanges.
    constexpr int NU = D / 4;
    float f[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) f[u] = __uint_as_float((u & 1) ? (qw[u >> 1] & 0xffff0000u) : (qw[u >> 1] << 16));
#pragma unroll
    for (int h = 1; h < NU; h <<= 1)
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if ((u & h) == 0) {
          const float x0 = f[u], x1 = f[u + h];
          f[u] = x0 + x1;
          f[u + h] = x0 - x1;
        }
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float p = __shfl_xor(f[u], m);
        f[u] = upper ? p - f[u] : f[u] + p;
      }
    }
    const float norm = 1.0f / sqrtf((float)D);
#pragma unroll
    for (int w = 0; w < NU / 2; ++w) qw[w] = pack2_bf16(f[2 * w] * norm, f[2 * w + 1] * norm);
  }
  __syncthreads();

  const char *kbase = (const char *)c.k;
  const char *vbase = (const char *)c.v;
  const long head_row0 = ((long)b * Hkv + g) * (long)c.capacity;  // RING: row of slot 0 of (b, g)
  const int C = c.capacity;

  // Tile geometry: cached row of tile row r, and whether the tile maps to memory.
  struct TileAt {
    long row0;  // PAGED: row of tile row 0 (0 for a null block); RING: row of slot 0
    int pos0;   // PAGED: position of row 0; RING: slot of row 0
    bool ok;
  };
  auto tile_at = [&](int tile) -> TileAt {
    TileAt t;
    if (kPaged) {
      const int bid = s_bid[tile - t_begin];
      const int blk = tile < st.nsb ? tile : st.fr + (tile - st.nsb);
      t.pos0 = blk * kTile;
      t.ok = bid >= 0 && bid < c.num_blocks;
      t.row0 = t.ok ? ((long)bid * Hkv + g) * kTile : 0;
    } else {
      t.pos0 = tile * kTile;
      t.ok = true;
      t.row0 = head_row0;
    }
    return t;
  };
  auto row_of = [&](const TileAt &t, int r) -> long { return kPaged ? t.row0 + r : t.row0 + min(t.pos0 + r, C - 1); };

  // Start the direct loads of one tile into a stage: always NI wave instructions, all in bounds
  // (a null block reads pool row 0 and is never visible).
  auto issue = [&](int tile, int stage) {
    const TileAt t = tile_at(tile);
    I8Stage<D> &S = s_st[wave][stage];
#pragma unroll
    for (int n = 0; n < KI; ++n) {
      const int p = 64 * n + lane;
      const int r = p / CPR;
      const int ch = (p % CPR) ^ kswz<D>(r);
      dma16(kbase + row_of(t, r) * D + ch * 16, S.k + 1024 * n);
    }
#pragma unroll
    for (int n = 0; n < KI; ++n) {
      const int p = 64 * n + lane;
      dma16(vbase + row_of(t, p / CPR) * D + (p % CPR) * 16, S.v + 1024 * n);
    }
    if (lane < 32) {
      const float *src = (lane < 16 ? c.k_scale : c.v_scale) + row_of(t, lane & 15);
      dma4(src, S.sc);
    }
  };
  auto visible = [&](const TileAt &t, int r) -> bool {
    if (!t.ok) return false;
    if (kPaged) {
      const int pos = t.pos0 + r;
      return pos < st.ns || (pos >= st.rs && pos < st.n);
    }
    const int slot = t.pos0 + r;
    if (slot >= C) return false;
    if (slot < c.sinks) return slot < st.ns;
    int i = slot - c.sinks - st.oldest;
    if (i < 0) i += c.window;
    return i < st.count;
  };

  float m_run = kNegBig, l_run = 0.f;
  f32x4 acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool bad_tile = false;
  const int first = t_begin + wave;
  const int nk = first < t_end ? (t_end - first + 3) / 4 : 0;  // tiles of this wave: first + 4 k
#pragma unroll
  for (int k = 0; k < NST - 1; ++k)
    if (k < nk) issue(first + 4 * k, k);
  // One tile: stage u of the ring (a constant after unrolling, so the compiler can
  // tell the stage being read from the stage being filled).
  auto step = [&](int k, int u) {
    if (k + NST - 1 < nk) {
      issue(first + 4 * (k + NST - 1), (u + NST - 1) % NST);
      wait_vmcnt<(NST - 1) * NI>();
    } else {
      const int ahead = nk - 1 - k;  // stages issued after this one (< NST - 1)
      if (ahead >= 2) wait_vmcnt<2 * NI>();
      else if (ahead == 1) wait_vmcnt<NI>();
      else wait_vmcnt<0>();
    }
    const I8Stage<D> &S = s_st[wave][u];
    const TileAt t = tile_at(first + 4 * k);
    bad_tile |= !t.ok;
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < QB / 16; ++i) {
      const int ch = 4 * i + grp;
      const u32x4_t kp = *(const u32x4_t *)(S.k + (col * CPR + (ch ^ kswz<D>(col))) * 16);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int tt = 2 * i + h;  // MFMA step: local elements 8 tt .. 8 tt + 7
        const uint32_t w0 = kp[2 * h], w1 = kp[2 * h + 1];
        const u32x4_t av = {pack2_bf16(code_f(w0, 0), code_f(w0, 1)), pack2_bf16(code_f(w0, 2), code_f(w0, 3)),
                            pack2_bf16(code_f(w1, 0), code_f(w1, 1)), pack2_bf16(code_f(w1, 2), code_f(w1, 3))};
        const u32x4_t bv = {qw[4 * tt], qw[4 * tt + 1], qw[4 * tt + 2], qw[4 * tt + 3]};
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv),
                                                       sacc, 0, 0, 0);
      }
    }
    const float4 ks = *(const float4 *)&S.sc[4 * grp];
    const float4 vs = *(const float4 *)&S.sc[16 + 4 * grp];
    const float ksj[4] = {ks.x, ks.y, ks.z, ks.w};
    const float vsj[4] = {vs.x, vs.y, vs.z, vs.w};
    float s[4];
    float mx = kNegBig;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = visible(t, 4 * grp + j) ? sacc[j] * (ksj[j] * sl2) : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float pv[4], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m_new);  // 0 for an invisible key
      psum += p;
      pv[j] = p > 0.f ? p * vsj[j] : 0.f;   // scale rows of invisible keys may hold anything
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    // rescale the output rows (heads 4 grp + j) whose running maximum moved
    if (__any(corr != 1.f)) {
      float cj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) cj[j] = __shfl(corr, 4 * grp + j);
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[e][j] *= cj[j];
    }
    const short4_t pa = __builtin_bit_cast(short4_t, (uint2){pack2_bf16(pv[0], pv[1]), pack2_bf16(pv[2], pv[3])});
    uint32_t vw[4][(E + 3) / 4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t *src = S.v + (4 * grp + j) * D + col * E;
      if constexpr (E == 8) {
        const uint2 x = *(const uint2 *)src;
        vw[j][0] = x.x;
        vw[j][1] = x.y;
      } else {
        vw[j][0] = *(const uint32_t *)src;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int wsel = e >> 2, byte = e & 3;
      const short4_t vb = __builtin_bit_cast(
          short4_t, (uint2){pack2_bf16(code_f(vw[0][wsel], byte), code_f(vw[1][wsel], byte)),
                            pack2_bf16(code_f(vw[2][wsel], byte), code_f(vw[3][wsel], byte))});
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[e], 0, 0, 0);
    }
  };
  for (int k0 = 0; k0 < nk; k0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u)
      if (k0 + u < nk) step(k0 + u, u);
  }
  if (bad_tile && lane == 0) dev_error(c.err_word, ROPEKV_DEV_NULL_BLOCK);

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // every wave is done with its stages: they now hold the merge buffer
  float(*s_acc)[NREP][D] = reinterpret_cast<float(*)[NREP][D]>(&s_st[0][0]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * grp + j;
    if (h < NREP) {
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][h][col * E + e] = acc[e][j];
    }
  }
  if (grp == 0 && col < NREP) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  __syncthreads();
  const int nwaves = min(4, t_end - t_begin);
  float *dst = ws + (((long)(b * Hkv + g) * splits + split) * NREP) * (D + 2);
  for (int idx = threadIdx.x; idx < NREP * D; idx += 256) {
    const int h = idx / D, dd = idx % D;
    float m = kNegBig;
    for (int w = 0; w < nwaves; ++w) m = fmaxf(m, s_m[w][h]);
    float a = 0.f, l = 0.f;
    for (int w = 0; w < nwaves; ++w) {
      const float f = exp2f(s_m[w][h] - m);
      a += f * s_acc[w][h][dd];
      l += f * s_l[w][h];
    }
    float *o = dst + (long)h * (D + 2);
    o[dd] = a;
    if (dd == 0) {
      o[D] = m;
      o[D + 1] = l;
    }
  }
}

// Merge the split partials of one (sequence, query head): weights exp2(m_s - m)
// computed once per split, then one coalesced pass over the partial rows.
constexpr int kMaxSplits = 1024;

template <typename T, int D, int NREP>
__global__ __launch_bounds__(128) void decode_combine_kernel(ropekv_kv_cache c, const float *__restrict__ ws,
                                                             const float *__restrict__ sinks, void *__restrict__ out,
                                                             int tps, int splits) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[128];
  const int h = blockIdx.x, b = blockIdx.y;
  const int Hkv = c.num_kv_heads;
  const int g = h / NREP, hh = h % NREP;
  const SeqTiles st = seq_tiles(c, b);
  const int used = min(min((st.ntiles + tps - 1) / tps, splits), kMaxSplits);
  const long obase = ((long)b * Hkv * NREP + h) * D;
  const float *src = ws + (((long)(b * Hkv + g) * splits) * NREP + hh) * (D + 2);
  const long sstride = (long)NREP * (D + 2);
  // global max over splits
  float m = kNegBig;
  for (int s = threadIdx.x; s < used; s += blockDim.x) m = fmaxf(m, src[s * sstride + D]);
  s_red[threadIdx.x] = m;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) s_red[threadIdx.x] = fmaxf(s_red[threadIdx.x], s_red[threadIdx.x + w]);
    __syncthreads();
  }
  m = s_red[0];
  // a learned sink logit joins the normaliser (log2 units like the partial maxima)
  const float sink2 = sinks ? sinks[h] * kLog2e : -INFINITY;
  if (used > 0) m = fmaxf(m, sink2);
  __syncthreads();
  // per-split weights and the total weight l
  float l = 0.f;
  for (int s = threadIdx.x; s < used; s += blockDim.x) {
    const float w = exp2f(src[s * sstride + D] - m);
    s_w[s] = w;
    l += w * src[s * sstride + D + 1];
  }
  s_red[threadIdx.x] = l;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) s_red[threadIdx.x] += s_red[threadIdx.x + w];
    __syncthreads();
  }
  l = s_red[0];
  if (sinks && used > 0) l += exp2f(sink2 - m);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int dd = threadIdx.x; dd < D; dd += blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < used; ++s) a = fmaf(s_w[s], src[s * sstride + dd], a);
    ElemTraits<T>::put(out, obase + dd, a * inv);
  }
}

template <typename T, int D, int NREP>
hipError_t launch_decode_t(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                           void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  dim3 grid(pl.splits, c.num_kv_heads, batch);
  hipLaunchKernelGGL((decode_split_kernel<T, D, NREP>), grid, dim3(256), 0, s, q, c, sl2, ws, pl.tiles_per_split,
                     pl.splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, NREP>), dim3(c.num_kv_heads * NREP, batch), dim3(128), 0, s, c,
                     ws, sinks, out, pl.tiles_per_split, pl.splits);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sk, void *out,
                           float *ws, const DecodePlan &pl, hipStream_t s) {
  switch (pl.n_rep) {
    case 1: return launch_decode_t<T, D, 1>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 2: return launch_decode_t<T, D, 2>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 4: return launch_decode_t<T, D, 4>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 8: return launch_decode_t<T, D, 8>(q, batch, c, sl2, sk, out, ws, pl, s);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kI8Stages = 3;  // tile stages per wave (int8 decode)

template <int D, int NREP>
hipError_t launch_decode_i8_t(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                              void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  dim3 grid(pl.splits, c.num_kv_heads, batch);
  if (c.layout == ROPEKV_PAGED)
    hipLaunchKernelGGL((decode_split_i8_kernel<D, NREP, ROPEKV_PAGED, kI8Stages>), grid, dim3(256), 0, s, q, c, sl2, ws,
                       pl.tiles_per_split, pl.splits);
  else
    hipLaunchKernelGGL((decode_split_i8_kernel<D, NREP, ROPEKV_RING, kI8Stages>), grid, dim3(256), 0, s, q, c, sl2, ws,
                       pl.tiles_per_split, pl.splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<bf16_t, D, NREP>), dim3(c.num_kv_heads * NREP, batch), dim3(128), 0, s,
                     c, ws, sinks, out, pl.tiles_per_split, pl.splits);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_i8_d(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sk,
                              void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  switch (pl.n_rep) {
    case 1: return launch_decode_i8_t<D, 1>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 2: return launch_decode_i8_t<D, 2>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 4: return launch_decode_i8_t<D, 4>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 8: return launch_decode_i8_t<D, 8>(q, batch, c, sl2, sk, out, ws, pl, s);
    default: return hipErrorInvalidValue;
  }
}

// --- visible-slot enumeration (test-facing; one thread walks the set) ---
__global__ void visible_slots_kernel(ropekv_kv_cache c, int b, int32_t *pos_out, int64_t *off_out, int max_out,
                                     int32_t *n_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int D = c.head_dim;
  const int n = c.seq_len[b];
  int cnt = 0;
  auto emit = [&](int pos, long off) {
    if (cnt < max_out) {
      pos_out[cnt] = pos;
      off_out[cnt] = off;
    }
    ++cnt;
  };
  if (n > 0) {
    if (c.layout == ROPEKV_PAGED) {
      for (int p = 0; p < n; ++p) {
        const bool vis = c.window == 0 || p < c.sinks || (n - 1) - p < c.window;
        if (!vis) continue;
        const int blk = p / c.block_size;
        const int bid = blk < c.max_blocks ? c.block_table[(long)b * c.max_blocks + blk] : -1;
        emit(p, bid < 0 ? -1 : (((long)bid * c.num_kv_heads) * c.block_size + p % c.block_size) * D);
      }
    } else {
      const SeqTiles st = seq_tiles(c, b);
      const long base = ((long)b * c.num_kv_heads) * (long)c.capacity * D;
      for (int p = 0; p < st.ns; ++p) emit(p, base + (long)p * D);
      for (int i = 0; i < st.count; ++i) {
        const int slot = c.sinks + (st.oldest + i) % c.window;
        emit(n - st.count + i, base + (long)slot * D);
      }
    }
  }
  *n_out = cnt;
}

}  // namespace

DecodePlan plan_decode(int batch, int n_q_heads, const ropekv_kv_cache &c) {
  DecodePlan pl;
  pl.n_rep = n_q_heads / c.num_kv_heads;
  int max_tiles;
  if (c.layout == ROPEKV_PAGED) {
    if (c.window == 0) {
      max_tiles = c.max_blocks;
    } else {
      max_tiles = (c.sinks + kTile - 1) / kTile + c.window / kTile + 2;
      if (max_tiles > c.max_blocks) max_tiles = c.max_blocks;
    }
  } else {
    max_tiles = (c.capacity + kTile - 1) / kTile;
  }
  if (max_tiles < 1) max_tiles = 1;
  // tiles per split: aim for ~8192 workgroups over the batch, 8..128 tiles each
  const long work = (long)max_tiles * batch * c.num_kv_heads;
  int tps = 8;
  while (tps < 128 && (long)tps * 8192 < work) tps *= 2;
  if (const char *e = getenv("ROPEKV_DECODE_TPS")) {
    const int v = atoi(e);
    if (v >= 1 && v <= kMaxTps) tps = v;
  }
  while ((max_tiles + tps - 1) / tps > kMaxSplits && tps < kMaxTps) tps *= 2;
  pl.max_tiles = max_tiles;
  pl.tiles_per_split = tps;
  pl.splits = (max_tiles + tps - 1) / tps;
  const int dd = c.head_dim + 2;
  pl.ws_bytes = (size_t)batch * c.num_kv_heads * pl.splits * pl.n_rep * dd * sizeof(float);
  return pl;
}

hipError_t launch_decode(const void *q, int batch, int n_q_heads, const ropekv_kv_cache &c, float scale,
                         const float *sinks, void *out, void *ws, const DecodePlan &pl, hipStream_t s) {
  (void)n_q_heads;
  const float sl2 = scale * kLog2e;
  float *w = (float *)ws;
  if (c.kv_dtype == ROPEKV_BF16) {
    if (c.head_dim == 128) return launch_decode_d<bf16_t, 128>(q, batch, c, sl2, sinks, out, w, pl, s);
    if (c.head_dim == 64) return launch_decode_d<bf16_t, 64>(q, batch, c, sl2, sinks, out, w, pl, s);
  } else if (c.kv_dtype == ROPEKV_F32) {
    if (c.head_dim == 128) return launch_decode_d<float, 128>(q, batch, c, sl2, sinks, out, w, pl, s);
    if (c.head_dim == 64) return launch_decode_d<float, 64>(q, batch, c, sl2, sinks, out, w, pl, s);
  } else if (c.kv_dtype == ROPEKV_I8) {  // int8 codes, bf16 q and out
    if (c.head_dim == 128) return launch_decode_i8_d<128>(q, batch, c, sl2, sinks, out, w, pl, s);
    if (c.head_dim == 64) return launch_decode_i8_d<64>(q, batch, c, sl2, sinks, out, w, pl, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_visible_slots(const ropekv_kv_cache &c, int seq, int32_t *pos_out, int64_t *off_out, int max_out,
                                int32_t *n_out, hipStream_t s) {
  hipLaunchKernelGGL(visible_slots_kernel, dim3(1), dim3(64), 0, s, c, seq, pos_out, off_out, max_out, n_out);
  return hipGetLastError();
}

}  // namespace ropekv
