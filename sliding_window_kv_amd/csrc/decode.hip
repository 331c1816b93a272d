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
// the log2 domain, masked, online softmax per query head.  bf16 caches:
// O^T += V^T . P^T on MFMA (16x16x16): the S^T fragment a lane holds (keys
// 4 grp + j, head col) is the B operand once rounded to bf16, and the lane's
// V pieces (keys 4 grp + j, dims E col .. E col + E - 1, E = d / 16) give, dim
// by dim, the A operand of E MFMAs (block mt covers dims E i + mt, i = 0..15).  fp32 caches
// keep P in fp32: P and the correction factors go through a small per-wave LDS
// slot to the layout in which each lane holds 4 keys x (d/16) dims of V, and
// O += P V on the VALU.
#include <stdlib.h>

#include <mutex>

#include "decode_common.hpp"

namespace ropekv {

// Split-K partials of the allocation-free decode call: one copy of this array
// per GPU, loaded with the library's code object and held until the process
// ends.  Host code never passes the array's name to a kernel (on the host the
// name is a stand-in, not a device address); it asks for each device's address
// once (decode_scratch) and passes that.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {

using namespace decode_detail;

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

typedef short short4v __attribute__((ext_vector_type(4)));

// K and V pieces of one tile held by one lane, plus which of its 4 V keys are visible.
template <int QB, int VB>
struct TileFrag {
  uint32_t kw[QB / 4];
  uint32_t vw[4][VB / 4];
  bool vis[4];
};

// NW waves per workgroup, each taking every NW-th tile of the workgroup's run.  Split mode
// (out == nullptr): the merged partial (acc, m, l) goes to ws for the combine launch.  Direct
// mode (one split per sequence and KV head): the workgroup merges its waves, adds the learned
// sink logit and writes the normalised output itself, so no partial leaves the chip and no
// second launch runs.
template <typename T, int D, int NREP, int NW>
__global__ __launch_bounds__(64 * NW, sizeof(T) == 2 ? 3 : 2) void decode_split_kernel(
    const void *__restrict__ qp, ropekv_kv_cache c, float sl2, float *__restrict__ ws, int tps, int splits,
    const float *__restrict__ sinks, void *__restrict__ out) {
  using TR = ElemTraits<T>;
  constexpr int NT = 64 * NW;                // threads
  constexpr int QB = (D / 4) * TR::kBytes;   // bytes of a lane's K / Q quarter-row
  constexpr int E = D / 16;                  // V dims per lane per key
  constexpr int VB = E * TR::kBytes;         // bytes of a lane's V piece per key
  using Frag = TileFrag<QB, VB>;
  constexpr bool kMfmaPV = sizeof(T) == 2;
  __shared__ float s_p[kMfmaPV ? 1 : NW][NREP][kTile];
  __shared__ float s_corr[kMfmaPV ? 1 : NW][NREP];
  __shared__ float s_m[NW][NREP], s_l[NW][NREP];
  __shared__ float s_acc[NW][NREP][D];
  __shared__ int s_bid[kMaxDirectTiles];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int Hkv = c.num_kv_heads;
  const SeqTiles st = seq_tiles(c, b);
  // a length the planned splits cannot cover (table too short for seq_len) is flagged, not read
  if (split == splits - 1 && threadIdx.x == 0 && st.ntiles > splits * tps) dev_error(c.err_word, ROPEKV_DEV_BLOCK_RANGE);
  const int t_begin = split * tps;
  if (t_begin >= st.ntiles) {
    if (out != nullptr) {  // direct mode, empty sequence: a zero row
      const long obase = ((long)b * Hkv + g) * NREP * D;
      for (int idx = threadIdx.x; idx < NREP * D; idx += NT) TR::put(out, obase + idx, 0.f);
    }
    return;
  }
  const int t_end = min(st.ntiles, t_begin + tps);

  // stage this split's block ids (paged) so no tile waits on a dependent table load
  if (c.layout == ROPEKV_PAGED) {
    for (int i = threadIdx.x; i < t_end - t_begin; i += NT) {
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
  float acc[kMfmaPV ? 1 : NREP][E];      // VALU path: head h, dims col * E + e
  f32x4 oacc[kMfmaPV ? D / 16 : 1];     // MFMA path: O^T block mt, dims E (4 grp + r) + mt, head col
#pragma unroll
  for (int h = 0; h < (kMfmaPV ? 1 : NREP); ++h)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int mt = 0; mt < (kMfmaPV ? D / 16 : 1); ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool bad_tile = false;
  int tile = t_begin + wave;
  Frag cur, nxt;
  bool cur_ok = tile < t_end ? load_tile(cur, tile) : false;
  for (; tile < t_end; tile += NW) {
    bool nxt_ok = false;
    if (tile + NW < t_end) nxt_ok = load_tile(nxt, tile + NW);
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
      // invisible keys have p = 0, but their rows may hold anything: zero them once
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!cur.vis[j]) {
#pragma unroll
          for (int w = 0; w < VB / 4; ++w) cur.vw[j][w] = 0u;
        }
      if constexpr (kMfmaPV) {
        // rescale this lane's column (its head) when its running maximum moved
        if (__any(corr != 1.f)) {
#pragma unroll
          for (int mt = 0; mt < D / 16; ++mt) oacc[mt] *= corr;
        }
        // B = P^T (keys 4 grp + j, head col) in bf16; columns beyond NREP stay zero
        const float pc[4] = {col < NREP ? pj[0] : 0.f, col < NREP ? pj[1] : 0.f, col < NREP ? pj[2] : 0.f,
                             col < NREP ? pj[3] : 0.f};
        const short4v pb = __builtin_bit_cast(short4v, (uint2){pack2_bf16_rne(pc[0], pc[1]), pack2_bf16_rne(pc[2], pc[3])});
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
          // A = V^T rows E i + mt: element mt of this lane's E dims, from each of its 4 keys
          const int w = mt >> 1;
          const uint32_t sel = (mt & 1) ? 0x07060302u : 0x05040100u;  // high or low halves of two words
          const uint32_t a01 = __builtin_amdgcn_perm(cur.vw[1][w], cur.vw[0][w], sel);
          const uint32_t a23 = __builtin_amdgcn_perm(cur.vw[3][w], cur.vw[2][w], sel);
          const short4v av = __builtin_bit_cast(short4v, (uint2){a01, a23});
          oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, oacc[mt], 0, 0, 0);
        }
      } else {
        if (col < NREP) {
          *(float4 *)&s_p[wave][col][4 * grp] = make_float4(pj[0], pj[1], pj[2], pj[3]);
          if (grp == 0) s_corr[wave][col] = corr;
        }
        float vf[4][E];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < E; ++e) vf[j][e] = TR::get(cur.vw[j], e);
        wave_lds_sync();
        // V layout: this lane holds keys 4*grp + j, dims [col*E, col*E + E)
#pragma unroll
        for (int h = 0; h < (kMfmaPV ? 1 : NREP); ++h) {
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
    }
    cur = nxt;
    cur_ok = nxt_ok;
  }
  if (bad_tile && lane == 0) dev_error(c.err_word, ROPEKV_DEV_NULL_BLOCK);

  // merge the 4 lane groups of this wave (they share m per query head)
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if constexpr (kMfmaPV) {
    // the MFMAs summed over all 16 keys of each tile: lanes hold distinct (dim, head) entries
    if (col < NREP) {
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_acc[wave][col][E * (4 * grp + r) + mt] = oacc[mt][r];
      if (grp == 0) {
        s_m[wave][col] = m_run;
        s_l[wave][col] = l_run;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < (kMfmaPV ? 1 : NREP); ++h)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = acc[h][e];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        acc[h][e] = a;
      }
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < (kMfmaPV ? 1 : NREP); ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) s_acc[wave][h][col * E + e] = acc[h][e];
      if (col < NREP) {
        s_m[wave][col] = m_run;
        s_l[wave][col] = l_run;
      }
    }
  }
  __syncthreads();
  // merge the waves: this split's partial, or (direct mode) the normalised output
  const int nwaves = min(NW, t_end - t_begin);
  if (out == nullptr) {
    float *dst = ws + (((long)(b * Hkv + g) * splits + split) * NREP) * (D + 2);
    for (int idx = threadIdx.x; idx < NREP * D; idx += NT) {
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
  } else {
    const long obase = ((long)b * Hkv + g) * NREP * D;
    for (int idx = threadIdx.x; idx < NREP * D; idx += NT) {
      const int h = idx / D, dd = idx % D;
      float m = kNegBig;
      for (int w = 0; w < nwaves; ++w) m = fmaxf(m, s_m[w][h]);
      // a learned sink logit joins the normaliser (log2 units like the running maxima)
      const float sink2 = sinks ? sinks[g * NREP + h] * kLog2e : -INFINITY;
      m = fmaxf(m, sink2);
      float a = 0.f, l = 0.f;
      for (int w = 0; w < nwaves; ++w) {
        const float f = exp2f(s_m[w][h] - m);
        a += f * s_acc[w][h][dd];
        l += f * s_l[w][h];
      }
      if (sinks) l += exp2f(sink2 - m);
      TR::put(out, obase + idx, l > 0.f ? a * (1.f / l) : 0.f);
    }
  }
}

template <typename T, int D, int NREP>
hipError_t launch_decode_t(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                           void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  dim3 grid(pl.splits, c.num_kv_heads, batch);
  if (pl.direct) {
    constexpr int NWD = sizeof(T) == 2 ? kDirectWaves : kDirectWavesF32;
    hipLaunchKernelGGL((decode_split_kernel<T, D, NREP, NWD>), grid, dim3(64 * NWD), 0, s, q, c, sl2, ws,
                       pl.tiles_per_split, pl.splits, sinks, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_split_kernel<T, D, NREP, 4>), grid, dim3(256), 0, s, q, c, sl2, ws, pl.tiles_per_split,
                     pl.splits, (const float *)nullptr, (void *)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, NREP>), dim3(c.num_kv_heads, batch), dim3(256), 0, s, c,
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
  // splits: the fewest that still give about two workgroups per CU (512 over the batch and
  // KV heads) with at most kMaxTps tiles each, the tiles then spread evenly over them.  Long
  // splits amortise each workgroup's start (sequence state, block ids, first loads): on the
  // ring-window layer 2 splits of 129 tiles run 12% faster than 9 of 29, and the batch-64 x
  // 32768 and batch-32 x 131072 layers gain 1-3% over 128-tile splits.
  const long units = (long)batch * c.num_kv_heads;
  pl.direct = false;
  if ((c.kv_dtype == ROPEKV_BF16 || c.kv_dtype == ROPEKV_F32) && units >= 256 && max_tiles <= kMaxDirectTiles) {
    // enough (sequence, KV head) units to give every CU a workgroup, and short runs: one wide
    // workgroup per unit writes its output directly (no partials, no combine launch)
    pl.direct = true;
    pl.max_tiles = max_tiles;
    pl.tiles_per_split = max_tiles;
    pl.splits = 1;
    pl.ws_bytes = 0;
    return pl;
  }
  int splits = (int)((512 + units - 1) / units);
  splits = max(splits, (max_tiles + kMaxTps - 1) / kMaxTps);
  splits = min(splits, max_tiles);
  int tps = (max_tiles + splits - 1) / splits;
  while ((max_tiles + tps - 1) / tps > kMaxSplits && tps < kMaxTps) tps = min(2 * tps, kMaxTps);
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
  } else if (c.kv_dtype == ROPEKV_I8 || c.kv_dtype == ROPEKV_FP8) {  // 8-bit codes, bf16 q and out
    return launch_decode_8bit(q, batch, c, sl2, sinks, out, w, pl, s);
  }
  return hipErrorInvalidValue;
}

hipError_t decode_scratch(float **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = (float *)p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_visible_slots(const ropekv_kv_cache &c, int seq, int32_t *pos_out, int64_t *off_out, int max_out,
                                int32_t *n_out, hipStream_t s) {
  hipLaunchKernelGGL(visible_slots_kernel, dim3(1), dim3(64), 0, s, c, seq, pos_out, off_out, max_out, n_out);
  return hipGetLastError();
}

}  // namespace ropekv
