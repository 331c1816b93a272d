// Split-K decode attention over an 8-bit KV cache (int8 or E4M3 codes + one fp32
// scale per cached row), the same visible-set walk and split merge as the 16-bit
// path.
//
// "#2961 rope: --rope-scaling dynamic" ("What it does": int8 K with or without
// the Hadamard) stores keys as int8 rows; "vLLM, from the inside out" (memory
// levers) stores the KV cache as FP8; "Inference & 128K Long Context" (4.3:
// decode is memory bound) is why halving the bytes per key matters.
#include "decode_common.hpp"

namespace ropekv {

namespace {

using namespace decode_detail;

// ---- 8-bit KV (codes + one fp32 scale per cached row) ----
//
// K and V rows are 8-bit codes c with a per-row scale sc (x ~ c * sc, the row
// quantizer of the append).  Every int8 code (|c| <= 127) and every finite E4M3
// value (3 mantissa bits, exponents -9 .. 8) is exact in bf16, so both products
// run on bf16 MFMAs with the codes converted in registers:
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// The four codes of a word (byte b = code b) as exact floats: int8 by sign
// extension, E4M3 by the hardware's fp8 -> fp32 conversion (two per instruction).
// The E4M3 operands of the products skip the floats: fp8x2_bf16 below converts two
// codes straight to a packed bf16 word.
template <int KVDT>
__device__ __forceinline__ void codes4(uint32_t w, float *f) {
  if constexpr (KVDT == ROPEKV_FP8) {
    const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) f[b] = (float)(int8_t)(w >> (8 * b));
  }
}

// two E4M3 codes (the low or the high half of w) -> one packed bf16 word, exactly (every finite
// E4M3 value is a bf16 value; unit scale)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// two floats -> one packed bf16 word (round to nearest even; exact for codes)
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const float2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
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

template <int D, int NREP, int LAYOUT, int NST, int KVDT>
__global__ __launch_bounds__(256) void decode_split_8bit_kernel(const void *__restrict__ qp, ropekv_kv_cache c,
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
      dma16_stream(kbase + row_of(t, r) * D + ch * 16, S.k + 1024 * n);
    }
#pragma unroll
    for (int n = 0; n < KI; ++n) {
      const int p = 64 * n + lane;
      dma16_stream(vbase + row_of(t, p / CPR) * D + (p % CPR) * 16, S.v + 1024 * n);
    }
    // the scales go through the caches: a tile's 16 scales are half of a 128-byte line whose other
    // half (the next KV head's tile) another workgroup reads soon after; streamed past the L2 that
    // line was fetched twice (+1.4 % HBM bytes, 4 % slower)
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
        u32x4_t av;
        if constexpr (KVDT == ROPEKV_FP8) {
          av = u32x4_t{fp8x2_bf16<false>(kp[2 * h]), fp8x2_bf16<true>(kp[2 * h]), fp8x2_bf16<false>(kp[2 * h + 1]),
                       fp8x2_bf16<true>(kp[2 * h + 1])};
        } else {
          float kf[8];
          codes4<KVDT>(kp[2 * h], kf);
          codes4<KVDT>(kp[2 * h + 1], kf + 4);
          av = u32x4_t{pack2_bf16(kf[0], kf[1]), pack2_bf16(kf[2], kf[3]), pack2_bf16(kf[4], kf[5]),
                       pack2_bf16(kf[6], kf[7])};
        }
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
    if constexpr (KVDT == ROPEKV_FP8) {
      // bytes (key 0, key 1) and (key 2, key 3) of dims e, e + 1 gathered into one word each, then
      // converted two at a time straight to bf16
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        const int w = e / 4;
        const uint32_t sel = (e % 4) ? 0x07030602u : 0x05010400u;
        const uint32_t p01 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], sel);
        const short4_t vb0 = __builtin_bit_cast(short4_t, (uint2){fp8x2_bf16<false>(p01), fp8x2_bf16<false>(p23)});
        const short4_t vb1 = __builtin_bit_cast(short4_t, (uint2){fp8x2_bf16<true>(p01), fp8x2_bf16<true>(p23)});
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb0, acc[e], 0, 0, 0);
        acc[e + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb1, acc[e + 1], 0, 0, 0);
      }
    } else {
      float vf[4][E];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int w = 0; w < E / 4; ++w) codes4<KVDT>(vw[j][w], vf[j] + 4 * w);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const short4_t vb = __builtin_bit_cast(
            short4_t, (uint2){pack2_bf16(vf[0][e], vf[1][e]), pack2_bf16(vf[2][e], vf[3][e])});
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[e], 0, 0, 0);
      }
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

constexpr int k8bitStages = 3;  // tile stages per wave (8-bit decode)

template <int D, int NREP, int KVDT>
hipError_t launch_split_8bit(const void *q, int batch, const ropekv_kv_cache &c, float sl2, float *ws,
                             const DecodePlan &pl, hipStream_t s) {
  dim3 grid(pl.splits, c.num_kv_heads, batch);
  if (c.layout == ROPEKV_PAGED)
    hipLaunchKernelGGL((decode_split_8bit_kernel<D, NREP, ROPEKV_PAGED, k8bitStages, KVDT>), grid, dim3(256), 0, s, q,
                       c, sl2, ws, pl.tiles_per_split, pl.splits);
  else
    hipLaunchKernelGGL((decode_split_8bit_kernel<D, NREP, ROPEKV_RING, k8bitStages, KVDT>), grid, dim3(256), 0, s, q,
                       c, sl2, ws, pl.tiles_per_split, pl.splits);
  return hipGetLastError();
}

template <int D, int NREP>
hipError_t launch_decode_8bit_t(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                                void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  hipError_t e = c.kv_dtype == ROPEKV_FP8 ? launch_split_8bit<D, NREP, ROPEKV_FP8>(q, batch, c, sl2, ws, pl, s)
                                          : launch_split_8bit<D, NREP, ROPEKV_I8>(q, batch, c, sl2, ws, pl, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<bf16_t, D, NREP>), dim3(c.num_kv_heads, batch), dim3(256), 0, s,
                     c, ws, sinks, out, pl.tiles_per_split, pl.splits);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_8bit_d(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sk,
                                void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  switch (pl.n_rep) {
    case 1: return launch_decode_8bit_t<D, 1>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 2: return launch_decode_8bit_t<D, 2>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 4: return launch_decode_8bit_t<D, 4>(q, batch, c, sl2, sk, out, ws, pl, s);
    case 8: return launch_decode_8bit_t<D, 8>(q, batch, c, sl2, sk, out, ws, pl, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_8bit(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                              void *out, float *ws, const DecodePlan &pl, hipStream_t s) {
  if (c.head_dim == 128) return launch_decode_8bit_d<128>(q, batch, c, sl2, sinks, out, ws, pl, s);
  if (c.head_dim == 64) return launch_decode_8bit_d<64>(q, batch, c, sl2, sinks, out, ws, pl, s);
  return hipErrorInvalidValue;
}

}  // namespace ropekv
