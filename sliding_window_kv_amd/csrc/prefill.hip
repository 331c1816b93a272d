// Prefill attention of one sequence's chunk over the sink + window mask.
//
// "Inference & 128K Long Context" (5.5: query t of the chunk sits at
// absolute position pos0 + t; a key j is allowed iff j <= pos0 + t and
// pos0 + t - j < window) with the sink rule of "Attention Sink 与 Streaming
// KV Cache" (keys j < S stay visible).  Key tiles no query of a workgroup can
// see are never loaded ("FlashAttention can skip invisible tiles").
//
// Workgroup: one KV head g and BM = 128 / n_rep consecutive chunk positions
// for all n_rep query heads of g (128 query rows, so every K/V byte staged in
// LDS serves all heads of the group).  Four waves, 32 rows each (two 16-row
// tiles of one head).  Key tiles of 64 keys, double-buffered in LDS: the next
// tile's global loads are in flight while the current one is computed.
//   S^T = K . Q^T   (MFMA; lane keeps its query row's 16 scores per tile)
//   online softmax in the log2 domain, fp32
//   O^T += V^T . P^T (MFMA; V stays row-major in LDS and the V^T operand is
//                     read with the gfx950 LDS transpose read; P rounded to bf16)
#include "kernels.hpp"

namespace ropekv {

namespace {

constexpr int kBN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int imod2(int x, int m) {
  int r = x % m;
  return r < 0 ? r + m : r;
}

struct PrefillArgs {
  const void *q, *k, *v;
  int T, pos0, n_q_heads, seq;
  ropekv_kv_cache c;
  float sl2;
  const float *sinks;  // optional learned sink logit per query head
  void *out;
};

// Element offset (into the chunk k/v when *chunk, else into the cache) of the
// key row at position j for KV head g; -1 when the row is not available.
__device__ inline long key_row(const PrefillArgs &a, int j, int g, int D, bool *chunk) {
  const ropekv_kv_cache &c = a.c;
  *chunk = false;
  if (j >= a.pos0) {
    if (j - a.pos0 >= a.T) return -1;
    *chunk = true;
    return ((long)(j - a.pos0) * c.num_kv_heads + g) * D;
  }
  if (c.layout == ROPEKV_PAGED) {
    const int blk = j / c.block_size;
    if (blk >= c.max_blocks) return -1;
    const int bid = c.block_table[(long)a.seq * c.max_blocks + blk];
    if (bid < 0 || bid >= c.num_blocks) return -1;
    return (((long)bid * c.num_kv_heads + g) * c.block_size + j % c.block_size) * D;
  }
  if (c.layout == ROPEKV_RING) {
    const long base = ((long)a.seq * c.num_kv_heads + g) * (long)c.capacity * D;
    if (j < c.sinks) return base + (long)j * D;
    const int n = c.seq_len[a.seq];
    const int cnt = c.ring_count[a.seq];
    if (j >= n || n - j > cnt) return -1;
    const int slot = c.sinks + imod2(c.ring_head[a.seq] - (n - j), c.window);
    return base + (long)slot * D;
  }
  return -1;
}

template <int NB>
__device__ __forceinline__ void copy16(void *dst, const void *src) {
#pragma unroll
  for (int i = 0; i < NB / 16; ++i) ((uint4 *)dst)[i] = ((const uint4 *)src)[i];
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 (round to nearest even, hardware conversion)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const float2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// LDS transpose read: within each 16-lane group, lane i receives element i % 4 of
// the 8 bytes addressed by lanes 4j + i / 4 (j = 0..3) of its group.
__device__ __forceinline__ uint2 lds_read_tr16(const void *p) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v *)(p));
  return __builtin_bit_cast(uint2, r);
}

template <typename T, int D, int NREP>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int EB = sizeof(T);
  constexpr int BM = 128 / NREP;           // chunk positions per workgroup
  constexpr int KP = kBF ? D + 8 : D + 4;  // K / V LDS row pitch in elements
  constexpr int QB = (D / 4) * EB;         // bytes of a quarter row
  constexpr int CH = QB;                   // bytes staged per thread per tile and tensor
  constexpr int TILE = kBN * KP;           // elements of one staged tile
  __shared__ __attribute__((aligned(16))) T k_lds[2][TILE];
  __shared__ __attribute__((aligned(16))) T v_lds[2][TILE];

  const ropekv_kv_cache &c = a.c;
  const int g = blockIdx.y;
  const int t0 = (gridDim.x - 1 - blockIdx.x) * BM;  // latest (longest) position blocks first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int Hq = a.n_q_heads;
  const int S = c.sinks, W = c.window;
  const int qp_lo = a.pos0 + t0;
  const int qp_hi = a.pos0 + min(t0 + BM, a.T) - 1;

  // this lane's query row in each of its two row tiles
  int tq[2], head[2];
  uint32_t qw[2][QB / 4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int R = 32 * wave + 16 * rt + col;
    tq[rt] = t0 + R % BM;
    head[rt] = g * NREP + R / BM;
    if (tq[rt] < a.T) {
      copy16<QB>(qw[rt], (const char *)a.q + (((long)tq[rt] * Hq + head[rt]) * D) * EB + grp * QB);
    } else {
#pragma unroll
      for (int i = 0; i < QB / 4; ++i) qw[rt][i] = 0u;
    }
  }

  // key tiles: sink tiles [0, nst), then recent tiles [first, last]
  const int last = qp_hi / kBN;
  int nst = 0, first = 0;
  if (W > 0) {
    const int sink_hi = min(S, qp_hi + 1);
    nst = (sink_hi + kBN - 1) / kBN;
    const int lo = max(0, qp_lo - W + 1);
    first = max(lo / kBN, nst);
  }
  const int ntiles = nst + max(0, last - first + 1);

  // staging: thread = (key, quarter of the row); K and V rows go to LDS unchanged
  const int skey = tid >> 2, sq = tid & 3;
  bool lost = false;
  uint32_t kreg[CH / 4], vreg[CH / 4];
  auto fetch = [&](int kt) {
    const int kb = kt < nst ? kt : first + (kt - nst);
    const int j = kb * kBN + skey;
    bool chunk;
    const long off = key_row(a, j, g, D, &chunk);
    const bool needed = j <= qp_hi && (W == 0 || j < S || j > qp_lo - W);
    if (off < 0 && needed && j < a.pos0) lost = true;
    if (off >= 0) {
      copy16<CH>(kreg, (const char *)(chunk ? a.k : c.k) + off * EB + sq * CH);
      copy16<CH>(vreg, (const char *)(chunk ? a.v : c.v) + off * EB + sq * CH);
    } else {
#pragma unroll
      for (int i = 0; i < CH / 4; ++i) kreg[i] = vreg[i] = 0u;
    }
  };
  auto stash = [&](int buf) {
    copy16<CH>(&k_lds[buf][skey * KP + sq * (D / 4)], kreg);
    copy16<CH>(&v_lds[buf][skey * KP + sq * (D / 4)], vreg);
  };

  float m_run[2] = {kNegBig, kNegBig}, l_run[2] = {0.f, 0.f};
  f32x4 o[2][D / 16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) o[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) fetch(kt + 1);  // in flight while this tile is computed
    const T *kl = k_lds[buf];
    const T *vl = v_lds[buf];
    const int kb = kt < nst ? kt : first + (kt - nst);
    const int j0 = kb * kBN;

    // ---- scores S^T = K Q^T (raw dot products)
    f32x4 sc[2][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint32_t kw[QB / 4];
      copy16<QB>(kw, &kl[(16 * st + col) * KP + grp * (D / 4)]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kBF) {
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 av = {kw[4 * t], kw[4 * t + 1], kw[4 * t + 2], kw[4 * t + 3]};
            const u32x4 bv = {qw[rt][4 * t], qw[rt][4 * t + 1], qw[rt][4 * t + 2], qw[rt][4 * t + 3]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int t = 0; t < D / 4; ++t)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[t]), __uint_as_float(qw[rt][t]), acc, 0,
                                                       0, 0);
        }
        sc[rt][st] = acc;
      }
    }
    // does every query of this workgroup see every key of the tile?
    const int jmax = j0 + kBN - 1;
    const bool full = jmax <= qp_lo && (W == 0 || jmax < S || qp_hi - j0 < W);
    bool moved = false;
    float corr[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (!full) {
        const int qpos = a.pos0 + tq[rt];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int jp = j0 + 16 * st + 4 * grp + j;
            const bool vis = jp <= qpos && (W == 0 || jp < S || qpos - jp < W);
            sc[rt][st][j] = vis ? sc[rt][st][j] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[rt][st][j]);
      mx = wave_max_xor(mx, 16);
      mx = wave_max_xor(mx, 32);
      const float m_new = fmaxf(m_run[rt], mx * a.sl2);  // sl2 > 0: the max commutes with the scale
      corr[rt] = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
      moved |= m_new != m_run[rt];
      float ps = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[rt][st][j], a.sl2, -m_new));
          sc[rt][st][j] = p;
          ps += p;
        }
      l_run[rt] = l_run[rt] * corr[rt] + ps;
      m_run[rt] = m_new;
    }
    // rows whose max did not move keep their accumulators as they are
    if (__any(moved)) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) o[rt][mt] *= corr[rt];
    }

    // ---- O^T += V^T P^T
    if constexpr (kBF) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t pw[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x4 pp = sc[rt][2 * u + h2];
            pw[rt][2 * h2] = pack_bf16(pp[0], pp[1]);
            pw[rt][2 * h2 + 1] = pack_bf16(pp[2], pp[3]);
          }
        // lane (grp, src = col) points at V[32u + 4grp + src/4 (+16)][16 mt + 4 (src % 4)]
        const int vrow = 32 * u + 4 * grp + (col >> 2);
        const int vcol = 4 * (col & 3);
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
          const uint2 lo = lds_read_tr16(&vl[vrow * KP + 16 * mt + vcol]);
          const uint2 hi = lds_read_tr16(&vl[(vrow + 16) * KP + 16 * mt + vcol]);
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const u32x4 bv = {pw[rt][0], pw[rt][1], pw[rt][2], pw[rt][3]};
            o[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                __builtin_bit_cast(bf16x8, bv), o[rt][mt], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float vv = ((const float *)vl)[(16 * st + 4 * grp + j) * KP + 16 * mt + col];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
              o[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, sc[rt][st][j], o[rt][mt], 0, 0, 0);
          }
    }
    if (kt + 1 < ntiles) stash(buf ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
  }
  if (lost) dev_error(c.err_word, ROPEKV_DEV_PREFIX_LOST);

  // ---- normalise and store: lane holds O^T[16 mt + 4 grp + j][its row]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.sinks) {
      // learned sink logit in the normaliser: rescale to max(m, sink) and add its weight
      const float sink2 = a.sinks[head[rt]] * kLog2e;
      const float m_f = fmaxf(m_run[rt], sink2);
      const float f = __builtin_amdgcn_exp2f(m_run[rt] - m_f);
      const float lt = l * f + __builtin_amdgcn_exp2f(sink2 - m_f);
      inv = lt > 0.f ? f / lt : 0.f;
    }
    if (tq[rt] < a.T) {
      const long ob = ((long)tq[rt] * Hq + head[rt]) * D;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const int d0 = 16 * mt + 4 * grp;
        if constexpr (kBF) {
          uint2 w;
          w.x = pack_bf16(o[rt][mt][0] * inv, o[rt][mt][1] * inv);
          w.y = pack_bf16(o[rt][mt][2] * inv, o[rt][mt][3] * inv);
          *(uint2 *)((uint16_t *)a.out + ob + d0) = w;
        } else {
          *(float4 *)((float *)a.out + ob + d0) =
              make_float4(o[rt][mt][0] * inv, o[rt][mt][1] * inv, o[rt][mt][2] * inv, o[rt][mt][3] * inv);
        }
      }
    }
  }
}

// ---- bf16: tiles staged by direct global -> LDS loads into swizzled rows ----
//
// Same workgroup and tile walk as above.  K and V tiles are copied into LDS
// with direct loads (no staging registers, the next tile in flight while the
// current one is computed) in rows of D / 8 16-byte chunks, chunk c of row r
// stored at c ^ kswz(r) (K) or c ^ vswz(r) (V).  The 32 lanes of a transposing
// V read (8 rows x 4 column groups) hit 32 different 8-byte bank slots and
// time as fast as linear reads.  The K swizzle gives the 16 lanes reading one
// chunk column 16 different 16-byte bank groups, yet on gfx950 those 16-byte
// reads still meet two-way bank conflicts (the lane grouping of such reads is
// not documented; counters show half of the K read cycles as conflicts).  A
// conflict-free order exists (bit reversal of r mod 16, found by timing XOR
// patterns) but ran this kernel 2 % slower, as LDS bandwidth is not what
// bounds it, so the simpler swizzle stays.
//
// The running maximum is raised only when a tile's maximum exceeds it by more
// than kLazy (log2 units): in between, p = exp2(s - m) stays below 2^kLazy,
// which fp32 sums and bf16 P hold exactly as well, and the output accumulators
// are rescaled only on those (rare) raises.
constexpr float kLazy = 8.0f;

template <int D>
__device__ __forceinline__ int kswz(int row) {
  constexpr int CPR = D / 8;
  return (row * CPR / 16) % CPR;
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  constexpr int CPR = D / 8;
  return ((row * CPR / 16) & (CPR / 2 - 1)) << 1;
}

template <int D, int NREP>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BM = 128 / NREP;      // chunk positions per workgroup
  constexpr int CPR = D / 8;          // 16-byte chunks per K / V row
  constexpr int QC = D / 32;          // chunks of a lane's quarter row = MFMA k-steps
  constexpr int TB = kBN * D * 2;     // bytes of one staged tile
  constexpr int NI = TB / 4096;       // direct loads per thread per tile and tensor
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2][TB];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[2][TB];

  const ropekv_kv_cache &c = a.c;
  // consecutive workgroups (which the dispatcher spreads over the XCDs round-robin) take
  // consecutive KV heads, so each XCD walks one head's positions in order and the K / V
  // tiles its workgroups share stay in that XCD's L2
  const int bid = blockIdx.x + blockIdx.y * gridDim.x;
  const int g = bid % c.num_kv_heads;
  // position blocks in decreasing order: under a causal mask the late positions see the most
  // keys, and starting the longest workgroups first packs the grid's tail (-3 % on the
  // 8192-token chunk)
  const int t0 = (gridDim.x * gridDim.y / c.num_kv_heads - 1 - bid / c.num_kv_heads) * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int Hq = a.n_q_heads;
  const int S = c.sinks, W = c.window;
  const int qp_lo = a.pos0 + t0;
  const int qp_hi = a.pos0 + min(t0 + BM, a.T) - 1;

  // this lane's query row in each of its two row tiles; chunk grp * QC + t of the row
  int tq[2], head[2];
  u32x4 qv[2][QC];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int R = 32 * wave + 16 * rt + col;
    tq[rt] = t0 + R % BM;
    head[rt] = g * NREP + R / BM;
    const char *qrow = (const char *)a.q + ((long)tq[rt] * Hq + head[rt]) * D * 2;
#pragma unroll
    for (int t = 0; t < QC; ++t)
      qv[rt][t] = tq[rt] < a.T ? *(const u32x4 *)(qrow + (grp * QC + t) * 16) : u32x4{0u, 0u, 0u, 0u};
  }

  // key tiles: sink tiles [0, nst), then recent tiles [first, last]
  const int last = qp_hi / kBN;
  int nst = 0, first = 0;
  if (W > 0) {
    const int sink_hi = min(S, qp_hi + 1);
    nst = (sink_hi + kBN - 1) / kBN;
    const int lo = max(0, qp_lo - W + 1);
    first = max(lo / kBN, nst);
  }
  const int ntiles = nst + max(0, last - first + 1);

  // Direct loads of one tile: instruction n of wave w fills chunk slots 64 (4 n + w) + lane,
  // i.e. row r = slot / CPR, stored chunk slot % CPR (= logical chunk ^ swizzle of r).
  int row_n[NI], kch_n[NI], vch_n[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int p = 64 * (4 * n + wave) + lane;
    row_n[n] = p / CPR;
    kch_n[n] = ((p % CPR) ^ kswz<D>(row_n[n])) * 16;
    vch_n[n] = ((p % CPR) ^ vswz<D>(row_n[n])) * 16;
  }
  const long chunk_row_bytes = (long)c.num_kv_heads * D * 2;  // one position of the chunk's k / v
  // per-lane byte offsets of the direct loads within a tile of the chunk's k / v (fast path)
  uint32_t koff_n[NI], voff_n[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    koff_n[n] = (uint32_t)(row_n[n] * chunk_row_bytes + kch_n[n]);
    voff_n[n] = (uint32_t)(row_n[n] * chunk_row_bytes + vch_n[n]);
  }
  bool lost = false;
  auto issue = [&](int kt, int buf) {
    const int kb = kt < nst ? kt : first + (kt - nst);
    const int j0 = kb * kBN;
    if (j0 >= a.pos0 && j0 + kBN <= a.pos0 + a.T) {
      // every key of the tile is in the chunk: rows are (j - pos0, g) of k and v
      const long tb = (long)(j0 - a.pos0) * chunk_row_bytes + (long)g * D * 2;
      const char *kt = (const char *)a.k + tb;  // wave-uniform tile bases
      const char *vt = (const char *)a.v + tb;
#pragma unroll
      for (int n = 0; n < NI; ++n) dma16_so(kt, koff_n[n], &k_lds[buf][(4 * n + wave) * 1024]);
#pragma unroll
      for (int n = 0; n < NI; ++n) dma16_so(vt, voff_n[n], &v_lds[buf][(4 * n + wave) * 1024]);
      return;
    }
    const char *ksrc[NI];
    const char *vsrc[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int j = j0 + row_n[n];
      bool chunk;
      long off = key_row(a, j, g, D, &chunk);
      const bool needed = j <= qp_hi && (W == 0 || j < S || j > qp_lo - W);
      if (off < 0 && needed && j < a.pos0) lost = true;
      if (off < 0) {  // beyond the chunk (never visible) or a lost prefix key (flagged): an in-bounds row
        off = (long)g * D;
        chunk = true;
      }
      ksrc[n] = (const char *)(chunk ? a.k : c.k) + off * 2 + kch_n[n];
      vsrc[n] = (const char *)(chunk ? a.v : c.v) + off * 2 + vch_n[n];
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) dma16(ksrc[n], &k_lds[buf][(4 * n + wave) * 1024]);
#pragma unroll
    for (int n = 0; n < NI; ++n) dma16(vsrc[n], &v_lds[buf][(4 * n + wave) * 1024]);
  };

  // byte offsets of this lane's transposing V reads, block mt of rows 4 grp + col / 4 (+16, +32:
  // the same swizzle, so those are immediates): chunk (2 mt + (col % 4) / 2) ^ swizzle
  int voff[D / 16];
  {
    const int vrow = 4 * grp + (col >> 2);
    const int vx = vswz<D>(vrow);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      voff[mt] = (vrow * CPR + ((2 * mt + ((col & 3) >> 1)) ^ vx)) * 16 + (col & 1) * 8;
  }
  float m_run[2] = {kNegBig, kNegBig};
  f32x4 o[2][D / 16];
  // row sums of P on the MFMA: a block of ones as the A operand gives sum_k P[k][row] in every
  // element of lsum (the same bf16 P as the numerator)
  f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const short8 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80};
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) o[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) issue(0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  // unrolled by two so that the buffer (kt & 1) is a constant in each copy and the
  // buffer offsets become instruction immediates
#pragma unroll 2
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) issue(kt + 1, buf ^ 1);  // in flight while this tile is computed
    const uint8_t *kl = k_lds[buf];
    const uint8_t *vl = v_lds[buf];
    const int kb = kt < nst ? kt : first + (kt - nst);
    const int j0 = kb * kBN;

    __builtin_amdgcn_s_setprio(1);
    // ---- scores S^T = K Q^T (raw dot products); two key sub-tiles at a time, four
    // independent accumulation chains
    f32x4 sc[2][4];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      u32x4 kf[2][QC];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int row = 16 * (2 * sp + s2) + col;
#pragma unroll
        for (int t = 0; t < QC; ++t)
          kf[s2][t] = *(const u32x4 *)(kl + (row * CPR + ((grp * QC + t) ^ kswz<D>(row))) * 16);
      }
      f32x4 acc[2][2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[s2][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < QC; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
            acc[s2][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[s2][t]),
                                                                  __builtin_bit_cast(bf16x8, qv[rt][t]), acc[s2][rt],
                                                                  0, 0, 0);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) sc[rt][2 * sp + s2] = acc[s2][rt];
    }
    __builtin_amdgcn_s_setprio(0);
    // does every query of this workgroup see every key of the tile?
    const int jmax = j0 + kBN - 1;
    const bool full = jmax <= qp_lo && (W == 0 || jmax < S || qp_hi - j0 < W);
    bool raised = false;
    float corr[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      if (!full) {
        const int qpos = a.pos0 + tq[rt];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int jp = j0 + 16 * st + 4 * grp + j;
            const bool vis = jp <= qpos && (W == 0 || jp < S || qpos - jp < W);
            sc[rt][st][j] = vis ? sc[rt][st][j] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[rt][st][j]);
      mx = max_xor32(max_xor16(mx));
      const float m_tile = mx * a.sl2;  // sl2 > 0: the max commutes with the scale; -inf if all masked
      corr[rt] = 1.f;
      if (m_tile > m_run[rt] + kLazy) {
        corr[rt] = __builtin_amdgcn_exp2f(m_run[rt] - m_tile);
        m_run[rt] = m_tile;
        raised = true;
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[rt][st][j] = __builtin_amdgcn_exp2f(fmaf(sc[rt][st][j], a.sl2, -m_run[rt]));
    }
    if (__any(raised)) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) o[rt][mt] *= corr[rt];
        lsum[rt] *= corr[rt];
      }
    }

    __builtin_amdgcn_s_setprio(1);  // MFMA phases at raised priority: the SIMD keeps issuing them
    // ---- O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4 pb[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const f32x4 p0 = sc[rt][2 * u], p1 = sc[rt][2 * u + 1];
        pb[rt] = u32x4{pack_bf16(p0[0], p0[1]), pack_bf16(p0[2], p0[3]), pack_bf16(p1[0], p1[1]),
                       pack_bf16(p1[2], p1[3])};
        lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones),
                                                           __builtin_bit_cast(bf16x8, pb[rt]), lsum[rt], 0, 0, 0);
      }
      // lane (grp, col) addresses V[32u + 4grp + col/4 (+16)][16 mt + 4 (col % 4)]
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        typedef __attribute__((address_space(3))) short4v lds_s4;
        const uint8_t *vp = vl + voff[mt] + 32 * u * CPR * 16;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)vp);
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vp + 16 * CPR * 16));
        const short8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          o[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                              __builtin_bit_cast(bf16x8, pb[rt]), o[rt][mt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();  // this wave's loads of the next tile have landed
    __syncthreads();  // ... and everyone's; this tile's buffers may be refilled
  }
  if (lost) dev_error(c.err_word, ROPEKV_DEV_PREFIX_LOST);

  // ---- normalise and store: lane holds O^T[16 mt + 4 grp + j][its row]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float l = lsum[rt][0];
    float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.sinks) {
      const float sink2 = a.sinks[head[rt]] * kLog2e;
      const float m_f = fmaxf(m_run[rt], sink2);
      const float f = __builtin_amdgcn_exp2f(m_run[rt] - m_f);
      const float lt = l * f + __builtin_amdgcn_exp2f(sink2 - m_f);
      inv = lt > 0.f ? f / lt : 0.f;
    }
    if (tq[rt] < a.T) {
      const long ob = ((long)tq[rt] * Hq + head[rt]) * D;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        const int d0 = 16 * mt + 4 * grp;
        uint2 w;
        w.x = pack_bf16(o[rt][mt][0] * inv, o[rt][mt][1] * inv);
        w.y = pack_bf16(o[rt][mt][2] * inv, o[rt][mt][3] * inv);
        *(uint2 *)((uint16_t *)a.out + ob + d0) = w;
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_prefill_d(const PrefillArgs &a, int n_rep, hipStream_t s) {
  const int bm = 128 / n_rep;
  dim3 grid((a.T + bm - 1) / bm, a.c.num_kv_heads);
  if constexpr (sizeof(T) == 2) {
    switch (n_rep) {
      case 1: hipLaunchKernelGGL((prefill_bf16_kernel<D, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((prefill_bf16_kernel<D, 2>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((prefill_bf16_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
      case 8: hipLaunchKernelGGL((prefill_bf16_kernel<D, 8>), grid, dim3(256), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (n_rep) {
      case 1: hipLaunchKernelGGL((prefill_kernel<T, D, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((prefill_kernel<T, D, 2>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((prefill_kernel<T, D, 4>), grid, dim3(256), 0, s, a); break;
      case 8: hipLaunchKernelGGL((prefill_kernel<T, D, 8>), grid, dim3(256), 0, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const void *q, const void *k, const void *v, int T, int pos0, int n_q_heads,
                          const ropekv_kv_cache &c, int seq_id, float scale, const float *sink_logits, void *out,
                          hipStream_t s) {
  PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.T = T;
  a.pos0 = pos0;
  a.n_q_heads = n_q_heads;
  a.seq = seq_id;
  a.c = c;
  a.sl2 = scale * kLog2e;
  a.sinks = sink_logits;
  a.out = out;
  const int n_rep = n_q_heads / c.num_kv_heads;
  if (c.kv_dtype == ROPEKV_BF16) {
    if (c.head_dim == 128) return launch_prefill_d<bf16_t, 128>(a, n_rep, s);
    if (c.head_dim == 64) return launch_prefill_d<bf16_t, 64>(a, n_rep, s);
  } else if (c.kv_dtype == ROPEKV_F32) {
    if (c.head_dim == 128) return launch_prefill_d<float, 128>(a, n_rep, s);
    if (c.head_dim == 64) return launch_prefill_d<float, 64>(a, n_rep, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ropekv
