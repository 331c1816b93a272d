// Re-rotation of cached keys at a YaRN factor switch.
//
// "#2961 rope: --rope-scaling dynamic" ("What it does": the cached keys
// follow a change) and "Attention Sink 与 Streaming KV Cache" (R_a R_b =
// R_{a+b}): a key stored as mu_A R(p w_A) k becomes mu_B R(p w_B) k after one
// more rotation of pair i by p (w_B,i - w_A,i) and a gain mu_B / mu_A.
//
// A workgroup owns PT consecutive positions and walks every layer and KV
// head at those positions, so the fp64 angle work (PT x r/2 sincos) is shared
// by n_layers x Hkv rows; the per-pair frequency change w_B,i - w_A,i and the
// gain are evaluated once per call on the host, in fp64.  Float caches read and
// write only the rotary slice (the tail is never touched); int8 rows are read
// whole, turned in code units and requantised with a fresh per-row scale.
#include "kernels.hpp"

namespace ropekv {

namespace {

constexpr int kPT = 16;  // positions per workgroup
constexpr int kI8Threads = 256;  // int8 lane kernel: threads per workgroup
constexpr int kI8Layers = 2;     // int8 lane kernel: layers per workgroup (1: 16.4 ms, 2: 14.4, 4: 15.3 on the
                                 // 64-layer int8 switch; the float kernel is fastest at 1)
constexpr int kHadLayers = 4;    // Hadamard head_dim-128 kernels: layers per workgroup (r 64: 1: 16.2 ms, 2: 15.7, 4: 15.2, 8: 15.1)
// layers per workgroup of the staged NeoX r = 64 Hadamard kernel (64-layer switch: 2 layers ran
// 12.6 ms on one box and 14.2 on another, against 13.0 and 13.5 for 8; 4: 13.6)
constexpr int kHadNeoxLayers = 8;

struct RerotArgs {
  RopeParams from, to;
  void *k;
  float *scale;
  int rows_T;  // rows (positions) per layer
  int Hkv, D, pos0, n_layers;
  int keep_scale;  // int8: keep each row's scale unless a turned rotary code overflows
  int rpb;         // chunked kernels: rows per workgroup
  int chunks;      // chunked kernels: row chunks per layer
  int lg;          // chunked kernels: layers per workgroup
  double gain;     // mu_to / mu_from
  double dw[256];  // w_to,i - w_from,i per rotary pair, fp64, set on the host
};

// Chunked workgroups: each owns rpb consecutive rows (position-major, head-minor)
// of lg consecutive layers, and the grid runs chunk-major within a layer group,
// so the whole chip sweeps the cache front to back.  A thread reads its piece of
// a row, turns it and writes it back right away: on this part an in-place stream
// runs fastest that way (a probe with one read-modify-write per thread in 4 KiB
// workgroups moved 5.9 TB/s, against 4.7-5.1 TB/s when each workgroup walks many
// pieces or many layers).
struct ChunkRows {
  long row0;  // first row of the workgroup in its first layer (all layers counted)
  int nl;     // layers the workgroup walks
  int r0;     // first row within its layer
  int nrows;  // live rows
  int pa;     // position index (from pos0) of the first row
  int np;     // positions the rows span
};
__device__ inline ChunkRows chunk_rows(const RerotArgs &a) {
  const int group = blockIdx.x / a.chunks, chunk = blockIdx.x - group * a.chunks;
  const int layer = group * a.lg;
  const long layer_rows = (long)a.rows_T * a.Hkv;
  const int r0 = chunk * a.rpb;
  ChunkRows c;
  c.nrows = (int)min((long)a.rpb, layer_rows - r0);
  c.row0 = layer * layer_rows + r0;
  c.nl = min(a.lg, a.n_layers - layer);
  c.r0 = r0;
  c.pa = r0 / a.Hkv;
  c.np = (r0 + c.nrows - 1) / a.Hkv - c.pa + 1;
  return c;
}

// cos / sin of the turn of every rotary pair at positions pos0 + pa .. + np - 1,
// times the gain, into s_cs / s_sn [np][half].  The angle p (w_to,i - w_from,i)
// and its reduction modulo 2 pi are fp64; cos and sin of the reduced angle
// (|r| <= pi) are fp32, within a few 1e-7 of the exact values.
__device__ inline void turn_table(const RerotArgs &a, int pa, int np, float *s_cs, float *s_sn) {
  const int half = a.to.rotary_dim / 2;
  const float gain = (float)a.gain;
  for (int idx = threadIdx.x; idx < np * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx - pt * half;
    const double th = (double)(a.pos0 + pa + pt) * a.dw[i];
    const double k = rint(th * 0.15915494309189535);                  // turns of 2 pi
    const double rd = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, th));
    float sf, cf;
    sincosf((float)rd, &sf, &cf);
    s_cs[idx] = cf * gain;
    s_sn[idx] = sf * gain;
  }
  __syncthreads();
}

// As turn_table, with the frequency change w_to,i - w_from,i of this thread's pair i =
// threadIdx.x % half read by the caller up front (own_dw): the change sits in the kernel
// arguments and is read with a vector load, which the caller issues before its own global
// loads, so that waiting for it does not also wait for those.  When the workgroup size is a
// multiple of half, every entry a thread computes has that pair; otherwise later entries read
// their own change.
__device__ __forceinline__ double own_dw(const RerotArgs &a) {
  return a.dw[threadIdx.x % (a.to.rotary_dim / 2)];
}
__device__ inline void turn_table_w(const RerotArgs &a, int pa, int np, float *s_cs, float *s_sn, double dwt,
                                    float *s_nsn = nullptr) {
  const int half = a.to.rotary_dim / 2;
  const float gain = (float)a.gain;
  const bool same_pair = blockDim.x % half == 0;
  for (int idx = threadIdx.x; idx < np * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx - pt * half;
    const double th = (double)(a.pos0 + pa + pt) * (same_pair || idx == (int)threadIdx.x ? dwt : a.dw[i]);
    const double k = rint(th * 0.15915494309189535);                  // turns of 2 pi
    const double rd = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, th));
    float sf, cf;
    sincosf((float)rd, &sf, &cf);
    s_cs[idx] = cf * gain;
    s_sn[idx] = sf * gain;
    if (s_nsn) s_nsn[idx] = -(sf * gain);
  }
  // the table is LDS-only: wait for this wave's LDS writes, then the workgroup barrier, without
  // the wait on outstanding global loads a __syncthreads() fence would add (the memory clobber
  // keeps the compiler from moving the table's reads above the barrier)
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Keep-scale decision for one int8 row: every turned rotary value of the row must
// re-code within [-127, 127] at the row's old scale (decided like the quantiser, in
// fp32 with the reciprocal of the scale).  `mx` is this lane's largest such code,
// `lanes` the row's lane count (a power of two, lanes of a row adjacent).
__device__ __forceinline__ bool row_keeps_scale(float mx, int lanes) {
  for (int m = lanes >> 1; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
  return mx <= 127.f;
}

// Fills s_cs / s_sn [kPT][half] with cos / sin of (pos) * (w_to - w_from) in
// fp64, rounded to fp32, and returns the gain mu_to / mu_from.
__device__ inline float angle_setup(const RerotArgs &a, int t0, float *s_cs, float *s_sn) {
  const int half = a.to.rotary_dim / 2;
  for (int idx = threadIdx.x; idx < kPT * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx % half;
    const double ang = (double)(a.pos0 + t0 + pt) * a.dw[i];
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cs[idx] = (float)cs;
    s_sn[idx] = (float)sn;
  }
  __syncthreads();
  return (float)a.gain;
}

// Raw 16-bit / 32-bit element access inside a register vector.
template <typename T>
__device__ __forceinline__ float vget(const uint32_t *w, int e) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(w[e]);
  } else {
    const uint16_t h = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    return sizeof(T) == 2 && __is_same(T, bf16_t) ? bf16_to_f(h) : f16_to_f(h);
  }
}
template <typename T>
__device__ __forceinline__ void vput(uint32_t *w, int e, float v) {
  if constexpr (sizeof(T) == 4) {
    w[e] = __float_as_uint(v);
  } else {
    const uint32_t h = __is_same(T, bf16_t) ? f_to_bf16(v) : f_to_f16(v);
    w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xffffu) | (h << 16)) : ((w[e >> 1] & 0xffff0000u) | h);
  }
}
// elements e and e + 1 (e even) in one go: one packed conversion for 16-bit types
template <typename T>
__device__ __forceinline__ void vput2(uint32_t *w, int e, float v0, float v1) {
  if constexpr (sizeof(T) == 4) {
    w[e] = __float_as_uint(v0);
    w[e + 1] = __float_as_uint(v1);
  } else if constexpr (__is_same(T, bf16_t)) {
    w[e >> 1] = pack2_bf16_rne(v0, v1);
  } else {
    w[e >> 1] = pack2_f16_rne(v0, v1);
  }
}

template <int NB>
__device__ __forceinline__ void vld(uint32_t *w, const char *p) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 v = ((const uint4 *)p)[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (NB == 4) {
    w[0] = *(const uint32_t *)p;
  } else {
    w[0] = *(const uint16_t *)p;
  }
}
template <int NB>
__device__ __forceinline__ void vst(char *p, const uint32_t *w) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) ((uint4 *)p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (NB == 4) {
    *(uint32_t *)p = w[0];
  } else {
    *(uint16_t *)p = (uint16_t)w[0];
  }
}

// Float keys.  A thread turns PP consecutive pairs of one row: NeoX reads PP
// elements from each half, GPT-J 2 PP interleaved elements; tpr = half / PP
// threads per row, rpb = 256 / tpr rows per one-shot workgroup.
template <typename T, int PP>
__global__ __launch_bounds__(256) void rerotate_float_kernel(RerotArgs a) {
  constexpr int EB = sizeof(T);
  constexpr int NB = PP * EB;
  constexpr int NW = (NB + 3) / 4;
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const ChunkRows c = chunk_rows(a);
  float *s_cs = s_tab, *s_sn = s_tab + c.np * half;
  turn_table(a, c.pa, c.np, s_cs, s_sn);
  const int tpr = half / PP;
  const int rr = threadIdx.x / tpr, q = threadIdx.x - rr * tpr;
  if (rr >= c.nrows) return;
  const int j0 = q * PP;
  const int tab = ((c.r0 + rr) / a.Hkv - c.pa) * half + j0;
  const long layer_bytes = (long)a.rows_T * a.Hkv * a.D * EB;
  char *kb = (char *)a.k + (c.row0 + rr) * a.D * EB;
  char *p1 = kb + (a.to.neox ? j0 : 2 * j0) * EB;
  char *p2 = a.to.neox ? kb + (half + j0) * EB : p1 + NB;
  for (int l = 0; l < c.nl; ++l, p1 += layer_bytes, p2 += layer_bytes) {
  uint32_t w1[NW], w2[NW];
  vld<NB>(w1, p1);
  vld<NB>(w2, p2);
  const float *cs = &s_cs[tab];
  const float *sn = &s_sn[tab];
  if constexpr (PP % 2 == 0) {
    if (a.to.neox) {
#pragma unroll
      for (int e = 0; e < PP; e += 2) {
        const float x1a = vget<T>(w1, e), x2a = vget<T>(w2, e);
        const float x1b = vget<T>(w1, e + 1), x2b = vget<T>(w2, e + 1);
        vput2<T>(w1, e, x1a * cs[e] - x2a * sn[e], x1b * cs[e + 1] - x2b * sn[e + 1]);
        vput2<T>(w2, e, x2a * cs[e] + x1a * sn[e], x2b * cs[e + 1] + x1b * sn[e + 1]);
      }
    } else {
      // 2 PP interleaved elements: pair e is (2e, 2e+1), both in one NB-byte half
#pragma unroll
      for (int e = 0; e < PP; ++e) {
        uint32_t *b = 2 * e < PP ? w1 : w2;
        const int i1 = 2 * e < PP ? 2 * e : 2 * e - PP;
        const float x1 = vget<T>(b, i1), x2 = vget<T>(b, i1 + 1);
        vput2<T>(b, i1, x1 * cs[e] - x2 * sn[e], x2 * cs[e] + x1 * sn[e]);
      }
    }
  } else {
    // PP = 1: the pair is element 0 of each half (NeoX) or of the two halves (GPT-J)
    const float x1 = vget<T>(w1, 0), x2 = vget<T>(w2, 0);
    vput<T>(w1, 0, x1 * cs[0] - x2 * sn[0]);
    vput<T>(w2, 0, x2 * cs[0] + x1 * sn[0]);
  }
  vst<NB>(p1, w1);
  vst<NB>(p2, w2);
  }
}

// int8 keys with a per-row fp32 scale, L = D / 16 lanes per row, 16 codes per
// lane: NeoX lane q holds pairs [qH, qH + H) (H codes from each half) and
// TL = 16 - 2H tail codes [r + q TL, ...); GPT-J lane q holds the 2H
// interleaved codes of the same pairs.  No lane exchange is needed to turn a
// pair; the row's absmax is a reduction over its L lanes.  Codes are
// requantised as rne(y * (127 / max|y|)), the reciprocal correctly rounded.
template <int N>
__device__ __forceinline__ void ld_n(uint32_t *w, const int8_t *p) {
  if constexpr (N == 16) {
    const uint4 v = *(const uint4 *)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 12) {
    const uint3 v = *(const uint3 *)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (N == 8) {
    const uint2 v = *(const uint2 *)p;
    w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 4) {
    w[0] = *(const uint32_t *)p;
  } else if constexpr (N == 2) {
    w[0] = *(const uint16_t *)p;
  }
}
template <int N>
__device__ __forceinline__ void st_n(int8_t *p, const uint32_t *w) {
  if constexpr (N == 16) {
    *(uint4 *)p = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (N == 12) {
    *(uint3 *)p = make_uint3(w[0], w[1], w[2]);
  } else if constexpr (N == 8) {
    *(uint2 *)p = make_uint2(w[0], w[1]);
  } else if constexpr (N == 4) {
    *(uint32_t *)p = w[0];
  } else if constexpr (N == 2) {
    *(uint16_t *)p = (uint16_t)w[0];
  }
}
// code byte e of a word array -> float (the byte is a signed int8)
// rne(v * inv) as an int8 code in the low byte: the fp32 product, then adding 1.5 * 2^23
// rounds it to an integer (nearest even) held in the low mantissa bits.  Callers keep
// |v * inv| <= 127.5 (inv = 127 / row max, or a kept scale that passed the overflow
// test), so the code needs no clamp.
__device__ __forceinline__ uint32_t code_bits(float v, float inv) {
  return __float_as_uint(__fmul_rn(v, inv) + 12582912.0f);
}
// the low bytes of a, b, c, d -> one word (a in the low byte)
__device__ __forceinline__ uint32_t pack4_codes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
// n codes (n a multiple of 2, up to 16) -> n / 4 words (the last one half filled when n % 4 == 2)
template <int N>
__device__ __forceinline__ void pack_codes(uint32_t *w, const uint32_t *cb) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) w[i] = pack4_codes(cb[4 * i], cb[4 * i + 1], cb[4 * i + 2], cb[4 * i + 3]);
  if constexpr (N % 4 == 2) w[N / 4] = __builtin_amdgcn_perm(cb[N - 1], cb[N - 2], 0x0c0c0400u);
}

__device__ __forceinline__ float code_at(const uint32_t *w, int e) {
  return (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
}

// Turn table of one block in code units: cos and sin of pos (w_to - w_from), times
// the gain mu_to / mu_from, in fp64 and rounded once to fp32.  [kPT][half] each,
// in dynamic LDS (kPT x half x 8 bytes).
__device__ inline void gain_table(const RerotArgs &a, int t0, float *s_cs, float *s_sn) {
  const int half = a.to.rotary_dim / 2;
  for (int idx = threadIdx.x; idx < kPT * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx - pt * half;
    double sn, cs;
    sincos((double)(a.pos0 + t0 + pt) * a.dw[i], &sn, &cs);
    s_cs[idx] = (float)(cs * a.gain);
    s_sn[idx] = (float)(sn * a.gain);
  }
  __syncthreads();
}

// int8 keys turned in code units.  A row x = c * sc (codes c, row scale sc) turns
// into y * sc with y = R c (the pair turn with the gain folded into cos / sin),
// so the requantised row needs only the codes: amax = max|y| over the row (tail
// codes included), new codes rne(y * (127 / amax)) with 127 / amax correctly
// rounded and the product rounded once, new scale sc * (amax / 127) (a row that
// does not move keeps its codes and scale bit for bit).
// Keep-scale: the row keeps sc (tail codes untouched) when every turned rotary
// value re-codes within [-127, 127], i.e. max|y| < 127.5, and stores rne(y).
// A row with sc = 0 becomes all zero with scale 0, as its dequantised values are.
// Codes are rne(y * inv) by one fma with 1.5 * 2^23 (the integer lands in the
// low mantissa bits); |y * inv| <= 127.5 holds by the choice of inv.
__device__ __forceinline__ uint32_t code_fma(float y, float inv) {
  return __float_as_uint(__builtin_fmaf(y, inv, 12582912.0f));
}

// Lane-local pairs: L = D / 16 lanes per row, 16 codes per lane; NeoX lane q
// holds pairs [qH, qH + H) (H codes from each half) and TL = 16 - 2H tail codes
// [r + q TL, ...); GPT-J lane q holds the 2H interleaved codes of the same
// pairs.  No lane exchange is needed to turn a pair; the row maxima are
// reductions over the row's L adjacent lanes.  One-shot workgroups of
// rpb = kI8Threads / L whole rows, walking lg layers.
template <int H, bool NEOX, bool KEEP>
__global__ __launch_bounds__(kI8Threads) void rerotate_int8_lanes_kernel(RerotArgs a) {
  constexpr int TL = 16 - 2 * H;
  constexpr int NR = (2 * H + 3) / 4;  // words of the rotary codes (per half under NeoX)
  constexpr int NT = TL > 0 ? (TL + 3) / 4 : 1;
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const ChunkRows c = chunk_rows(a);
  float *s_cs = s_tab, *s_sn = s_tab + c.np * half;
  turn_table(a, c.pa, c.np, s_cs, s_sn);
  const int r = a.to.rotary_dim;
  const int L = a.D / 16;
  const int rr = threadIdx.x / L, q = threadIdx.x - rr * L;
  // rows past the layer's end turn zeros and store nothing; a row's lanes share that state
  const bool live = rr < c.nrows;
  const int tab = ((c.r0 + (live ? rr : 0)) / a.Hkv - c.pa) * half + q * H;
  const long layer_rows = (long)a.rows_T * a.Hkv;
  int8_t *rp = (int8_t *)a.k + (c.row0 + rr) * a.D;
  float *sp = a.scale + c.row0 + rr;
  for (int l = 0; l < c.nl; ++l, rp += layer_rows * a.D, sp += layer_rows) {
  uint32_t w1[NR], w2[NR], wt[NT];
#pragma unroll
  for (int i = 0; i < NR; ++i) w1[i] = w2[i] = 0u;
#pragma unroll
  for (int i = 0; i < NT; ++i) wt[i] = 0u;
  float sco = 0.f;
  if (live) {
    sco = *sp;
    if constexpr (NEOX) {
      ld_n<H>(w1, rp + q * H);
      ld_n<H>(w2, rp + half + q * H);
    } else {
      ld_n<2 * H>(w1, rp + 2 * q * H);
    }
    if constexpr (TL > 0) ld_n<TL>(wt, rp + r + q * TL);
  }
  float y[2 * H];  // turned rotary values: y[2e], y[2e + 1] = pair e
  float mrot = 0.f, mtail = 0.f;
#pragma unroll
  for (int e = 0; e < H; ++e) {
    const float cs = s_cs[tab + e], sn = s_sn[tab + e];
    const float x1 = NEOX ? code_at(w1, e) : code_at(w1, 2 * e);
    const float x2 = NEOX ? code_at(w2, e) : code_at(w1, 2 * e + 1);
    y[2 * e] = x1 * cs - x2 * sn;
    y[2 * e + 1] = x2 * cs + x1 * sn;
    mrot = fmaxf(mrot, fmaxf(fabsf(y[2 * e]), fabsf(y[2 * e + 1])));
  }
  float yt[TL > 0 ? TL : 1];
#pragma unroll
  for (int e = 0; e < TL; ++e) {
    yt[e] = code_at(wt, e);
    mtail = fmaxf(mtail, fabsf(yt[e]));
  }
  for (int m = L >> 1; m >= 1; m >>= 1) {
    mrot = fmaxf(mrot, __shfl_xor(mrot, m));
    if constexpr (TL > 0) mtail = fmaxf(mtail, __shfl_xor(mtail, m));
  }
  const bool keep = KEEP && mrot < 127.5f;
  const float amax = fmaxf(mrot, mtail);
  const float inv = keep ? 1.0f : (amax > 0.f && sco > 0.f ? 127.0f / amax : 0.f);
  if (!live) continue;
  uint32_t c1[NEOX ? H : 2 * H], c2[H];
#pragma unroll
  for (int e = 0; e < H; ++e) {
    if constexpr (NEOX) {
      c1[e] = code_fma(y[2 * e], inv);
      c2[e] = code_fma(y[2 * e + 1], inv);
    } else {
      c1[2 * e] = code_fma(y[2 * e], inv);
      c1[2 * e + 1] = code_fma(y[2 * e + 1], inv);
    }
  }
  uint32_t p1[NR], p2[NR];
  if constexpr (NEOX) {
    pack_codes<H>(p1, c1);
    pack_codes<H>(p2, c2);
    st_n<H>(rp + q * H, p1);
    st_n<H>(rp + half + q * H, p2);
  } else {
    pack_codes<2 * H>(p1, c1);
    st_n<2 * H>(rp + 2 * q * H, p1);
  }
  if (!keep) {
    if constexpr (TL > 0) {
      uint32_t ct[TL], pt[NT];
#pragma unroll
      for (int e = 0; e < TL; ++e) ct[e] = code_fma(yt[e], inv);
      pack_codes<TL>(pt, ct);
      st_n<TL>(rp + r + q * TL, pt);
    }
    if (q == 0) *sp = inv > 0.f ? sco * (amax / 127.0f) : 0.f;
  }
  }
}

// ---- Chunk kernels: one 16-byte chunk of a row per thread.
//
// On this part an in-place stream of 16-byte chunks runs fastest in small one-shot
// workgroups (128 threads, one layer each) whose loads and stores stream past the
// caches (sc0 sc1 nt): a probe over a 32 GiB buffer moved 6.5 TB/s both for whole
// rows and for the rotary half of 256-byte fp16 rows (read + write counted), against
// 5.3 TB/s for the same half rows with cached loads and stores in 256-thread
// workgroups.  A row's chunks sit in adjacent lanes; under NeoX pairing the chunks of
// the first half of the rotary slice hold the first members of pairs and the chunks
// of the second half the partners, R / 2 lanes away (R rotary chunks per row, R / 2 a
// power of two), so a pair's partner comes from one lane exchange.  GPT-J pairs
// (2i, 2i + 1) lie inside a chunk.

// The value of lane l ^ M for M = 1, 2, 4, 8 (lane groups inside rows of 16 lanes) by DPP lane
// moves, no LDS round trip; larger M by a cross-lane permute.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm 1, 0, 3, 2
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm 2, 3, 0, 1
  } else if constexpr (M == 4 || M == 8) {
    // row_shl:M reads lane l + M, row_shr:M lane l - M; a lane keeps the one inside its row
    const uint32_t up = __builtin_amdgcn_mov_dpp(v, 0x100 + M, 0xF, 0xF, true);
    const uint32_t dn = __builtin_amdgcn_mov_dpp(v, 0x110 + M, 0xF, 0xF, true);
    return (__lane_id() & M) ? dn : up;
  } else {
    return (uint32_t)__shfl_xor((int)v, M);
  }
}
template <int M>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __uint_as_float(xor_lane<M>(__float_as_uint(v)));
}
// max over the aligned group of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, xor_lane_f<1>(v));
  if constexpr (G >= 4) v = fmaxf(v, xor_lane_f<2>(v));
  if constexpr (G >= 8) v = fmaxf(v, xor_lane_f<4>(v));
  if constexpr (G >= 16) v = fmaxf(v, xor_lane_f<8>(v));
  if constexpr (G >= 32) v = fmaxf(v, xor_lane_f<16>(v));
  if constexpr (G >= 64) v = fmaxf(v, xor_lane_f<32>(v));
  return v;
}

constexpr int kChunkThreads = 128;
constexpr int kI8Chunks = 4;  // int8 chunk kernel: row blocks (chunks per thread) per workgroup
constexpr int kFloatChunks = 1;  // float chunk kernel: row blocks per workgroup
constexpr int kI8HalfChunks = 1;  // int8 half-rotary kernel: row blocks per workgroup
constexpr int kStream = 19;  // buffer cache policy: sc0 | nt | sc1
// Row scales go through the caches: a wave writes the 4-byte scales of 8 rows (32 bytes of a
// 128-byte line, the rest from other waves and blocks); streamed, those partial lines cost the
// int8 pass 6 % (13.25 -> 12.49 ms on the 64-layer switch)
constexpr int kScalePolicy = 0;

typedef decltype(__builtin_amdgcn_raw_buffer_load_b128(__amdgpu_buffer_rsrc_t(), 0, 0, 0)) b128_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(void *base, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
template <int POLICY = kStream>
__device__ __forceinline__ void chunk_load(uint32_t *w, __amdgpu_buffer_rsrc_t r, int off) {
  const b128_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
  w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
}
__device__ __forceinline__ void chunk_store(const uint32_t *w, __amdgpu_buffer_rsrc_t r, int off) {
  b128_t v;
  v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStream);
}

// Float keys: R = r * sizeof(T) / 16 rotary chunks per row (R a power of two, R <= 32); a
// workgroup owns NCH blocks of kChunkThreads / R consecutive rows of one layer, each thread one
// chunk of every block, all loads issued before the first turn; chunk c sits at byte 16 c of
// its row.  Rows past the layer's end lie beyond the buffer resource's extent: their loads
// return zeros without touching memory and they store nothing.
template <typename T, int R, int NCH, bool NEOX>
__global__ __launch_bounds__(kChunkThreads) void rerotate_float_chunk_kernel(RerotArgs a) {
  constexpr int EB = sizeof(T);
  constexpr int CPE = 16 / EB;  // elements per chunk
  constexpr int RB = kChunkThreads / R;  // rows per block
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const ChunkRows c = chunk_rows(a);
  const int rr = threadIdx.x / R, ch = threadIdx.x % R;
  const int rowb = a.D * EB;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc((char *)a.k + c.row0 * rowb, (long)c.nrows * rowb);
  const double dwt = own_dw(a);
  uint32_t w[NCH][4];
#pragma unroll
  for (int k = 0; k < NCH; ++k) chunk_load(w[k], rs, (rr + k * RB) * rowb + 16 * ch);  // in flight during the table
  float *s_cs = s_tab, *s_sn = s_tab + c.np * half;
  turn_table_w(a, c.pa, c.np, s_cs, s_sn, dwt);
  // pair base of this chunk
  const int pb = NEOX ? CPE * (ch % (R / 2)) : CPE / 2 * ch;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int row = rr + k * RB;
    const bool live = row < c.nrows;
    const float *cs = &s_cs[((c.r0 + (live ? row : 0)) / a.Hkv - c.pa) * half + pb];
    const float *sn = &s_sn[((c.r0 + (live ? row : 0)) / a.Hkv - c.pa) * half + pb];
    uint32_t *v = w[k];
    if constexpr (NEOX) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = xor_lane<R / 2>(v[i]);
      const bool first = ch < R / 2;  // holds first members (x1), the partner holds x2
#pragma unroll
      for (int e = 0; e < CPE; e += 2) {
        const float own0 = vget<T>(v, e), own1 = vget<T>(v, e + 1);
        const float par0 = vget<T>(pw, e), par1 = vget<T>(pw, e + 1);
        const float y0 = first ? own0 * cs[e] - par0 * sn[e] : own0 * cs[e] + par0 * sn[e];
        const float y1 = first ? own1 * cs[e + 1] - par1 * sn[e + 1] : own1 * cs[e + 1] + par1 * sn[e + 1];
        vput2<T>(v, e, y0, y1);
      }
    } else {
#pragma unroll
      for (int e = 0; e < CPE; e += 2) {
        const float x1 = vget<T>(v, e), x2 = vget<T>(v, e + 1);
        vput2<T>(v, e, x1 * cs[e / 2] - x2 * sn[e / 2], x2 * cs[e / 2] + x1 * sn[e / 2]);
      }
    }
    if (live) chunk_store(v, rs, row * rowb + 16 * ch);
  }
}

// int8 keys with a per-row fp32 scale, turned in code units (see the lane kernel below):
// L = D / 16 lanes per row with 16 codes each, RC = r / 16 rotary chunks (NeoX: RC / 2 a
// power of two).  A workgroup owns NCH blocks of kChunkThreads / L consecutive rows of one
// layer and each thread one chunk of every block: all the blocks' loads are issued before
// any of them is turned, so one wait for memory serves NCH chunks (workgroups are short-lived
// and their lifetime is the memory wait plus the turn).  Every lane runs the same
// instructions: a lane of the tail turns by the identity (cos 1, sin 0, from a constant block
// of the table), and the NeoX sign of the partner term comes from a negated copy of the sine
// rows, so no lane waits while its row's other lanes take another branch.  The row's turned
// rotary maximum and overall maximum are reductions over its L lanes.
// Table layout (dynamic LDS, floats): cos [np][half], sin [np][half], -sin [np][half], then 16
// ones and 16 zeros.
template <int L, bool NEOX, bool KEEP>
__device__ __forceinline__ void turn_i8_chunk(const uint32_t *w, float sco, bool live, bool rot, int hc,
                                              const float *cs, const float *sn, __amdgpu_buffer_rsrc_t rs,
                                              __amdgpu_buffer_rsrc_t rsc, int off, int soff, bool lead) {
  uint32_t pw[4] = {0u, 0u, 0u, 0u};
  if constexpr (NEOX) {
    // partner chunk hc = RC / 2 lanes away, a power of two <= L / 2 (checked on the host); tail
    // lanes exchange too and multiply the partner by zero (uniform branch on the rotary width)
    switch (hc) {
      case 1:
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = xor_lane<1>(w[i]);
        break;
      case 2:
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = xor_lane<2>(w[i]);
        break;
      case 4:
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = xor_lane<4>(w[i]);
        break;
      default:
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = xor_lane<8>(w[i]);
        break;
    }
  }
  float y[16];
  float m = 0.f;
  if constexpr (NEOX) {
    // 16 cos and 16 sin, 16-byte reads (every table row and block starts 64-byte aligned)
    float4 c4[4], s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c4[i] = ((const float4 *)cs)[i];
      s4[i] = ((const float4 *)sn)[i];
    }
    const float *cv = (const float *)c4, *sv = (const float *)s4;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      y[e] = fmaf(code_at(pw, e), sv[e], code_at(w, e) * cv[e]);
      m = fmaxf(m, fabsf(y[e]));
    }
  } else {
    float4 c4[2], s4[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c4[i] = ((const float4 *)cs)[i];
      s4[i] = ((const float4 *)sn)[i];
    }
    const float *cv = (const float *)c4, *sv = (const float *)s4;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float x1 = code_at(w, e), x2 = code_at(w, e + 1);
      y[e] = x1 * cv[e / 2] - x2 * sv[e / 2];
      y[e + 1] = x2 * cv[e / 2] + x1 * sv[e / 2];
      m = fmaxf(m, fmaxf(fabsf(y[e]), fabsf(y[e + 1])));
    }
  }
  const float amax = group_max<L>(m);
  bool keep = false;
  if constexpr (KEEP) keep = group_max<L>(rot ? m : 0.f) < 127.5f;
  const float inv = keep ? 1.0f : (amax > 0.f && sco > 0.f ? 127.0f / amax : 0.f);
  if (!live || (keep && !rot)) return;
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = pack4_codes(code_fma(y[4 * i], inv), code_fma(y[4 * i + 1], inv), code_fma(y[4 * i + 2], inv),
                         code_fma(y[4 * i + 3], inv));
  chunk_store(out, rs, off);
  if (!keep && lead)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, inv > 0.f ? sco * (amax / 127.0f) : 0.f), rsc,
                                          soff, 0, kScalePolicy);
}

template <int L, int NCH, bool NEOX, bool KEEP>
__global__ __launch_bounds__(kChunkThreads) void rerotate_int8_chunk_kernel(RerotArgs a) {
  constexpr int RB = kChunkThreads / L;  // rows per block
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const ChunkRows c = chunk_rows(a);
  const int rr = threadIdx.x / L, ch = threadIdx.x % L;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc((char *)a.k + c.row0 * a.D, (long)c.nrows * a.D);
  const __amdgpu_buffer_rsrc_t rsc = span_rsrc(a.scale + c.row0, (long)c.nrows * 4);
  const double dwt = own_dw(a);
  // every block's chunk and scale in flight while the turn table is built; rows past the
  // layer's end lie beyond the buffer resources' extents, so their loads return zeros without
  // touching memory
  uint32_t w[NCH][4];
  float sco[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    chunk_load(w[k], rs, (rr + k * RB) * a.D + 16 * ch);
    sco[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, 4 * (rr + k * RB), 0, kScalePolicy));
  }
  const int nt = c.np * half;
  float *s_cs = s_tab, *s_sn = s_tab + nt, *s_nsn = s_tab + 2 * nt, *s_id = s_tab + 3 * nt;
  if (threadIdx.x < 32) s_id[threadIdx.x] = threadIdx.x < 16 ? 1.0f : 0.0f;
  turn_table_w(a, c.pa, c.np, s_cs, s_sn, dwt, s_nsn);
  // this lane's table columns (the same in every block) and rows (one per position)
  const int RC = a.to.rotary_dim / 16, hc = RC >> 1;
  const bool rot = ch < RC;
  const int col = NEOX ? 16 * (ch & (hc - 1)) : 8 * ch;
  const float *cs0 = rot ? s_cs + col : s_id;
  const float *sn0 = rot ? (NEOX && ch < hc ? s_nsn : s_sn) + col : s_id + 16;  // NeoX first members: x1 cos - x2 sin
  const int rstep = rot ? half : 0;  // tail lanes stay on the identity block
  const int pos_r = (c.r0 + rr) / a.Hkv - c.pa;
  const bool even = RB % a.Hkv == 0;  // blocks start at whole positions: positions step by RB / Hkv
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int row = rr + k * RB;
    const bool live = row < c.nrows;
    const int pr = even ? pos_r + k * (RB / a.Hkv) : (c.r0 + (live ? row : 0)) / a.Hkv - c.pa;
    const int prow = (live ? pr : 0) * rstep;
    turn_i8_chunk<L, NEOX, KEEP>(w[k], sco[k], live, rot, hc, cs0 + prow, sn0 + prow, rs, rsc, row * a.D + 16 * ch,
                                 4 * row, ch == 0);
  }
}

// int8 keys whose rotary slice is half the row (r = D / 2): H = D / 32 lanes per row, lane q
// holding rotary chunk q (codes 16 q ..) and tail chunk q (codes r + 16 q ..), so every lane
// turns 16 codes and requantises 32 with no lane idle; NeoX partners sit RC / 2 = H / 2 lanes
// away.  A workgroup owns NCH blocks of kChunkThreads / H rows of one layer, all loads issued
// before the first turn (as the chunk kernel above).  Table layout as the chunk kernel's,
// without the identity block.
template <int H, int NCH, bool NEOX, bool KEEP>
__global__ __launch_bounds__(kChunkThreads) void rerotate_int8_half_kernel(RerotArgs a) {
  constexpr int RB = kChunkThreads / H;  // rows per block
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;  // = 8 H pairs
  const ChunkRows c = chunk_rows(a);
  const int rr = threadIdx.x / H, q = threadIdx.x % H;
  const __amdgpu_buffer_rsrc_t rs = span_rsrc((char *)a.k + c.row0 * a.D, (long)c.nrows * a.D);
  const __amdgpu_buffer_rsrc_t rsc = span_rsrc(a.scale + c.row0, (long)c.nrows * 4);
  const double dwt = own_dw(a);
  uint32_t wr[NCH][4], wt[NCH][4];
  float sco[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int o = (rr + k * RB) * a.D + 16 * q;
    // the two 64-byte halves of a row's line come from separate loads, which run faster through
    // the caches than streamed past them (measured: streamed, the keep-scale pass takes 6 % longer)
    chunk_load<0>(wr[k], rs, o);
    chunk_load<0>(wt[k], rs, o + a.to.rotary_dim);
    sco[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, 4 * (rr + k * RB), 0, kScalePolicy));
  }
  const int nt = c.np * half;
  float *s_cs = s_tab, *s_sn = s_tab + nt, *s_nsn = s_tab + 2 * nt;
  turn_table_w(a, c.pa, c.np, s_cs, s_sn, dwt, s_nsn);
  constexpr int HC = H / 2;  // NeoX: partner lane distance
  const int col = NEOX ? 16 * (q & (HC - 1)) : 8 * q;
  const float *cs0 = s_cs + col;
  const float *sn0 = (NEOX && q < HC ? s_nsn : s_sn) + col;  // NeoX first members: x1 cos - x2 sin
  const int pos_r = (c.r0 + rr) / a.Hkv - c.pa;
  const bool even = RB % a.Hkv == 0;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int row = rr + k * RB;
    const bool live = row < c.nrows;
    const int pr = even ? pos_r + k * (RB / a.Hkv) : (c.r0 + (live ? row : 0)) / a.Hkv - c.pa;
    const float *cs = cs0 + (live ? pr : 0) * half;
    const float *sn = sn0 + (live ? pr : 0) * half;
    const uint32_t *w = wr[k];
    float y[16], t[16];
    float mr = 0.f, mt = 0.f;
    if constexpr (NEOX) {
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = xor_lane<HC>(w[i]);
      float4 c4[4], s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = ((const float4 *)cs)[i];
        s4[i] = ((const float4 *)sn)[i];
      }
      const float *cv = (const float *)c4, *sv = (const float *)s4;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        y[e] = fmaf(code_at(pw, e), sv[e], code_at(w, e) * cv[e]);
        mr = fmaxf(mr, fabsf(y[e]));
      }
    } else {
      float4 c4[2], s4[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        c4[i] = ((const float4 *)cs)[i];
        s4[i] = ((const float4 *)sn)[i];
      }
      const float *cv = (const float *)c4, *sv = (const float *)s4;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float x1 = code_at(w, e), x2 = code_at(w, e + 1);
        y[e] = x1 * cv[e / 2] - x2 * sv[e / 2];
        y[e + 1] = x2 * cv[e / 2] + x1 * sv[e / 2];
        mr = fmaxf(mr, fmaxf(fabsf(y[e]), fabsf(y[e + 1])));
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      t[e] = code_at(wt[k], e);
      mt = fmaxf(mt, fabsf(t[e]));
    }
    mr = group_max<H>(mr);
    const float amax = fmaxf(mr, group_max<H>(mt));
    const bool keep = KEEP && mr < 127.5f;
    const float inv = keep ? 1.0f : (amax > 0.f && sco[k] > 0.f ? 127.0f / amax : 0.f);
    if (!live) continue;
    const int o = row * a.D + 16 * q;
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[i] = pack4_codes(code_fma(y[4 * i], inv), code_fma(y[4 * i + 1], inv), code_fma(y[4 * i + 2], inv),
                           code_fma(y[4 * i + 3], inv));
    chunk_store(out, rs, o);
    if (!keep) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[i] = pack4_codes(code_fma(t[4 * i], inv), code_fma(t[4 * i + 1], inv), code_fma(t[4 * i + 2], inv),
                             code_fma(t[4 * i + 3], inv));
      chunk_store(out, rs, o + a.to.rotary_dim);
      if (q == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, inv > 0.f ? sco[k] * (amax / 127.0f) : 0.f),
                                              rsc, 4 * row, 0, kScalePolicy);
    }
  }
}

// int8 keys with a per-row fp32 scale.  LPR = D / 16 lanes per row, each
// holding 16 consecutive codes; NeoX partners sit half / 16 lanes apart and
// are exchanged by shuffles.
__global__ __launch_bounds__(256) void rerotate_int8_kernel(RerotArgs a) {
  __shared__ float s_cs[kPT * 256], s_sn[kPT * 256];
  const int t0 = blockIdx.x * kPT;
  const float gain = angle_setup(a, t0, s_cs, s_sn);
  const int half = a.to.rotary_dim / 2;
  const int r = a.to.rotary_dim;
  const int lpr = a.D / 16;               // lanes per row (power of two, <= 64)
  const int rows_per_pass = 256 / lpr;
  const int npos = min(kPT, a.rows_T - t0);
  const int nrows = npos * a.Hkv;
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x % lpr;        // chunk of this lane within its row
  const int part = half / 16;             // NeoX partner distance in lanes
  const int neox = a.to.neox;
  const long layer_rows = (long)a.rows_T * a.Hkv;
  int8_t *kc = (int8_t *)a.k;
  for (int layer = 0; layer < a.n_layers; ++layer) {
    const long row0 = layer * layer_rows + (long)t0 * a.Hkv;
    // every lane runs the same number of passes so the shuffles stay converged
    for (int base = 0; base < nrows; base += rows_per_pass) {
      const int rr = base + threadIdx.x / lpr;
      const bool live = rr < nrows;
      const long row = row0 + (live ? rr : 0);
      const int pt = (live ? rr : 0) / a.Hkv;
      const float sc_old = live ? a.scale[row] : 0.f;
      uint4 w = live ? *(const uint4 *)(kc + row * a.D + q * 16) : make_uint4(0, 0, 0, 0);
      float x[16];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = (float)(int8_t)((ww[e >> 2] >> (8 * (e & 3))) & 0xff) * sc_old;
      float y[16];
      if (neox) {
        // partner chunk: first-half lanes q < part pair with q + part
        const bool rot = q < 2 * part && 16 * q < r;
        const int src = (q < part) ? lane + part : lane - part;
        float px[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) px[e] = __shfl(x[e], src);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (rot) {
            const int j = (q < part ? q : q - part) * 16 + e;
            const float cs = s_cs[pt * half + j], sn = s_sn[pt * half + j];
            y[e] = (q < part) ? (x[e] * cs - px[e] * sn) * gain : (x[e] * cs + px[e] * sn) * gain;
          } else {
            y[e] = x[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int j = (q * 16 + e) / 2;
          if (16 * q + e < r) {
            const float cs = s_cs[pt * half + j], sn = s_sn[pt * half + j];
            y[e] = (x[e] * cs - x[e + 1] * sn) * gain;
            y[e + 1] = (x[e + 1] * cs + x[e] * sn) * gain;
          } else {
            y[e] = x[e];
            y[e + 1] = x[e + 1];
          }
        }
      }
      const bool rot_chunk = 16 * q < r;  // rotary_dim is a multiple of 16: chunks are rotary or tail
      bool keep = false;
      float inv = 0.f, amax = 0.f;
      if (a.keep_scale) {
        const float inv_old = sc_old > 0.f ? 1.0f / sc_old : 0.f;
        float mx = 0.f;
        if (rot_chunk) {
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(rintf(y[e] * inv_old)));
        }
        keep = row_keeps_scale(mx, lpr);
        inv = inv_old;
      }
      if (!keep) {
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(y[e]));
        for (int m = lpr >> 1; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        inv = amax > 0.f ? 127.0f / amax : 0.f;
      }
      uint32_t out[4], cb[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) cb[e] = code_bits(y[e], inv);
      pack_codes<16>(out, cb);
      if (live) {
        if (!keep || rot_chunk) *(uint4 *)(kc + row * a.D + q * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        if (q == 0 && !keep) a.scale[row] = amax / 127.0f;
      }
    }
  }
}

// Hadamard-rotated int8 keys: a row holds the codes of H k, H the orthonormal
// Walsh-Hadamard transform over its D dims.  Per row: transform the codes
// (unnormalised butterflies, exact in fp32), turn the rotary pairs, transform
// again and multiply by scale / D (the two transforms' normalisation), then
// requantise the row.  L = D / 32 lanes per row; lane q holds dims
// [32 q, 32 q + 32), so butterflies over bits 0..4 stay in the lane and the
// rest are lane exchanges.  NeoX partners (i, i + r/2) sit r / 64 lanes apart,
// GPT-J partners in the same lane.
__device__ __forceinline__ void fwht_lane32(float (&x)[32], int q, int L) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & h) == 0) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
  for (int m = 1; m < L; m <<= 1) {
    const bool upper = (q & m) != 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float p = __shfl_xor(x[j], m);
      x[j] = upper ? p - x[j] : x[j] + p;
    }
  }
}

__global__ __launch_bounds__(256) void rerotate_int8_hadamard_kernel(RerotArgs a) {
  __shared__ float s_cs[kPT * 256], s_sn[kPT * 256];
  const int t0 = blockIdx.x * kPT;
  const float gain = angle_setup(a, t0, s_cs, s_sn);
  const int half = a.to.rotary_dim / 2;
  const int r = a.to.rotary_dim;
  const int L = a.D / 32;                // lanes per row (power of two, 2..16)
  const int rows_per_pass = 256 / L;
  const int npos = min(kPT, a.rows_T - t0);
  const int nrows = npos * a.Hkv;
  const int q = threadIdx.x % L;
  const int part = half / 32;            // NeoX partner distance in lanes (power of two)
  const int neox = a.to.neox;
  const float post = 1.0f / (float)a.D;  // H H unnormalised = D x identity
  const long layer_rows = (long)a.rows_T * a.Hkv;
  int8_t *kc = (int8_t *)a.k;
  for (int layer = 0; layer < a.n_layers; ++layer) {
    const long row0 = layer * layer_rows + (long)t0 * a.Hkv;
    // every lane runs the same number of passes so the lane exchanges stay converged
    for (int base = 0; base < nrows; base += rows_per_pass) {
      const int rr = base + threadIdx.x / L;
      const bool live = rr < nrows;
      const long row = row0 + (live ? rr : 0);
      const int pt = (live ? rr : 0) / a.Hkv;
      const float sc_old = live ? a.scale[row] : 0.f;
      const int8_t *src = kc + row * a.D + 32 * q;
      const uint4 w0 = live ? *(const uint4 *)src : make_uint4(0, 0, 0, 0);
      const uint4 w1 = live ? *(const uint4 *)(src + 16) : make_uint4(0, 0, 0, 0);
      const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float x[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = (float)(int8_t)((ww[e >> 2] >> (8 * (e & 3))) & 0xff);
      fwht_lane32(x, q, L);
      float y[32];
      if (neox) {
        const bool rot = q < 2 * part, first = q < part;
        const int i0 = 32 * (first ? q : q - part);
        float px[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) px[e] = __shfl_xor(x[e], part);
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          if (rot) {
            const float cs = s_cs[pt * half + i0 + e], sn = s_sn[pt * half + i0 + e];
            y[e] = first ? (x[e] * cs - px[e] * sn) * gain : (x[e] * cs + px[e] * sn) * gain;
          } else {
            y[e] = x[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 32; e += 2) {
          if (32 * q + e < r) {
            const int i = (32 * q + e) / 2;
            const float cs = s_cs[pt * half + i], sn = s_sn[pt * half + i];
            y[e] = (x[e] * cs - x[e + 1] * sn) * gain;
            y[e + 1] = (x[e + 1] * cs + x[e] * sn) * gain;
          } else {
            y[e] = x[e];
            y[e + 1] = x[e + 1];
          }
        }
      }
      fwht_lane32(y, q, L);
      const float f = sc_old * post;
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        y[e] *= f;
        amax = fmaxf(amax, fabsf(y[e]));
      }
      for (int m = L >> 1; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float inv = amax > 0.f ? 127.0f / amax : 0.f;
      uint32_t out[8], cb[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) cb[e] = code_bits(y[e], inv);
      pack_codes<16>(out, cb);
      pack_codes<16>(out + 4, cb + 16);
      if (live) {
        int8_t *dst = kc + row * a.D + 32 * q;
        *(uint4 *)dst = make_uint4(out[0], out[1], out[2], out[3]);
        *(uint4 *)(dst + 16) = make_uint4(out[4], out[5], out[6], out[7]);
        if (q == 0) a.scale[row] = amax / 127.0f;
      }
    }
  }
}

// Hadamard-rotated int8 keys at head_dim 128: two lanes per row, lane q holding
// the 64 consecutive dims [64 q, 64 q + 64), so six butterfly stages of each
// transform stay in the lane and the seventh is one exchange with the
// neighbouring lane (a DPP move, no LDS traffic).  Chunked workgroups of 128
// rows like the lane kernel; the turn runs in code units of H c (the first
// transform of integer codes is exact in fp32) with the gain in the cos / sin
// table, and the two unnormalised transforms' factor 1 / 128 goes into the scale.
// RN: 128 for NeoX over all dims (pair e is dim e of lane 0 with dim e of lane 1);
// 0: GPT-J, pairs (2i, 2i + 1) of dims < r.  NeoX with r = 64 has a kernel of its own
// below that transforms half rows.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
}

// unnormalised Walsh-Hadamard transform over 128 dims held as 64 per lane in lane
// pairs; sgn = +1 on the lower lane, -1 on the upper one
__device__ __forceinline__ void fwht128(float (&x)[64], float sgn) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int j = 0; j < 64; ++j)
      if ((j & h) == 0) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
#pragma unroll
  for (int j = 0; j < 64; ++j) x[j] = fmaf(sgn, x[j], dpp_xor1(x[j]));  // lower: x + p, upper: p - x
}

template <int RN>
__global__ __launch_bounds__(256) void rerotate_int8_hadamard128_kernel(RerotArgs a) {
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const int r = a.to.rotary_dim;
  const ChunkRows c = chunk_rows(a);
  float *s_cs = s_tab, *s_sn = s_tab + c.np * half;
  turn_table(a, c.pa, c.np, s_cs, s_sn);
  const int rr = threadIdx.x >> 1, q = threadIdx.x & 1;
  // rows past the layer's end turn zeros and store nothing; both lanes of a row share that state
  const bool live = rr < c.nrows;
  const int tab = ((c.r0 + (live ? rr : 0)) / a.Hkv - c.pa) * half;
  const long layer_rows = (long)a.rows_T * a.Hkv;
  int8_t *rp = (int8_t *)a.k + (c.row0 + rr) * 128 + 64 * q;
  float *sp = a.scale + c.row0 + rr;
  const float sgn = q ? -1.f : 1.f;
  for (int l = 0; l < c.nl; ++l, rp += layer_rows * 128, sp += layer_rows) {
    uint32_t w[16];
    float sco = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0u;
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = ((const uint4 *)rp)[i];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
      sco = *sp;
    }
    float x[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) x[e] = code_at(w, e);
    fwht128(x, sgn);
    // the turn, 8 pairs at a time: the scheduling fences keep the cos / sin reads of
    // one group from being hoisted over the others (which would hold 128 more registers)
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RN == 128) {
#pragma unroll
      for (int e0 = 0; e0 < 64; e0 += 8) {
#pragma unroll
        for (int e = e0; e < e0 + 8; ++e) {
          const float p = dpp_xor1(x[e]);
          x[e] = x[e] * s_cs[tab + e] - sgn * p * s_sn[tab + e];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i0 = 0; i0 < 32; i0 += 8) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
          const int d = 64 * q + 2 * i;
          const bool rot = d < r;
          const int ti = tab + (rot ? d / 2 : 0);
          const float cl = s_cs[ti], sl = s_sn[ti];
          const float cs = rot ? cl : 1.f, sn = rot ? sl : 0.f;
          const float x1 = x[2 * i], x2 = x[2 * i + 1];
          x[2 * i] = x1 * cs - x2 * sn;
          x[2 * i + 1] = x2 * cs + x1 * sn;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    fwht128(x, sgn);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, dpp_xor1(amax));
    const float inv = amax > 0.f && sco > 0.f ? 127.0f / amax : 0.f;
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      out[i] = pack4_codes(code_fma(x[4 * i], inv), code_fma(x[4 * i + 1], inv), code_fma(x[4 * i + 2], inv),
                           code_fma(x[4 * i + 3], inv));
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ((uint4 *)rp)[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
      if (q == 0) *sp = inv > 0.f ? sco * amax * (1.0f / (127.0f * 128.0f)) : 0.f;
    }
  }
}

// Hadamard-rotated int8 keys at head_dim 128 whose rotary dims lie in the leading 64
// (NeoX with r = 64: pairs (e, e + 32); GPT-J with r <= 64: pairs (2i, 2i + 1) of
// dims < r).  With H the unnormalised Sylvester-ordered transform of
// order 128 (H = [[H64, H64], [H64, -H64]]) the key in code units is x = H c, and
// the turn R (gain included) moves x[0..63] only, so
//   H R H c = 128 c + H [D; 0],  D = (R - I) x[0..63],  x[0..63] = H64 (c_lo + c_hi),
//   H [D; 0] = [H64 D; H64 D]    (c_lo, c_hi: codes 0..63 and 64..127).
// Two 64-point transforms on half a row replace two 128-point ones on the whole row.
// Lane q of a row's pair holds codes 32 q .. 32 q + 31 of each half, so its half of
// u = c_lo + c_hi is lane-local, the 64-point transforms run five stages in the lane
// and the top one across the pair, NeoX partners x[e] and x[e + 32] sit at the same
// index of the two lanes (GPT-J partners share a lane), and 128 c + H64 D needs only
// the lane's own indices.  The factor 1 / 128 of the two transforms goes into the scale
// as in the kernel above.  This kernel serves GPT-J pairs with r <= 64; NeoX r = 64 has
// the staged kernel below.
__device__ __forceinline__ void fwht64_pair(float (&x)[32], float sgn) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & h) == 0) {
        const float u = x[j], v = x[j + h];
        x[j] = u + v;
        x[j + h] = u - v;
      }
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = fmaf(sgn, x[j], dpp_xor1(x[j]));  // lower: x + p, upper: p - x
}

__global__ __launch_bounds__(256) void rerotate_int8_hadamard128_r64_kernel(RerotArgs a) {
  extern __shared__ float s_tab[];
  const int half = a.to.rotary_dim / 2;
  const int r = a.to.rotary_dim;
  const ChunkRows c = chunk_rows(a);
  float *s_cs = s_tab, *s_sn = s_tab + c.np * half;
  turn_table(a, c.pa, c.np, s_cs, s_sn);
  const int rr = threadIdx.x >> 1, q = threadIdx.x & 1;
  // rows past the layer's end turn zeros and store nothing; both lanes of a row share that state
  const bool live = rr < c.nrows;
  const int tab = ((c.r0 + (live ? rr : 0)) / a.Hkv - c.pa) * half;
  const long layer_rows = (long)a.rows_T * a.Hkv;
  int8_t *rp = (int8_t *)a.k + (c.row0 + rr) * 128 + 32 * q;  // + 64: the same lane's upper half
  float *sp = a.scale + c.row0 + rr;
  const float sgn = q ? -1.f : 1.f;
  for (int l = 0; l < c.nl; ++l, rp += layer_rows * 128, sp += layer_rows) {
    uint32_t w[16];  // words 0..7: codes 32 q + (0..31); 8..15: codes 64 + 32 q + (0..31)
    float sco = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = 0u;
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = ((const uint4 *)(rp + 64 * (i >> 1)))[i & 1];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
      sco = *sp;
    }
    float x[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = code_at(w, e) + code_at(w, 32 + e);
    fwht64_pair(x, sgn);  // x[e] = x[32 q + e] of H64 (c_lo + c_hi): integers, exact
    // D = (R - I) x
    __builtin_amdgcn_sched_barrier(0);
    {  // pair (2i, 2i + 1) = lane-local (e, e + 1) at dim 32 q + e; no turn from dim r on
#pragma unroll
      for (int e0 = 0; e0 < 32; e0 += 8) {
#pragma unroll
        for (int e = e0; e < e0 + 8; e += 2) {
          const int d = 32 * q + e;
          const bool rot = d < r;
          const int ti = tab + (rot ? d / 2 : 0);
          const float cl = s_cs[ti], sl = s_sn[ti];
          const float cs = rot ? cl : 1.f, sn = rot ? sl : 0.f;
          const float x1 = x[e], x2 = x[e + 1];
          x[e] = fmaf(-x2, sn, fmaf(x1, cs, -x1));
          x[e + 1] = fmaf(x1, sn, fmaf(x2, cs, -x2));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    fwht64_pair(x, sgn);  // x[e] = (H64 D)[32 q + e]
    float y[64];
#pragma unroll
    for (int e = 0; e < 64; ++e) y[e] = fmaf(code_at(w, e), 128.f, x[e & 31]);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 64; ++e) amax = fmaxf(amax, fabsf(y[e]));
    amax = fmaxf(amax, dpp_xor1(amax));
    const float inv = amax > 0.f && sco > 0.f ? 127.0f / amax : 0.f;
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      out[i] = pack4_codes(code_fma(y[4 * i], inv), code_fma(y[4 * i + 1], inv), code_fma(y[4 * i + 2], inv),
                           code_fma(y[4 * i + 3], inv));
    if (live) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ((uint4 *)(rp + 64 * (i >> 1)))[i & 1] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
      if (q == 0) *sp = inv > 0.f ? sco * amax * (1.0f / (127.0f * 128.0f)) : 0.f;
    }
  }
}

// NeoX r = 64 over Hadamard rows, with fewer vector instructions per row than the kernel
// above (same lane layout: lane q of a row's pair holds codes 32 q .. 32 q + 31 of each half).
//  * The first transform is exact integer arithmetic: u = c_lo + c_hi lies in [-256, 254]
//    and its 32-point transform within 32 x 256 = 8192, so it runs two values per
//    instruction on 16-bit halves; the sums of sign-extended code bytes are written
//    straight into the halves.
//  * The Sylvester transform splits as H64 = [[H32, H32], [H32, -H32]].  With
//    s = H32 u[0..31] (lane 0) and t = H32 u[32..63] (lane 1), the top stage of the first
//    transform, the turn R - I of the NeoX pairs (e, e + 32) and the top stage of the second
//    transform collapse into one map per pair:
//      H2 [[cm1, -sn], [sn, cm1]] H2 = 2 [[cm1, sn], [-sn, cm1]],   cm1 = cos - 1,
//    so (H64 D) / 2 is H32, on each lane, of (cm1 s + sn t, cm1 t - sn s): one partner
//    exchange replaces the two cross-lane butterfly stages, and sin / -sin come from two
//    table planes so both lanes run the same instructions.  cm1 is taken as
//    -2 sin^2(angle / 2) times the gain plus (gain - 1), exact for small angles.
//  * y / 2 = 64 c + (H64 D) / 2 is requantised against its row maximum; the factor 1 / 64 of
//    the unnormalised transforms goes into the scale.
// The table's layout in LDS: per position 36 floats (32 used), and the sin / -sin planes start
// 16 floats (mod 64) after the cos - 1 plane, so that a read of one entry group by the 8 distinct
// (plane, position) pairs of a wave falls in 8 distinct 16-byte bank groups.
__host__ __device__ constexpr int had_plane(int np) { return 36 * np; }
__host__ __device__ constexpr int had_off_sn(int np) { return (had_plane(np) + 47) / 64 * 64 + 16; }
__host__ __device__ constexpr int had_off_nsn(int np) { return had_off_sn(np) + (had_plane(np) + 63) / 64 * 64; }
__host__ __device__ constexpr int had_table_floats(int np) { return had_off_nsn(np) + had_plane(np); }
__device__ __forceinline__ void hadamard_pair_table(const RerotArgs &a, int pa, int np, float *s_tab, double dwt) {
  const int half = a.to.rotary_dim / 2;
  const float gain = (float)a.gain, gm1 = (float)(a.gain - 1.0);
  const bool same_pair = blockDim.x % half == 0;
  for (int idx = threadIdx.x; idx < np * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx - pt * half;
    const double th = (double)(a.pos0 + pa + pt) * (same_pair || idx == (int)threadIdx.x ? dwt : a.dw[i]);
    const double k = rint(th * 0.15915494309189535);  // turns of 2 pi
    const double rd = fma(-k, 2.4492935982947064e-16, fma(-k, 6.283185307179586, th));
    const float sf = sinf((float)rd), hs = sinf(0.5f * (float)rd);
    const int o = 36 * pt + i;
    s_tab[o] = fmaf(-2.f * gain * hs, hs, gm1);
    s_tab[had_off_sn(np) + o] = sf * gain;
    s_tab[had_off_nsn(np) + o] = -(sf * gain);
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
// 16-bit halves (sext(a.byte0) + sext(b.byte0), sext(a.byte2) + sext(b.byte2)), and the same
// for bytes 1 and 3: two byte adds written straight into the halves
__device__ __forceinline__ uint32_t add_bytes_02(uint32_t a, uint32_t b) {
  uint32_t r;
  __asm__("v_add_u32_sdwa %0, sext(%1), sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:BYTE_0\n\t"
          "v_add_u32_sdwa %0, sext(%1), sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_2 src1_sel:BYTE_2"
          : "=&v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t add_bytes_13(uint32_t a, uint32_t b) {
  uint32_t r;
  __asm__("v_add_u32_sdwa %0, sext(%1), sext(%2) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:BYTE_1\n\t"
          "v_add_u32_sdwa %0, sext(%1), sext(%2) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3 src1_sel:BYTE_3"
          : "=&v"(r) : "v"(a), "v"(b));
  return r;
}
// (lo, hi) -> (lo + hi, lo - hi) in one packed multiply-add: hi * 1 + lo and hi * 0xffff + lo
// (mod 2^16); k holds 0xffff0001
__device__ __forceinline__ uint32_t bfly_halves(uint32_t x, uint32_t k) {
  uint32_t r;
  __asm__("v_pk_mad_u16 %0, %1, %2, %1 op_sel:[1,0,0] op_sel_hi:[1,1,0]" : "=v"(r) : "v"(x), "v"(k));
  return r;
}

// o[e] += x'[e] * b[e] for 8 values, x' = x of the partner lane l ^ 1, as v_fmac_f32 with a DPP
// lane swap on its first operand (the compiler keeps the swap as a separate move).  The leading
// s_nop 1 gives the two wait states a DPP read needs after a vector write of its operand; inside
// the block no instruction reads a register another one writes.
__device__ __forceinline__ void fmac_partner8(float (&o)[8], const float *x, const float (&b)[8]) {
  __asm__("s_nop 1\n\t"
          "v_fmac_f32_dpp %0, %8, %16 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %17 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %18 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %19 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %20 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %21 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %22 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %23 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
          : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]), "+v"(o[4]), "+v"(o[5]), "+v"(o[6]), "+v"(o[7])
          : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
            "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]));
}

// Row staging for the kernel below: each wave owns 32 rows of the workgroup's 128 and walks the
// workgroup's layers; every 8 lanes move one whole 128-byte row (full cache lines, streamed) in
// and out.  The first layer's rows come by direct global -> LDS loads; each later layer's rows
// are loaded into registers two layers ahead and written into the stage once the layer before
// has left it.  Memory traffic and vector issue limit the pass together (on the 64-layer switch:
// no arithmetic 13.1 ms, arithmetic with no loads or stores 8.7 ms, the whole pass 13.0-13.5 ms,
// during which the chip holds about 1.9 GHz and the VALU issues at about its fp32 rate); the
// two-layer lead takes about 2 % off, one layer or a second LDS stage about 1 %.  Rows sit 144 bytes apart in the stage (9 slots of 16 bytes, the ninth unused), so that 8
// consecutive rows start in 8 distinct 16-byte bank groups and each lane reads its half row at
// fixed offsets from one address (the two lanes of a row read chunks 2 slots apart, which
// overlaps in banks two ways within 16 lanes).  Reading the rows in place (32 bytes of a row per
// lane pair and instruction) instead ran at the rate of the same pass with no arithmetic at all.
// Everything that depends on the lane is derived again in each layer from an opaque copy of the
// lane index: held across the layer loop, the turn table and the addresses took 150-190
// registers (3 waves per SIMD).
constexpr int kHadStage = 32 * 9 * 16;  // bytes per wave

__device__ __forceinline__ void had_load_rows(const int8_t *lk, uint8_t *stage, int ln, int nrows, int wrow0) {
#pragma unroll
  for (int jj = 0; jj < 5; ++jj) {
    const int sl = 64 * jj + ln, r = sl / 9, ch = min(sl - 9 * r, 7);
    if (jj < 4 || ln < 32) dma16_stream(lk + min(wrow0 + r, nrows - 1) * 128 + 16 * ch, stage + 1024 * jj);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void rerotate_int8_hadamard128_neox64_kernel(RerotArgs a) {
  extern __shared__ float s_tab[];  // [3][np][32] table, then one row stage per wave
  const int half = 32;
  const double dwt = own_dw(a);
  const ChunkRows c = chunk_rows(a);
  const int wv = threadIdx.x >> 6;
  const int wrow0 = 32 * wv;  // the wave's first row within the workgroup's rows
  const long layer_rows = (long)a.rows_T * a.Hkv;
  uint8_t *stage = (uint8_t *)(s_tab + had_table_floats(c.np)) + kHadStage * wv;
  // stage slot s = 64 j + lane (j < 5; the last load only in lanes < 32) holds chunk s % 9 of
  // the wave's row s / 9 (the ninth slot repeats chunk 7); rows past the layer's end load the
  // last live row, whose results are never stored
  had_load_rows((const int8_t *)a.k + c.row0 * 128, stage, threadIdx.x & 63, c.nrows, wrow0);
  hadamard_pair_table(a, c.pa, c.np, s_tab, dwt);
  const float *s_cm1 = s_tab, *s_sn = s_tab + had_off_sn(c.np), *s_nsn = s_tab + had_off_nsn(c.np);
  const uint32_t kbf = 0xffff0001u;
  // entering layer l: sco_a is its row scale and sco_b layer l + 1's, nxA holds layer l + 1's
  // rows and nxB takes layer l + 2's (rows past the layer's end lie beyond the resource's
  // extent and load zeros; their results are never stored)
  const int prow = min(wrow0 + (int)((threadIdx.x & 63) >> 1), c.nrows - 1);
  float sco_a = a.scale[c.row0 + prow], sco_b = 0.f;
  b128_t nxA[4], nxB[4];
  auto load_rows = [&](b128_t (&dst)[4], int layer) {
    const __amdgpu_buffer_rsrc_t rn = span_rsrc((int8_t *)a.k + (c.row0 + (long)layer * layer_rows) * 128, (long)c.nrows * 128);
    const int ln = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = __builtin_amdgcn_raw_buffer_load_b128(rn, (wrow0 + 8 * j + (ln >> 3)) * 128 + 16 * (ln & 7), 0, kStream);
  };
  if (c.nl > 1) {
    load_rows(nxA, 1);
    sco_b = a.scale[c.row0 + layer_rows + prow];
  }
  for (int l = 0; l < c.nl; ++l) {
    int lane = threadIdx.x & 63;
    __asm__ volatile("" : "+v"(lane));
    const long lrow = c.row0 + (long)l * layer_rows;  // the workgroup's first row in this layer
    // computing layout: lane l holds codes 32 q .. 32 q + 31 of each half of row rr = l / 2 (q = l % 2);
    // out = A x + B x' with x' the partner lane's value and (A, B) = (cm1, sn) on the lower lane
    // (x = s, x' = t) and (cm1, -sn) on the upper one (x = t, x' = s)
    const int rr = lane >> 1, q = lane & 1;
    const int row = wrow0 + rr;
    const bool live = row < c.nrows;
    const int tab = ((c.r0 + (live ? row : 0)) / a.Hkv - c.pa) * 36;
    const float *ta = s_cm1 + tab, *tb = (q ? s_nsn : s_sn) + tab;
    uint8_t *mine = stage + 16 * (9 * rr + 2 * q);
    const float sco = sco_a;
    sco_a = sco_b;
    if (l == 0) wait_vmcnt<0>();  // layer 0's rows came by direct loads
    if (l + 2 < c.nl) {
      load_rows(nxB, l + 2);
      sco_b = a.scale[lrow + 2 * layer_rows + (live ? row : 0)];
    }
    uint32_t w[16];  // words 0..7: codes 32 q + (0..31); 8..15: codes 64 + 32 q + (0..31)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *(const uint4 *)(mine + 16 * ((i & 1) + 4 * (i >> 1)));
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    // P[2 j + b] holds u[4 j + b] (low half) and u[4 j + 2 + b] (high half), u = c_lo + c_hi
    uint32_t P[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      P[2 * j] = add_bytes_02(w[j], w[8 + j]);
      P[2 * j + 1] = add_bytes_13(w[j], w[8 + j]);
    }
    // H32 over index bits 0, 2, 3, 4 (register index bits 0..3), then bit 1 inside the registers
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i & m) == 0) {
          const u16x2 x = as_u16x2(P[i]), y = as_u16x2(P[i | m]);
          P[i] = as_u32(x + y);
          P[i | m] = as_u32(x - y);
        }
#pragma unroll
    for (int i = 0; i < 16; ++i) P[i] = bfly_halves(P[i], kbf);
    float x[32];  // lower lane: s = H32 u[0..31]; upper lane: t = H32 u[32..63]
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t v = P[2 * (e >> 2) + (e & 1)];
      x[e] = (float)(short)(((e >> 1) & 1) ? (v >> 16) : (v & 0xffffu));
    }
    // the collapsed top stages and turn: lower lane cm1 s + sn t, upper lane cm1 t - sn s
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e0 = 0; e0 < 32; e0 += 8) {
      const float4 a0 = *(const float4 *)(ta + e0), a1 = *(const float4 *)(ta + e0 + 4);
      const float4 b0 = *(const float4 *)(tb + e0), b1 = *(const float4 *)(tb + e0 + 4);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = x[e0 + e] * av[e];
      fmac_partner8(o, x + e0, bv);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e0 + e] = o[e];
      __builtin_amdgcn_sched_barrier(0);
    }
    // H32 on each lane: x[e] = (H64 D)[32 q + e] / 2
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if ((j & h) == 0) {
          const float u = x[j], v = x[j + h];
          x[j] = u + v;
          x[j + h] = u - v;
        }
    // y / 2 = 64 c + x, in blocks behind scheduling fences so that each x dies as its two y are made
    float y[64];
    float amax = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e0 = 0; e0 < 32; e0 += 4) {
#pragma unroll
      for (int e = e0; e < e0 + 4; ++e) {
        y[e] = fmaf(code_at(w, e), 64.f, x[e]);
        y[32 + e] = fmaf(code_at(w, 32 + e), 64.f, x[e]);
        amax = fmaxf(fmaxf(amax, fabsf(y[e])), fabsf(y[32 + e]));  // one v_max3 per pair
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    amax = fmaxf(amax, dpp_xor1(amax));
    const float inv = amax > 0.f && sco > 0.f ? 127.0f / amax : 0.f;
    uint32_t out[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      out[i] = pack4_codes(code_fma(y[4 * i], inv), code_fma(y[4 * i + 1], inv), code_fma(y[4 * i + 2], inv),
                           code_fma(y[4 * i + 3], inv));
    // back into the same slots, then out by whole rows (lane l: row 8 j + l / 8, chunk l % 8)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(uint4 *)(mine + 16 * ((i & 1) + 4 * (i >> 1))) = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    __asm__ volatile("" ::: "memory");
    const __amdgpu_buffer_rsrc_t rs = span_rsrc((int8_t *)a.k + lrow * 128, (long)c.nrows * 128);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * j + (lane >> 3);
      const uint4 v = *(const uint4 *)(stage + 16 * (9 * r + (lane & 7)));
      b128_t o;
      o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
      // rows past the layer's end lie beyond the resource's extent: the store is dropped
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, (wrow0 + r) * 128 + 16 * (lane & 7), 0, kStream);
    }
    if (live && q == 0) a.scale[lrow + row] = inv > 0.f ? sco * amax * (1.0f / (127.0f * 64.0f)) : 0.f;
    if (l + 1 < c.nl) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stage has been read out
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *(uint4 *)(stage + 16 * (9 * (8 * j + (lane >> 3)) + (lane & 7))) = make_uint4(nxA[j][0], nxA[j][1], nxA[j][2], nxA[j][3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) nxA[j] = nxB[j];
    }
  }
}

// Uniform shift of cached keys by delta positions (local-position windows).
struct ShiftArgs {
  RopeParams p;
  int delta;
  void *k;
  int ring;          // 1: RING rows [B, Hkv, C], only valid ring slots move
  int Hkv, C, S, W;  // RING geometry
  const int32_t *head, *count;
  long rows;
  int D;
  float cs[256], sn[256];  // cos / sin of delta * w_i per rotary pair (fp64, rounded once), set on the host
};

template <typename T, int PP>
__global__ __launch_bounds__(256) void shift_kernel(ShiftArgs a) {
  constexpr int EB = sizeof(T);
  constexpr int NB = PP * EB;
  constexpr int NW = (NB + 3) / 4;
  const int half = a.p.rotary_dim / 2;
  const int tpr = half / PP;
  const long items = a.rows * tpr;
  const int neox = a.p.neox;
  char *kb = (char *)a.k;
  // one item per thread: read, turn and write back right away (the fastest in-place shape here)
  {
    const long it = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (it >= items) return;
    const long row = it / tpr;
    const int q = (int)(it - row * tpr);
    if (a.ring) {
      const int slot = (int)(row % a.C);
      const int b = (int)(row / a.C) / a.Hkv;
      if (slot < a.S) return;
      const int cnt = min(max(a.count[b], 0), a.W);
      int oldest = (a.head[b] - cnt) % a.W;
      if (oldest < 0) oldest += a.W;
      int rel = (slot - a.S - oldest) % a.W;
      if (rel < 0) rel += a.W;
      if (rel >= cnt) return;
    }
    const int j0 = q * PP;
    char *p1 = kb + (row * a.D + (neox ? j0 : 2 * j0)) * EB;
    char *p2 = neox ? kb + (row * a.D + half + j0) * EB : p1 + NB;
    uint32_t w1[NW], w2[NW];
    vld<NB>(w1, p1);
    vld<NB>(w2, p2);
    const float *cs = &a.cs[j0];
    const float *sn = &a.sn[j0];
    if constexpr (PP % 2 == 0) {
      if (neox) {
#pragma unroll
        for (int e = 0; e < PP; e += 2) {
          const float x1a = vget<T>(w1, e), x2a = vget<T>(w2, e);
          const float x1b = vget<T>(w1, e + 1), x2b = vget<T>(w2, e + 1);
          vput2<T>(w1, e, x1a * cs[e] - x2a * sn[e], x1b * cs[e + 1] - x2b * sn[e + 1]);
          vput2<T>(w2, e, x2a * cs[e] + x1a * sn[e], x2b * cs[e + 1] + x1b * sn[e + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < PP; ++e) {
          uint32_t *b = 2 * e < PP ? w1 : w2;
          const int i1 = 2 * e < PP ? 2 * e : 2 * e - PP;
          const float x1 = vget<T>(b, i1), x2 = vget<T>(b, i1 + 1);
          vput2<T>(b, i1, x1 * cs[e] - x2 * sn[e], x2 * cs[e] + x1 * sn[e]);
        }
      }
    } else {
      // PP = 1: the pair is element 0 of each half (NeoX) or of the two halves (GPT-J)
      const float x1 = vget<T>(w1, 0), x2 = vget<T>(w2, 0);
      vput<T>(w1, 0, x1 * cs[0] - x2 * sn[0]);
      vput<T>(w2, 0, x2 * cs[0] + x1 * sn[0]);
    }
    vst<NB>(p1, w1);
    vst<NB>(p2, w2);
  }
}

template <typename T>
hipError_t launch_shift_t(const ShiftArgs &a, hipStream_t s) {
  const int half = a.p.rotary_dim / 2;
  // 16-byte vectors only where every row starts on a 16-byte boundary
  const bool wide = half % (16 / (int)sizeof(T)) == 0 && (a.D * (int)sizeof(T)) % 16 == 0;
  const long items = a.rows * (wide ? half / (16 / (int)sizeof(T)) : half);
  const long blocks = (items + 255) / 256;
  if (blocks < 1) return hipSuccess;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  if (wide)
    hipLaunchKernelGGL((shift_kernel<T, 16 / sizeof(T)>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((shift_kernel<T, 1>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shift_keys(const RopeParams &p, const ropekv_kv_cache &c, int delta, int n_layers, hipStream_t s) {
  ShiftArgs a;
  a.p = p;
  a.delta = delta;
  a.k = c.k;
  a.ring = c.layout == ROPEKV_RING;
  a.Hkv = c.num_kv_heads;
  a.C = c.capacity;
  a.S = c.sinks;
  a.W = c.window;
  a.head = c.ring_head;
  a.count = c.ring_count;
  a.rows = a.ring ? (long)c.batch * c.num_kv_heads * c.capacity : (long)n_layers * c.capacity * c.num_kv_heads;
  a.D = c.head_dim;
  const int half = p.rotary_dim / 2;
  if (half > 256) return hipErrorInvalidValue;
  for (int i = 0; i < 256; ++i) {
    const double ang = i < half ? (double)delta * rope_omega(p, i) : 0.0;
    a.cs[i] = (float)cos(ang);
    a.sn[i] = (float)sin(ang);
  }
  switch (c.kv_dtype) {
    case ROPEKV_F32: return launch_shift_t<float>(a, s);
    case ROPEKV_BF16: return launch_shift_t<bf16_t>(a, s);
    case ROPEKV_F16: return launch_shift_t<f16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rerotate(const RopeParams &from, const RopeParams &to, const ropekv_kv_cache &c, int n_layers,
                           hipStream_t s) {
  RerotArgs a;
  a.from = from;
  a.to = to;
  a.k = c.k;
  a.scale = c.k_scale;
  a.rows_T = c.capacity;
  a.Hkv = c.num_kv_heads;
  a.D = c.head_dim;
  a.pos0 = c.pos0;
  a.n_layers = n_layers;
  a.keep_scale = (c.k_int8_mode & ROPEKV_I8_KEEP_SCALE) != 0;
  const int half = to.rotary_dim / 2;
  if (half > 256) return hipErrorInvalidValue;
  // per-pair frequency change and gain, fp64 on the host (the same formulas as the table kernel)
  a.gain = params_mscale(to) / params_mscale(from);
  for (int i = 0; i < 256; ++i) a.dw[i] = i < half ? rope_omega(to, i) - rope_omega(from, i) : 0.0;
  dim3 grid((c.capacity + kPT - 1) / kPT);
  // one-shot grids: rpb rows per workgroup, layer-major
  const long layer_rows = (long)c.capacity * c.num_kv_heads;
  const long max_rpb_chunks = ((layer_rows + 255) / 256) * 256;  // chunks of the smallest rpb, rounded up
  if (max_rpb_chunks * n_layers > 0x7fffffffL) return hipErrorInvalidValue;
  a.lg = 1;
  auto one_shot = [&](int rpb, size_t &shm1) -> dim3 {
    a.rpb = rpb;
    a.chunks = (int)((layer_rows + rpb - 1) / rpb);
    const int np = (rpb - 1) / a.Hkv + 2;  // positions a chunk of rpb rows can span
    shm1 = (size_t)np * half * 2 * sizeof(float);
    return dim3((unsigned)((long)a.chunks * ((n_layers + a.lg - 1) / a.lg)));
  };
  size_t shm1 = 0;
  // chunk kernels (one 16-byte chunk per thread) where the row shape allows them
  {
    auto pow2 = [](int x) { return x > 0 && (x & (x - 1)) == 0; };
    const bool nx = to.neox != 0;
    if (c.kv_dtype == ROPEKV_F16 || c.kv_dtype == ROPEKV_BF16 || c.kv_dtype == ROPEKV_F32) {
      const int eb = c.kv_dtype == ROPEKV_F32 ? 4 : 2;
      const int R = to.rotary_dim * eb / 16;
      // 16-byte chunks need rows that start on 16-byte boundaries (head_dim * eb a multiple of 16)
      if ((to.rotary_dim * eb) % 16 == 0 && (c.head_dim * eb) % 16 == 0 && pow2(R) && R >= 2 && R <= 32) {
        a.lg = 1;
        const dim3 g1 = one_shot(kFloatChunks * kChunkThreads / R, shm1);
        auto go = [&](auto tag, auto rtag) {
          using T = decltype(tag);
          constexpr int RR = decltype(rtag)::value, NC = kFloatChunks;
          if (nx) hipLaunchKernelGGL((rerotate_float_chunk_kernel<T, RR, NC, true>), g1, dim3(kChunkThreads), shm1, s, a);
          else hipLaunchKernelGGL((rerotate_float_chunk_kernel<T, RR, NC, false>), g1, dim3(kChunkThreads), shm1, s, a);
        };
        auto by_r = [&](auto tag) {
          switch (R) {
            case 2: go(tag, std::integral_constant<int, 2>()); break;
            case 4: go(tag, std::integral_constant<int, 4>()); break;
            case 8: go(tag, std::integral_constant<int, 8>()); break;
            case 16: go(tag, std::integral_constant<int, 16>()); break;
            default: go(tag, std::integral_constant<int, 32>()); break;
          }
        };
        if (c.kv_dtype == ROPEKV_F16) by_r(f16_t());
        else if (c.kv_dtype == ROPEKV_BF16) by_r(bf16_t());
        else by_r(float());
        return hipGetLastError();
      }
    } else if (c.kv_dtype == ROPEKV_I8 && !(c.k_int8_mode & ROPEKV_I8_HADAMARD)) {
      const int L = c.head_dim / 16, RC = to.rotary_dim / 16;
      if (a.keep_scale && c.head_dim % 32 == 0 && 2 * to.rotary_dim == c.head_dim && (L == 8 || L == 16)) {
        // keep-scale with the rotary slice half the row: one rotary and one tail chunk per lane
        // (measured on the 64-layer switch: 5.2 TB/s against 4.9 for the chunk kernel, which
        // stays ahead for the requantising turn, 5.6 against 5.3)
        a.lg = 1;
        const int H = L / 2;
        const dim3 g1 = one_shot(kI8HalfChunks * kChunkThreads / H, shm1);
        shm1 = shm1 / 2 * 3;  // cos, sin, -sin planes
        auto go = [&](auto htag) {
          constexpr int HH = decltype(htag)::value, NC = kI8HalfChunks;
          if (nx) hipLaunchKernelGGL((rerotate_int8_half_kernel<HH, NC, true, true>), g1, dim3(kChunkThreads), shm1, s, a);
          else hipLaunchKernelGGL((rerotate_int8_half_kernel<HH, NC, false, true>), g1, dim3(kChunkThreads), shm1, s, a);
        };
        if (H == 4) go(std::integral_constant<int, 4>());
        else go(std::integral_constant<int, 8>());
        return hipGetLastError();
      }
      const bool shape_ok = c.head_dim % 16 == 0 && (L == 4 || L == 8 || L == 16) && to.rotary_dim % 16 == 0 &&
                            (!nx || (RC % 2 == 0 && pow2(RC / 2)));
      if (shape_ok) {
        a.lg = 1;
        const dim3 g1 = one_shot(kI8Chunks * kChunkThreads / L, shm1);
        shm1 = shm1 / 2 * 3 + 32 * sizeof(float);  // cos, sin, -sin planes and the identity block
        const bool kp = a.keep_scale != 0;
        auto go = [&](auto ltag) {
          constexpr int LL = decltype(ltag)::value, NC = kI8Chunks;
          if (nx && kp) hipLaunchKernelGGL((rerotate_int8_chunk_kernel<LL, NC, true, true>), g1, dim3(kChunkThreads), shm1, s, a);
          else if (nx) hipLaunchKernelGGL((rerotate_int8_chunk_kernel<LL, NC, true, false>), g1, dim3(kChunkThreads), shm1, s, a);
          else if (kp) hipLaunchKernelGGL((rerotate_int8_chunk_kernel<LL, NC, false, true>), g1, dim3(kChunkThreads), shm1, s, a);
          else hipLaunchKernelGGL((rerotate_int8_chunk_kernel<LL, NC, false, false>), g1, dim3(kChunkThreads), shm1, s, a);
        };
        if (L == 4) go(std::integral_constant<int, 4>());
        else if (L == 8) go(std::integral_constant<int, 8>());
        else go(std::integral_constant<int, 16>());
        return hipGetLastError();
      }
    }
  }
  // the vector variants below move 16 bytes at a time: rows must start on 16-byte boundaries
  const bool rows16 = (c.head_dim * (c.kv_dtype == ROPEKV_F32 ? 4 : 2)) % 16 == 0;
  switch (c.kv_dtype) {
    case ROPEKV_I8: {
      if (c.k_int8_mode & ROPEKV_I8_HADAMARD) {
        if (c.head_dim == 128 && (!to.neox || to.rotary_dim == 64 || to.rotary_dim == 128)) {
          a.lg = kHadLayers;
          const dim3 g1 = one_shot(128, shm1);
          if (!to.neox && to.rotary_dim <= 64)
            hipLaunchKernelGGL(rerotate_int8_hadamard128_r64_kernel, g1, dim3(256), shm1, s, a);
          else if (!to.neox)
            hipLaunchKernelGGL(rerotate_int8_hadamard128_kernel<0>, g1, dim3(256), shm1, s, a);
          else if (to.rotary_dim == 64) {
            a.lg = kHadNeoxLayers;
            const dim3 g2 = one_shot(128, shm1);
            shm1 = sizeof(float) * had_table_floats((128 - 1) / c.num_kv_heads + 2) + 4 * kHadStage;  // table, four row stages
            hipLaunchKernelGGL(rerotate_int8_hadamard128_neox64_kernel, g2, dim3(256), shm1, s, a);
          }
          else
            hipLaunchKernelGGL(rerotate_int8_hadamard128_kernel<128>, g1, dim3(256), shm1, s, a);
        } else {
          hipLaunchKernelGGL(rerotate_int8_hadamard_kernel, grid, dim3(256), 0, s, a);
        }
        break;
      }
      // lane-local pairs when each lane's 16 codes split into whole pairs and tail: H = half / (D / 16)
      const int L = c.head_dim / 16;
      const int H = (half % L == 0) ? half / L : 0;
      const bool tail_ok = ((c.head_dim - to.rotary_dim) % L) == 0;
      const bool nx = to.neox != 0, kp = a.keep_scale != 0;
      if (tail_ok && (H == 8 || H == 4 || H == 2)) {
        a.lg = kI8Layers;
        const dim3 g1 = one_shot(kI8Threads / L, shm1);
        auto pick = [&](auto h) {
          constexpr int HH = decltype(h)::value;
          if (nx && kp) hipLaunchKernelGGL((rerotate_int8_lanes_kernel<HH, true, true>), g1, dim3(kI8Threads), shm1, s, a);
          else if (nx) hipLaunchKernelGGL((rerotate_int8_lanes_kernel<HH, true, false>), g1, dim3(kI8Threads), shm1, s, a);
          else if (kp) hipLaunchKernelGGL((rerotate_int8_lanes_kernel<HH, false, true>), g1, dim3(kI8Threads), shm1, s, a);
          else hipLaunchKernelGGL((rerotate_int8_lanes_kernel<HH, false, false>), g1, dim3(kI8Threads), shm1, s, a);
        };
        if (H == 8) pick(std::integral_constant<int, 8>());
        else if (H == 4) pick(std::integral_constant<int, 4>());
        else pick(std::integral_constant<int, 2>());
      } else {
        hipLaunchKernelGGL(rerotate_int8_kernel, grid, dim3(256), 0, s, a);
      }
      break;
    }
    case ROPEKV_F16:
      if (half % 8 == 0 && rows16) {
        const dim3 g1 = one_shot(256 / (half / 8), shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<f16_t, 8>), g1, dim3(256), shm1, s, a);
      } else {
        const dim3 g1 = one_shot(256 / half, shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<f16_t, 1>), g1, dim3(256), shm1, s, a);
      }
      break;
    case ROPEKV_BF16:
      if (half % 8 == 0 && rows16) {
        const dim3 g1 = one_shot(256 / (half / 8), shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<bf16_t, 8>), g1, dim3(256), shm1, s, a);
      } else {
        const dim3 g1 = one_shot(256 / half, shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<bf16_t, 1>), g1, dim3(256), shm1, s, a);
      }
      break;
    case ROPEKV_F32:
      if (half % 4 == 0 && rows16) {
        const dim3 g1 = one_shot(256 / (half / 4), shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<float, 4>), g1, dim3(256), shm1, s, a);
      } else {
        const dim3 g1 = one_shot(256 / half, shm1);
        hipLaunchKernelGGL((rerotate_float_kernel<float, 1>), g1, dim3(256), shm1, s, a);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ropekv
