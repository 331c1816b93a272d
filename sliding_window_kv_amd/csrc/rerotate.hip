// Re-rotation of cached keys at a YaRN factor switch.
//
// "#2961 rope: --rope-scaling dynamic" ("What it does": the cached keys
// follow a change) and "Attention Sink 与 Streaming KV Cache" (R_a R_b =
// R_{a+b}): a key stored as mu_A R(p w_A) k becomes mu_B R(p w_B) k after one
// more rotation of pair i by p (w_B,i - w_A,i) and a gain mu_B / mu_A.
//
// A workgroup owns PT consecutive positions and walks every layer and KV
// head at those positions, so the fp64 angle work (PT x r/2 sincos) is shared
// by n_layers x Hkv rows.  Float caches read and write only the rotary slice
// (the tail is never touched); int8 rows are read whole, dequantised, turned,
// and requantised with a fresh per-row scale.
#include "kernels.hpp"

namespace ropekv {

namespace {

constexpr int kPT = 16;  // positions per workgroup

struct RerotArgs {
  RopeParams from, to;
  void *k;
  float *scale;
  int rows_T;  // rows (positions) per layer
  int Hkv, D, pos0, n_layers;
};

// Fills s_cs / s_sn [kPT][half] with cos / sin of (pos) * (w_to - w_from) in
// fp64, rounded to fp32, and returns the gain mu_to / mu_from.
__device__ inline float angle_setup(const RerotArgs &a, int t0, float *s_cs, float *s_sn, double *s_dw) {
  const int half = a.to.rotary_dim / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) s_dw[i] = rope_omega(a.to, i) - rope_omega(a.from, i);
  __syncthreads();
  for (int idx = threadIdx.x; idx < kPT * half; idx += blockDim.x) {
    const int pt = idx / half, i = idx % half;
    const double ang = (double)(a.pos0 + t0 + pt) * s_dw[i];
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cs[idx] = (float)cs;
    s_sn[idx] = (float)sn;
  }
  __syncthreads();
  return (float)(rope_mscale(a.to.s) / rope_mscale(a.from.s));
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

// Float keys.  A thread turns PP consecutive pairs of one row: NeoX loads PP
// elements from each half, GPT-J 2 PP interleaved elements.
template <typename T, int PP>
__global__ __launch_bounds__(256) void rerotate_float_kernel(RerotArgs a) {
  constexpr int EB = sizeof(T);
  constexpr int NB = PP * EB;
  constexpr int NW = (NB + 3) / 4;
  __shared__ float s_cs[kPT * 256], s_sn[kPT * 256];
  __shared__ double s_dw[256];
  const int t0 = blockIdx.x * kPT;
  const float gain = angle_setup(a, t0, s_cs, s_sn, s_dw);
  const int half = a.to.rotary_dim / 2;
  const int tpr = half / PP;
  const int npos = min(kPT, a.rows_T - t0);
  const int items = npos * a.Hkv * tpr;
  const int neox = a.to.neox;
  const long layer_stride = (long)a.rows_T * a.Hkv * a.D;
  char *kb = (char *)a.k;
  for (int layer = 0; layer < a.n_layers; ++layer) {
    const long lbase = layer * layer_stride + (long)t0 * a.Hkv * a.D;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      const int rr = it / tpr, q = it % tpr;
      const int pt = rr / a.Hkv;
      const long rbase = lbase + (long)rr * a.D;
      const int j0 = q * PP;
      const float *cs = &s_cs[pt * half + j0];
      const float *sn = &s_sn[pt * half + j0];
      if (neox) {
        uint32_t w1[NW], w2[NW];
        char *p1 = kb + (rbase + j0) * EB;
        char *p2 = kb + (rbase + half + j0) * EB;
        vld<NB>(w1, p1);
        vld<NB>(w2, p2);
#pragma unroll
        for (int u = 0; u < PP; ++u) {
          const float x1 = vget<T>(w1, u), x2 = vget<T>(w2, u);
          vput<T>(w1, u, (x1 * cs[u] - x2 * sn[u]) * gain);
          vput<T>(w2, u, (x2 * cs[u] + x1 * sn[u]) * gain);
        }
        vst<NB>(p1, w1);
        vst<NB>(p2, w2);
      } else {
        uint32_t w[2 * NW];
        char *p = kb + (rbase + 2 * j0) * EB;
        vld<NB>(w, p);
        vld<NB>(w + NW, p + NB);
#pragma unroll
        for (int u = 0; u < PP; ++u) {
          // element 2u sits at w[...] in the first NB bytes when 2u < PP, else in the second
          const int e1 = 2 * u, e2 = 2 * u + 1;
          uint32_t *b1 = e1 < PP ? w : w + NW;
          uint32_t *b2 = e2 < PP ? w : w + NW;
          const int i1 = e1 < PP ? e1 : e1 - PP, i2 = e2 < PP ? e2 : e2 - PP;
          const float x1 = vget<T>(b1, i1), x2 = vget<T>(b2, i2);
          vput<T>(b1, i1, (x1 * cs[u] - x2 * sn[u]) * gain);
          vput<T>(b2, i2, (x2 * cs[u] + x1 * sn[u]) * gain);
        }
        vst<NB>(p, w);
        vst<NB>(p + NB, w + NW);
      }
    }
  }
}

// int8 keys with a per-row fp32 scale.  LPR = D / 16 lanes per row, each
// holding 16 consecutive codes; NeoX partners sit half / 16 lanes apart and
// are exchanged by shuffles.
__global__ __launch_bounds__(256) void rerotate_int8_kernel(RerotArgs a) {
  __shared__ float s_cs[kPT * 256], s_sn[kPT * 256];
  __shared__ double s_dw[256];
  const int t0 = blockIdx.x * kPT;
  const float gain = angle_setup(a, t0, s_cs, s_sn, s_dw);
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
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(y[e]));
      for (int m = lpr >> 1; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      const float sc_new = amax / 127.0f;
      uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float qv = 0.f;
        if (sc_new > 0.f) qv = fminf(fmaxf(rintf(y[e] / sc_new), -127.f), 127.f);
        out[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)qv) << (8 * (e & 3));
      }
      if (live) {
        *(uint4 *)(kc + row * a.D + q * 16) = make_uint4(out[0], out[1], out[2], out[3]);
        if (q == 0) a.scale[row] = sc_new;
      }
    }
  }
}

}  // namespace

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
  dim3 grid((c.capacity + kPT - 1) / kPT);
  const int half = to.rotary_dim / 2;
  switch (c.kv_dtype) {
    case ROPEKV_I8: hipLaunchKernelGGL(rerotate_int8_kernel, grid, dim3(256), 0, s, a); break;
    case ROPEKV_F16:
      if (half % 8 == 0)
        hipLaunchKernelGGL((rerotate_float_kernel<f16_t, 8>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((rerotate_float_kernel<f16_t, 1>), grid, dim3(256), 0, s, a);
      break;
    case ROPEKV_BF16:
      if (half % 8 == 0)
        hipLaunchKernelGGL((rerotate_float_kernel<bf16_t, 8>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((rerotate_float_kernel<bf16_t, 1>), grid, dim3(256), 0, s, a);
      break;
    case ROPEKV_F32:
      if (half % 4 == 0)
        hipLaunchKernelGGL((rerotate_float_kernel<float, 4>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((rerotate_float_kernel<float, 1>), grid, dim3(256), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ropekv
