// Device helpers shared by the ropekv HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ropekv.h"

namespace ropekv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bfloat16 / half stored as raw bits so the arithmetic is always fp32.
struct bf16_t { uint16_t x; };
struct f16_t { uint16_t x; };

__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (hardware conversion).
__device__ __forceinline__ uint16_t f_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float f16_to_f(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}
// fp32 -> half, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f_to_f16(float f) {
  _Float16 v = (_Float16)f;
  return __builtin_bit_cast(uint16_t, v);
}

// Two fp32 -> one word of two 16-bit values (lo in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16_rne(float lo, float hi) {
  typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2v_t));
}
__device__ __forceinline__ uint32_t pack2_f16_rne(float lo, float hi) {
  typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2v_t));
}

// element load/store by runtime dtype code (used off the hot loops)
__device__ __forceinline__ float load_elem(const void *p, long i, int dt) {
  switch (dt) {
    case ROPEKV_F32: return ((const float *)p)[i];
    case ROPEKV_BF16: return bf16_to_f(((const uint16_t *)p)[i]);
    case ROPEKV_F16: return f16_to_f(((const uint16_t *)p)[i]);
    default: return (float)((const int8_t *)p)[i];
  }
}
__device__ __forceinline__ void store_elem(void *p, long i, int dt, float v) {
  switch (dt) {
    case ROPEKV_F32: ((float *)p)[i] = v; break;
    case ROPEKV_BF16: ((uint16_t *)p)[i] = f_to_bf16(v); break;
    case ROPEKV_F16: ((uint16_t *)p)[i] = f_to_f16(v); break;
    default: break;
  }
}

// Rope parameters as passed to kernels.
struct RopeParams {
  double theta, s, beta_fast, beta_slow, ef, lff, hff;
  int rotary_dim, head_dim, neox, L0, type, pruned, served;
};

__host__ inline RopeParams make_rope_params(const ropekv_rope_cfg &c) {
  RopeParams p;
  p.theta = c.rope_theta;
  p.s = c.yarn_factor;
  p.beta_fast = c.beta_fast;
  p.beta_slow = c.beta_slow;
  p.ef = c.extrapolation_factor;
  p.lff = c.low_freq_factor;
  p.hff = c.high_freq_factor;
  p.rotary_dim = c.rotary_dim;
  p.head_dim = c.head_dim;
  p.neox = c.neox;
  p.L0 = c.orig_max_pos;
  p.type = c.rope_type;
  p.pruned = c.pruned_pairs;
  p.served = c.served_len;
  return p;
}

__host__ __device__ inline double yarn_omega(const RopeParams &p, int i);

// Angular frequency of pair i under the configured scheme, fp64.
__host__ __device__ inline double rope_omega(const RopeParams &p, int i) {
  if (i < p.pruned) return 0.0;
  const double r = (double)p.rotary_dim;
  const double e = (2.0 * (double)i) / r;
  switch (p.type) {
    case ROPEKV_ROPE_LINEAR: return 1.0 / pow(p.theta, e) / p.s;
    case ROPEKV_ROPE_NTK: return 1.0 / pow(p.theta * pow(p.s, r / (r - 2.0)), e);
    case ROPEKV_ROPE_DYNAMIC_NTK: {
      const double base = p.theta * pow(p.s * (double)p.served / (double)p.L0 - (p.s - 1.0), r / (r - 2.0));
      return 1.0 / pow(base, e);
    }
    case ROPEKV_ROPE_LLAMA3: {
      const double w = 1.0 / pow(p.theta, e);
      const double wavelen = 6.283185307179586476925286766559 / w;
      const double L0 = (double)p.L0;
      if (wavelen < L0 / p.hff) return w;
      if (wavelen > L0 / p.lff) return w / p.s;
      const double smooth = (L0 / wavelen - p.lff) / (p.hff - p.lff);
      return (1.0 - smooth) * w / p.s + smooth * w;
    }
    default: return yarn_omega(p, i);
  }
}

__host__ __device__ inline double rope_mscale(double s);
__host__ __device__ inline double params_mscale(const RopeParams &p) { return p.type == ROPEKV_ROPE_YARN ? rope_mscale(p.s) : 1.0; }

// YaRN frequency of pair i (plain RoPE when s <= 1).
__host__ __device__ inline double yarn_omega(const RopeParams &p, int i) {
  const double r = (double)p.rotary_dim;
  const double pos_freq = pow(p.theta, (2.0 * (double)i) / r);
  const double ext = 1.0 / pos_freq;
  if (!(p.s > 1.0)) return ext;
  const double interp = 1.0 / (p.s * pos_freq);
  const double two_pi = 6.283185307179586476925286766559;
  const double dlow = r * log((double)p.L0 / (p.beta_fast * two_pi)) / (2.0 * log(p.theta));
  const double dhigh = r * log((double)p.L0 / (p.beta_slow * two_pi)) / (2.0 * log(p.theta));
  double low = fmax(floor(dlow), 0.0);
  double high = fmin(ceil(dhigh), r - 1.0);
  if (low == high) high += 0.001;
  double ramp = ((double)i - low) / (high - low);
  ramp = fmin(fmax(ramp, 0.0), 1.0);
  const double mask = (1.0 - ramp) * p.ef;
  return interp * (1.0 - mask) + ext * mask;
}

__host__ __device__ inline double rope_mscale(double s) { return s > 1.0 ? 0.1 * log(s) + 1.0 : 1.0; }

__device__ __forceinline__ void dev_error(int32_t *err, int bit) {
  if (err) atomicOr(err, bit);
}

// Wait for this wave's LDS traffic and keep the compiler from moving memory
// operations across the point: lanes of one wave may then read what other
// lanes of the same wave wrote.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask)); }

// max / sum of a value over lanes l and l ^ 16 (l ^ 32) by the gfx950 lane swaps, no LDS
// round trip: with the same value in both operands the two results are v[l] and v[l ^ 16]
// (v[l ^ 32]) in some order, which is all a symmetric reduction needs.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Direct global -> LDS loads: the 64 lanes' N-byte reads land at LDS [m0 + N * lane]
// (m0 = the wave-uniform LDS base).  Issued as inline assembly so the compiler adds
// no waits of its own on them: callers wait with wait_vmcnt before reading the LDS
// they fill, and never fill a buffer that is still being read.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// lds_base must be the same for every lane of the wave (it is taken from the first lane).
__device__ __forceinline__ void dma16(const void *gsrc, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m0)
                   : "memory", "m0");
}
// The same with a wave-uniform 64-bit base (an SGPR pair) and a 32-bit per-lane byte offset:
// no per-lane address arithmetic when only the base moves.
__device__ __forceinline__ void dma16_so(const void *sbase, uint32_t voff, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                   : "memory", "m0");
}
// The same for data read once (decode K / V tiles): the load streams past the caches
// (sc0 sc1 nt), which on this part raises the rate of the 8-bit decode's loads by an eighth.
__device__ __forceinline__ void dma16_stream(const void *gsrc, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc0 sc1 nt" ::"v"(gsrc), "s"(m0)
                   : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *gsrc, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(m0)
                   : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
  __asm__ volatile("" ::: "memory");
}

}  // namespace ropekv
