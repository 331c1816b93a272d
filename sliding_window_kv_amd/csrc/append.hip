// Fused RoPE apply + KV append.
//
// "RoPE, scaling, sliding window, attention sinks" (the attention block and
// "Where the positions come from"): rotate q and k in place by the table row
// of the token's position, never v, and write the rotated k with the raw v
// to the cache slot derived from the same position.  Ring rules from
// "Inference & 128K Long Context" (ring buffer; 5.2 append); paged freeing
// from the null-block loop and window edge of the first page.
//
// Launch 1 (one workgroup per token) rotates and writes; it reads the cache
// state (seq_len, ring head/count) as it stood before the call.  Launch 2
// (one thread per token) lets the last token of each sequence's run advance
// that state and free expired blocks, so no thread reads state another one
// is changing.
#include "kernels.hpp"

namespace ropekv {

// 0 if token t (position p of sequence seq, whose cache held nb tokens) is in
// a run of consecutive positions that starts at nb; else an error bit.
__device__ inline int token_check(const AppendArgs &a, int t, int p, int seq, int nb) {
  const int off = p - nb;
  if (off < 0 || off > t) return ROPEKV_DEV_POSITION;
  const int t0 = t - off;
  if (a.seq[t0] != seq || a.pos[t0] != nb) return ROPEKV_DEV_POSITION;
  if (t0 > 0 && a.seq[t0 - 1] == seq) return ROPEKV_DEV_POSITION;
  if (t > t0 && (a.seq[t - 1] != seq || a.pos[t - 1] != p - 1)) return ROPEKV_DEV_POSITION;
  return 0;
}

// Index of the last token of t's run (runs are consecutive): the call's last token when
// the run reaches it (one chunk of one sequence), else a binary search.
__device__ inline int run_last(const AppendArgs &a, int t, int p, int seq) {
  const int tl = a.n_tokens - 1;
  if (a.seq[tl] == seq && a.pos[tl] == p + (tl - t)) return tl;
  int lo = t, hi = a.n_tokens;
  while (hi - lo > 1) {
    const int mid = lo + ((hi - lo) >> 1);
    if (a.seq[mid] == seq && a.pos[mid] == p + (mid - t))
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// One 8-bit code of the quotient y = x / scale, scale = max|x| / qmax (qmax 127
// for int8, 448 for E4M3; both IEEE fp32 divisions): int8 rounds to nearest
// even and clamps to [-127, 127]; E4M3 clamps to [-448, 448] and takes the
// nearest code, ties to even, by the hardware's fp32 -> fp8 conversion (the
// OCP format on this chip).
__device__ __forceinline__ uint8_t code8(float y, int kvdt) {
  if (kvdt == ROPEKV_FP8)
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(y, -448.f), 448.f), 0.f, 0, false) & 0xff);
  return (uint8_t)(int8_t)fminf(fmaxf(rintf(y), -127.f), 127.f);
}

__device__ __forceinline__ int mod_pos(long x, int m) {
  long r = x % m;
  return (int)(r < 0 ? r + m : r);
}

// 16-byte unit of T values <-> fp32
template <typename T>
__device__ __forceinline__ float unit_get(const uint4 &u, int e) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(w[e]);
  } else {
    const uint16_t h = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    return __is_same(T, bf16_t) ? bf16_to_f(h) : f16_to_f(h);
  }
}
template <typename T>
__device__ __forceinline__ uint4 unit_pack(const float *y) {
  uint32_t w[4];
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(y[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __is_same(T, bf16_t) ? pack2_bf16_rne(y[2 * i], y[2 * i + 1]) : pack2_f16_rne(y[2 * i], y[2 * i + 1]);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The vector path of one token: every thread of the workgroup takes 16-byte units
// (NeoX: a unit of each half; GPT-J: a unit of interleaved pairs; k tail and v units
// are copies), rotating q and k in place and writing k and v to the cache row.
template <typename T>
__device__ __forceinline__ void append_units(const AppendArgs &a, int t, const float *trow, bool write, long base,
                                             long hstride) {
  constexpr int PP = 16 / (int)sizeof(T);
  const ropekv_kv_cache &c = a.c;
  const int d = a.head_dim, r = a.rotary_dim, half = r / 2;
  const int Hkv = c.num_kv_heads, nq = a.n_q_heads;
  const int iq = a.neox ? half / PP : r / PP;  // rotation items per row
  const int tu = (d - r) / PP, du = d / PP;
  const int nqi = nq * iq, nki = Hkv * (iq + tu);
  const int nvi = (write && a.v != nullptr && c.v != nullptr) ? Hkv * du : 0;
  const int total = nqi + nki + nvi;
  for (int it = threadIdx.x; it < total; it += blockDim.x) {
    if (it < nqi + nki) {
      const bool is_k = it >= nqi;
      const int kk = is_k ? it - nqi : it;
      const int per = is_k ? iq + tu : iq;
      const int h = kk / per, j = kk - h * per;
      char *x = (char *)(is_k ? a.k : a.q) + ((long)t * (is_k ? Hkv : nq) + h) * d * (long)sizeof(T);
      char *cd = (write && is_k) ? (char *)c.k + (base + (long)h * hstride) * (long)sizeof(T) : nullptr;
      if (j < iq) {
        if (a.neox) {
          const int e0 = j * PP;
          uint4 *p1 = (uint4 *)(x + e0 * sizeof(T));
          uint4 *p2 = (uint4 *)(x + (half + e0) * sizeof(T));
          const uint4 u1 = *p1, u2 = *p2;
          float y1[PP], y2[PP];
#pragma unroll
          for (int e = 0; e < PP; ++e) {
            const float x1 = unit_get<T>(u1, e), x2 = unit_get<T>(u2, e);
            const float cs = trow[e0 + e], sn = trow[half + e0 + e];
            y1[e] = x1 * cs - x2 * sn;
            y2[e] = x2 * cs + x1 * sn;
          }
          const uint4 o1 = unit_pack<T>(y1), o2 = unit_pack<T>(y2);
          *p1 = o1;
          *p2 = o2;
          if (cd) {
            *(uint4 *)(cd + e0 * sizeof(T)) = o1;
            *(uint4 *)(cd + (half + e0) * sizeof(T)) = o2;
          }
        } else {
          const int e0 = j * PP;  // elements e0 .. e0 + PP - 1 = pairs e0 / 2 ..
          uint4 *p = (uint4 *)(x + e0 * sizeof(T));
          const uint4 u = *p;
          float y[PP];
#pragma unroll
          for (int e = 0; e < PP / 2; ++e) {
            const float x1 = unit_get<T>(u, 2 * e), x2 = unit_get<T>(u, 2 * e + 1);
            const int pi = e0 / 2 + e;
            const float cs = trow[pi], sn = trow[half + pi];
            y[2 * e] = x1 * cs - x2 * sn;
            y[2 * e + 1] = x2 * cs + x1 * sn;
          }
          const uint4 o = unit_pack<T>(y);
          *p = o;
          if (cd) *(uint4 *)(cd + e0 * sizeof(T)) = o;
        }
      } else if (cd) {  // tail unit of a k row: unchanged, copied to the cache
        const int e0 = r + (j - iq) * PP;
        *(uint4 *)(cd + e0 * sizeof(T)) = *(const uint4 *)(x + e0 * sizeof(T));
      }
    } else {
      const int kk = it - nqi - nki;
      const int h = kk / du, j = kk - h * du;
      const char *vr = (const char *)a.v + ((long)t * Hkv + h) * d * (long)sizeof(T);
      char *cd = (char *)c.v + (base + (long)h * hstride) * (long)sizeof(T);
      *(uint4 *)(cd + j * 16) = *(const uint4 *)(vr + j * 16);
    }
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ float rowbuf[4][512];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const ropekv_kv_cache &c = a.c;
  const int p = a.pos[t];
  if (p < 0 || p >= a.table_len) {
    if (threadIdx.x == 0) dev_error(c.err_word, ROPEKV_DEV_TABLE_RANGE);
    return;
  }
  const int d = a.head_dim;
  const int Hkv = c.num_kv_heads;
  int err = 0;
  bool write = true;
  long base = 0, hstride = 0;
  if (c.layout == ROPEKV_CONTIG) {
    const long row = (long)p - c.pos0;
    if (row < 0 || row >= c.capacity) {
      write = false;
      err = ROPEKV_DEV_BLOCK_RANGE;
    } else {
      base = row * Hkv * d;
      hstride = d;
    }
  } else {
    const int seq = a.seq[t];
    if (seq < 0 || seq >= c.batch) {
      write = false;
      err = ROPEKV_DEV_SEQ_RANGE;
    } else {
      const int nb = c.seq_len[seq];
      err = token_check(a, t, p, seq, nb);
      if (err) {
        write = false;
      } else if (c.layout == ROPEKV_RING) {
        const int S = c.sinks, W = c.window, C = c.capacity;
        int slot = -1;
        if (p < S) {
          slot = p;
        } else {
          const int n_after = p + (run_last(a, t, p, seq) - t) + 1;
          const int hb = mod_pos(c.ring_head[seq], W);
          const int cb = c.ring_count[seq];
          const int first = nb > S ? nb : S;  // first non-sink position of this run
          const int kprime = n_after - first;
          if (p >= n_after - W) {  // survives the chunk
            if (cb == 0 && kprime >= W)
              slot = S + (p - (n_after - W));
            else
              slot = S + mod_pos((long)hb + (p - first), W);
          }
        }
        if (slot < 0) {
          write = false;
        } else {
          base = ((long)seq * Hkv * C + slot) * d;
          hstride = (long)C * d;
        }
      } else {  // PAGED
        const int bs = c.block_size;
        const int blk = p / bs;
        if (blk >= c.max_blocks) {
          write = false;
          err = ROPEKV_DEV_BLOCK_RANGE;
        } else {
          const int bid = c.block_table[(long)seq * c.max_blocks + blk];
          if (bid < 0 || bid >= c.num_blocks) {
            write = false;
            err = ROPEKV_DEV_NULL_BLOCK;
          } else {
            base = ((long)bid * Hkv * bs + (p % bs)) * d;
            hstride = (long)bs * d;
          }
        }
      }
    }
  }
  if (err && threadIdx.x == 0) dev_error(c.err_word, err);

  const int r = a.rotary_dim;
  const int half = r >> 1;
  const float *trow = a.table + (long)p * r;
  const int nq = a.n_q_heads;
  const int act = a.act;
  const int kvdt = c.kv_dtype;
  const bool q8 = kvdt == ROPEKV_I8 || kvdt == ROPEKV_FP8;  // codes + per-row scale
  const float qmax = kvdt == ROPEKV_FP8 ? 448.f : 127.f;
  if (a.vec) {
    if (act == ROPEKV_BF16) append_units<bf16_t>(a, t, trow, write, base, hstride);
    else if (act == ROPEKV_F16) append_units<f16_t>(a, t, trow, write, base, hstride);
    else append_units<float>(a, t, trow, write, base, hstride);
    return;
  }
  const int n_rows = nq + 2 * Hkv;
  for (int row = wave; row < n_rows; row += 4) {
    if (row < nq + Hkv) {
      const bool is_k = row >= nq;
      const int h = is_k ? row - nq : row;
      void *x = is_k ? a.k : a.q;
      const long xoff = ((long)t * (is_k ? Hkv : nq) + h) * d;
      const bool to_cache = is_k && write;
      const long coff = base + (long)h * hstride;
      for (int j = lane; j < half; j += 64) {
        const int i1 = a.neox ? j : 2 * j;
        const int i2 = a.neox ? j + half : 2 * j + 1;
        const float x1 = load_elem(x, xoff + i1, act);
        const float x2 = load_elem(x, xoff + i2, act);
        const float cs = trow[j];
        const float sn = trow[half + j];
        const float o1 = x1 * cs - x2 * sn;
        const float o2 = x2 * cs + x1 * sn;
        store_elem(x, xoff + i1, act, o1);
        store_elem(x, xoff + i2, act, o2);
        if (to_cache) {
          if (q8) {
            rowbuf[wave][i1] = o1;
            rowbuf[wave][i2] = o2;
          } else {
            store_elem(c.k, coff + i1, kvdt, o1);
            store_elem(c.k, coff + i2, kvdt, o2);
          }
        }
      }
      if (to_cache) {
        for (int e = r + lane; e < d; e += 64) {
          const float val = load_elem(x, xoff + e, act);
          if (q8)
            rowbuf[wave][e] = val;
          else
            store_elem(c.k, coff + e, kvdt, val);
        }
        if (q8) {
          wave_lds_sync();
          if (c.k_int8_mode & ROPEKV_I8_HADAMARD) {
            // Hadamard-rotated storage: the row becomes H k (orthonormal Walsh-Hadamard,
            // butterflies over pairs (j, j + h) for h = 1, 2, 4, ... < d), then is quantised
            float *x = rowbuf[wave];
            for (int h = 1; h < d; h <<= 1) {
              for (int bf = lane; bf < d / 2; bf += 64) {
                const int j = (bf / h) * 2 * h + (bf % h);
                const float u = x[j], w = x[j + h];
                x[j] = u + w;
                x[j + h] = u - w;
              }
              wave_lds_sync();
            }
            const float norm = 1.0f / sqrtf((float)d);
            for (int e = lane; e < d; e += 64) x[e] *= norm;
            wave_lds_sync();
          }
          // per-row symmetric codes: scale = max|x| / qmax, code = code8(x / scale)
          float amax = 0.f;
          for (int e = lane; e < d; e += 64) amax = fmaxf(amax, fabsf(rowbuf[wave][e]));
          for (int m = 32; m >= 1; m >>= 1) amax = wave_max_xor(amax, m);
          const float scale = amax / qmax;
          uint8_t *kc = (uint8_t *)c.k;
          for (int e = lane; e < d; e += 64)
            kc[coff + e] = code8(scale > 0.f ? rowbuf[wave][e] / scale : 0.f, kvdt);
          if (lane == 0) c.k_scale[coff / d] = scale;
          wave_lds_sync();
        }
      }
    } else {
      const int h = row - nq - Hkv;
      if (write && a.v != nullptr && c.v != nullptr) {
        const long voff = ((long)t * Hkv + h) * d;
        const long coff = base + (long)h * hstride;
        if (q8) {
          // values: the same per-row quantiser as the keys, scale in v_scale
          float amax = 0.f;
          for (int e = lane; e < d; e += 64) {
            const float val = load_elem(a.v, voff + e, act);
            rowbuf[wave][e] = val;
            amax = fmaxf(amax, fabsf(val));
          }
          for (int m = 32; m >= 1; m >>= 1) amax = wave_max_xor(amax, m);
          wave_lds_sync();
          const float scale = amax / qmax;
          uint8_t *vc = (uint8_t *)c.v;
          for (int e = lane; e < d; e += 64)
            vc[coff + e] = code8(scale > 0.f ? rowbuf[wave][e] / scale : 0.f, kvdt);
          if (lane == 0) c.v_scale[coff / d] = scale;
          wave_lds_sync();
        } else {
          for (int e = lane; e < d; e += 64) store_elem(c.v, coff + e, kvdt, load_elem(a.v, voff + e, act));
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void append_state_kernel(AppendArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n_tokens) return;
  const ropekv_kv_cache &c = a.c;
  const int p = a.pos[t];
  const int seq = a.seq[t];
  if (p < 0 || p >= a.table_len || seq < 0 || seq >= c.batch) return;
  const bool last = (t == a.n_tokens - 1) || a.seq[t + 1] != seq || a.pos[t + 1] != p + 1;
  if (!last) return;
  const int nb = c.seq_len[seq];
  if (token_check(a, t, p, seq, nb)) return;
  const int na = p + 1;
  if (c.layout == ROPEKV_RING) {
    const int S = c.sinks, W = c.window;
    const int first = nb > S ? nb : S;
    const int kp = na - first;
    if (kp > 0) {
      const int hb = mod_pos(c.ring_head[seq], W);
      const int cb = c.ring_count[seq];
      if (cb == 0 && kp >= W) {
        c.ring_head[seq] = 0;
        c.ring_count[seq] = W;
      } else {
        c.ring_head[seq] = mod_pos((long)hb + kp, W);
        c.ring_count[seq] = (cb + kp < W) ? cb + kp : W;
      }
    }
  } else if (c.layout == ROPEKV_PAGED && c.window > 0 && a.freed != nullptr) {
    const int bs = c.block_size;
    const int e = nb - c.window + 1 > 0 ? nb - c.window + 1 : 0;
    const int last_block = (e / bs < c.max_blocks) ? e / bs : c.max_blocks;
    const int first_block = (c.sinks + bs - 1) / bs;
    int32_t *row = c.block_table + (long)seq * c.max_blocks;
    int cnt = 0;
    for (int j = last_block - 1; j >= first_block; --j) {
      if (row[j] == -1) break;
      ++cnt;
    }
    if (cnt > 0) {
      const int at = atomicAdd(a.n_freed, cnt);
      if (at + cnt > a.freed_cap) {
        dev_error(c.err_word, ROPEKV_DEV_FREE_OVERFLOW);
      } else {
        int j = last_block - 1;
        for (int i = 0; i < cnt; ++i, --j) {
          a.freed[at + i] = row[j];
          row[j] = -1;
        }
      }
    }
  }
  c.seq_len[seq] = na;
}

hipError_t launch_apply_append(const AppendArgs &a, hipStream_t s) {
  if (a.n_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(a.n_tokens), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.c.layout != ROPEKV_CONTIG) {
    hipLaunchKernelGGL(append_state_kernel, dim3((a.n_tokens + 255) / 256), dim3(256), 0, s, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ropekv
