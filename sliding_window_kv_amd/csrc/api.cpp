// C ABI of libropekv.so: host-side validation, then launches on the caller's
// stream.  Nothing here allocates device memory or synchronises the host.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "kernels.hpp"

using namespace ropekv;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return ROPEKV_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(ROPEKV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int check_rope(const ropekv_rope_cfg *c, const char *name) {
  if (!c) return fail(ROPEKV_EINVAL, "%s is NULL", name);
  if (c->rotary_dim < 2 || (c->rotary_dim & 1) || c->rotary_dim > 512)
    return fail(ROPEKV_EINVAL, "%s: rotary_dim %d must be even and in [2, 512]", name, c->rotary_dim);
  if (c->head_dim < c->rotary_dim)
    return fail(ROPEKV_EINVAL, "%s: rotary_dim %d exceeds head_dim %d", name, c->rotary_dim, c->head_dim);
  if (!(c->rope_theta > 1.0) || !isfinite(c->rope_theta))
    return fail(ROPEKV_EINVAL, "%s: rope_theta must be finite and > 1", name);
  if (!isfinite(c->yarn_factor)) return fail(ROPEKV_EINVAL, "%s: yarn_factor must be finite", name);
  if (c->rope_type < ROPEKV_ROPE_YARN || c->rope_type > ROPEKV_ROPE_LLAMA3)
    return fail(ROPEKV_EINVAL, "%s: unknown rope_type %d", name, c->rope_type);
  if (c->pruned_pairs < 0 || c->pruned_pairs > c->rotary_dim / 2)
    return fail(ROPEKV_EINVAL, "%s: pruned_pairs must be in [0, r/2]", name);
  const double s = c->yarn_factor;
  switch (c->rope_type) {
    case ROPEKV_ROPE_YARN:
      if (s > 1.0) {
        if (c->orig_max_pos < 1) return fail(ROPEKV_EINVAL, "%s: orig_max_pos must be >= 1 with yarn", name);
        if (!(c->beta_fast > 0.0) || !(c->beta_slow > 0.0))
          return fail(ROPEKV_EINVAL, "%s: beta_fast and beta_slow must be > 0", name);
        if (!isfinite(c->extrapolation_factor)) return fail(ROPEKV_EINVAL, "%s: extrapolation_factor", name);
      }
      break;
    case ROPEKV_ROPE_LINEAR:
    case ROPEKV_ROPE_NTK:
      if (!(s > 0.0)) return fail(ROPEKV_EINVAL, "%s: the scaling factor must be > 0", name);
      if (c->rope_type == ROPEKV_ROPE_NTK && c->rotary_dim < 4) return fail(ROPEKV_EINVAL, "%s: NTK needs r >= 4", name);
      break;
    case ROPEKV_ROPE_DYNAMIC_NTK:
      if (!(s > 0.0) || c->served_len < 1 || c->orig_max_pos < 1 || c->rotary_dim < 4)
        return fail(ROPEKV_EINVAL, "%s: dynamic NTK needs s > 0, served_len >= 1, orig_max_pos >= 1, r >= 4", name);
      if (!(s * (double)c->served_len / (double)c->orig_max_pos - (s - 1.0) > 0.0))
        return fail(ROPEKV_EINVAL, "%s: dynamic NTK base factor s P / L0 - (s - 1) must be > 0", name);
      break;
    case ROPEKV_ROPE_LLAMA3:
      if (!(s > 0.0) || c->orig_max_pos < 1 || !(c->low_freq_factor > 0.0) ||
          !(c->high_freq_factor > c->low_freq_factor))
        return fail(ROPEKV_EINVAL, "%s: Llama-3 needs s > 0, orig_max_pos >= 1, 0 < low < high freq factor", name);
      break;
  }
  return ROPEKV_OK;
}

// The kernels move cache rows, scales, queries and outputs with 16-byte vector accesses.
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int dt) {
  return dt == ROPEKV_F32 || dt == ROPEKV_BF16 || dt == ROPEKV_F16 || dt == ROPEKV_I8 || dt == ROPEKV_FP8;
}

// 8-bit caches: codes plus one fp32 scale per row
bool coded8(int dt) { return dt == ROPEKV_I8 || dt == ROPEKV_FP8; }

int check_cache(const ropekv_kv_cache *c) {
  if (!c) return fail(ROPEKV_EINVAL, "cache is NULL");
  if (!valid_dtype(c->kv_dtype)) return fail(ROPEKV_EDTYPE, "unknown kv_dtype %d", c->kv_dtype);
  if (c->num_kv_heads < 1) return fail(ROPEKV_EINVAL, "num_kv_heads must be >= 1");
  if (c->head_dim < 2 || (c->head_dim & 1) || c->head_dim > 512)
    return fail(ROPEKV_EINVAL, "head_dim %d must be even and in [2, 512]", c->head_dim);
  if (!c->k) return fail(ROPEKV_EINVAL, "cache k is NULL");
  if (!c->err_word) return fail(ROPEKV_EINVAL, "cache err_word is NULL");
  if (c->sinks < 0 || c->window < 0) return fail(ROPEKV_EINVAL, "sinks and window must be >= 0");
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->k_scale) || !aligned16(c->v_scale))
    return fail(ROPEKV_EINVAL, "cache k, v, k_scale and v_scale must be 16-byte aligned");
  if (c->k_int8_mode != 0) {
    if (c->kv_dtype != ROPEKV_I8) return fail(ROPEKV_EINVAL, "k_int8_mode needs an I8 cache");
    if (c->k_int8_mode & ~(ROPEKV_I8_KEEP_SCALE | ROPEKV_I8_HADAMARD))
      return fail(ROPEKV_EINVAL, "unknown k_int8_mode bits %d", c->k_int8_mode);
    if (c->k_int8_mode == (ROPEKV_I8_KEEP_SCALE | ROPEKV_I8_HADAMARD))
      return fail(ROPEKV_EINVAL, "ROPEKV_I8_KEEP_SCALE does not apply to Hadamard-rotated keys");
    if ((c->k_int8_mode & ROPEKV_I8_HADAMARD) && (c->head_dim < 64 || (c->head_dim & (c->head_dim - 1))))
      return fail(ROPEKV_ERANGE, "Hadamard-rotated keys need head_dim = 2^k in [64, 512]");
  }
  switch (c->layout) {
    case ROPEKV_RING:
      if (coded8(c->kv_dtype) && (!c->k_scale || !c->v_scale))
        return fail(ROPEKV_EINVAL, "8-bit RING needs k_scale and v_scale");
      if (c->batch < 1) return fail(ROPEKV_EINVAL, "batch must be >= 1");
      if (c->window < 1) return fail(ROPEKV_EINVAL, "RING needs window >= 1");
      if (c->capacity != c->sinks + c->window)
        return fail(ROPEKV_EINVAL, "RING capacity %d != sinks %d + window %d", c->capacity, c->sinks, c->window);
      if (!c->v || !c->ring_head || !c->ring_count || !c->seq_len)
        return fail(ROPEKV_EINVAL, "RING needs v, ring_head, ring_count and seq_len");
      break;
    case ROPEKV_PAGED:
      if (coded8(c->kv_dtype) && (!c->k_scale || !c->v_scale))
        return fail(ROPEKV_EINVAL, "8-bit PAGED needs k_scale and v_scale");
      if (c->batch < 1) return fail(ROPEKV_EINVAL, "batch must be >= 1");
      if (c->block_size < 1 || c->max_blocks < 1 || c->num_blocks < 1)
        return fail(ROPEKV_EINVAL, "PAGED needs block_size, max_blocks, num_blocks >= 1");
      if (!c->v || !c->block_table || !c->seq_len)
        return fail(ROPEKV_EINVAL, "PAGED needs v, block_table and seq_len");
      break;
    case ROPEKV_CONTIG:
      if (c->capacity < 1) return fail(ROPEKV_EINVAL, "CONTIG capacity must be >= 1");
      if (c->pos0 < 0) return fail(ROPEKV_EINVAL, "CONTIG pos0 must be >= 0");
      if ((long)c->pos0 + c->capacity - 1 > 0x7fffffffL) return fail(ROPEKV_ERANGE, "CONTIG positions overflow int32");
      if (coded8(c->kv_dtype)) {
        if (!c->k_scale) return fail(ROPEKV_EINVAL, "CONTIG 8-bit keys need k_scale");
        if (c->v && !c->v_scale) return fail(ROPEKV_EINVAL, "CONTIG 8-bit values need v_scale");
      }
      break;
    default: return fail(ROPEKV_ELAYOUT, "unknown layout %d", c->layout);
  }
  return ROPEKV_OK;
}

int check_attention_shape(const ropekv_kv_cache *c, int n_q_heads, bool int8_ok) {
  if (c->kv_dtype != ROPEKV_F32 && c->kv_dtype != ROPEKV_BF16 && !(int8_ok && coded8(c->kv_dtype)))
    return fail(ROPEKV_EDTYPE, int8_ok ? "decode supports F32, BF16, I8 and FP8 caches"
                                       : "prefill supports F32 and BF16 caches");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(ROPEKV_ERANGE, "attention supports head_dim 64 and 128");
  if (n_q_heads < 1 || n_q_heads % c->num_kv_heads)
    return fail(ROPEKV_EINVAL, "n_q_heads %d must be a positive multiple of num_kv_heads %d", n_q_heads,
                c->num_kv_heads);
  const int n_rep = n_q_heads / c->num_kv_heads;
  if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8)
    return fail(ROPEKV_ERANGE, "n_q_heads / num_kv_heads = %d must be 1, 2, 4 or 8", n_rep);
  return ROPEKV_OK;
}

// Checks shared by both decode entry points; on success *pl is the launch plan.
int check_decode(const void *q, int batch, int n_q_heads, const ropekv_kv_cache *cache, float scale,
                 const void *out, DecodePlan *pl) {
  int e = check_cache(cache);
  if (e) return e;
  if (cache->layout != ROPEKV_RING && cache->layout != ROPEKV_PAGED)
    return fail(ROPEKV_ELAYOUT, "decode needs a RING or PAGED cache");
  e = check_attention_shape(cache, n_q_heads, true);
  if (e) return e;
  if (cache->layout == ROPEKV_PAGED && cache->block_size != 16)
    return fail(ROPEKV_EINVAL, "decode needs block_size 16");
  if (batch < 1 || batch > cache->batch) return fail(ROPEKV_EINVAL, "batch %d outside [1, %d]", batch, cache->batch);
  if (!q || !out) return fail(ROPEKV_EINVAL, "q and out are required");
  if (!aligned16(q) || !aligned16(out)) return fail(ROPEKV_EINVAL, "q and out must be 16-byte aligned");
  if (!(scale >= 0.f) || !isfinite(scale)) return fail(ROPEKV_EINVAL, "scale must be finite and >= 0");
  *pl = plan_decode(batch, n_q_heads, *cache);
  if (pl->splits > kMaxDecodeSplits)
    return fail(ROPEKV_ERANGE, "cache too long for one decode call (%d splits)", pl->splits);
  return ROPEKV_OK;
}

float resolve_scale(float scale, int d) { return scale == 0.f ? 1.0f / sqrtf((float)d) : scale; }

}  // namespace

extern "C" {

const char *ropekv_last_error(void) { return g_err.c_str(); }

int ropekv_build_table(const ropekv_rope_cfg *cfg, int32_t max_pos, float *cos_sin, float *mscale_dev,
                       ropekv_stream_t stream) {
  int e = check_rope(cfg, "cfg");
  if (e) return e;
  if (max_pos < 1) return fail(ROPEKV_EINVAL, "max_pos must be >= 1");
  if (!cos_sin) return fail(ROPEKV_EINVAL, "cos_sin is NULL");
  return hip_status(launch_build_table(make_rope_params(*cfg), max_pos, cos_sin, mscale_dev, (hipStream_t)stream),
                    "build_table launch");
}

int ropekv_apply_append(const ropekv_rope_cfg *cfg, const float *cos_sin, int32_t table_len, void *q,
                        int32_t n_q_heads, void *k, const void *v, int32_t act_dtype, int32_t n_tokens,
                        const int32_t *positions, const int32_t *seq_ids, const ropekv_kv_cache *cache,
                        int32_t *freed_blocks, int32_t freed_capacity, int32_t *n_freed, ropekv_stream_t stream) {
  int e = check_rope(cfg, "cfg");
  if (e) return e;
  e = check_cache(cache);
  if (e) return e;
  if (cfg->head_dim != cache->head_dim)
    return fail(ROPEKV_EINVAL, "cfg head_dim %d != cache head_dim %d", cfg->head_dim, cache->head_dim);
  if (!cos_sin || table_len < 1) return fail(ROPEKV_EINVAL, "cos_sin table missing or empty");
  if (act_dtype != ROPEKV_F32 && act_dtype != ROPEKV_BF16 && act_dtype != ROPEKV_F16)
    return fail(ROPEKV_EDTYPE, "act_dtype must be F32, BF16 or F16");
  if (n_tokens < 0) return fail(ROPEKV_EINVAL, "n_tokens must be >= 0");
  if (n_q_heads < 0 || (n_q_heads > 0) != (q != nullptr))
    return fail(ROPEKV_EINVAL, "q must be given exactly when n_q_heads > 0");
  if (!k || !positions) return fail(ROPEKV_EINVAL, "k and positions are required");
  if (cache->layout != ROPEKV_CONTIG) {
    if (cache->kv_dtype != act_dtype && !coded8(cache->kv_dtype))
      return fail(ROPEKV_EDTYPE, "RING / PAGED need kv_dtype == act_dtype, I8 or FP8");
    if (!seq_ids) return fail(ROPEKV_EINVAL, "seq_ids are required for RING / PAGED");
  }
  if (cache->v && !v) return fail(ROPEKV_EINVAL, "v is required when the cache holds values");
  if (freed_blocks && (!n_freed || freed_capacity < 0))
    return fail(ROPEKV_EINVAL, "freed_blocks needs n_freed and freed_capacity >= 0");
  if (n_tokens == 0) return ok();
  AppendArgs a;
  a.rotary_dim = cfg->rotary_dim;
  a.head_dim = cfg->head_dim;
  a.neox = cfg->neox ? 1 : 0;
  a.table = cos_sin;
  a.table_len = table_len;
  a.q = q;
  a.n_q_heads = n_q_heads;
  a.k = k;
  a.v = v;
  a.act = act_dtype;
  a.n_tokens = n_tokens;
  a.pos = positions;
  a.seq = seq_ids;
  a.c = *cache;
  a.freed = cache->layout == ROPEKV_PAGED ? freed_blocks : nullptr;
  a.freed_cap = freed_capacity;
  a.n_freed = n_freed;
  {
    // the vector path moves 16-byte units: same dtype in and out, units that tile the halves
    // of the rotary slice and the tail, 16-byte aligned activations
    const int esz = act_dtype == ROPEKV_F32 ? 4 : 2;
    const int pp = 16 / esz;
    const int r = cfg->rotary_dim, d = cfg->head_dim;
    a.vec = cache->kv_dtype == act_dtype && act_dtype != ROPEKV_I8 && (r / 2) % pp == 0 && (d - r) % pp == 0 &&
            aligned16(q) && aligned16(k) && aligned16(v) && d % pp == 0;
  }
  return hip_status(launch_apply_append(a, (hipStream_t)stream), "apply_append launch");
}

size_t ropekv_decode_workspace_size(int32_t batch, int32_t n_q_heads, const ropekv_kv_cache *cache) {
  if (check_cache(cache)) return 0;
  if (batch < 1 || n_q_heads < 1 || n_q_heads % cache->num_kv_heads) return 0;
  return plan_decode(batch, n_q_heads, *cache).ws_bytes;
}

int ropekv_decode_attn(const void *q, int32_t batch, int32_t n_q_heads, const ropekv_kv_cache *cache, float scale,
                       const float *sink_logits, void *out, void *ws, size_t ws_bytes, ropekv_stream_t stream) {
  DecodePlan pl;
  int e = check_decode(q, batch, n_q_heads, cache, scale, out, &pl);
  if (e) return e;
  if (!ws) return fail(ROPEKV_EINVAL, "ws is required");
  if (!aligned16(ws)) return fail(ROPEKV_EINVAL, "ws must be 16-byte aligned");
  if (ws_bytes < pl.ws_bytes)
    return fail(ROPEKV_ENOSPACE, "workspace %zu bytes < %zu needed", ws_bytes, pl.ws_bytes);
  return hip_status(launch_decode(q, batch, n_q_heads, *cache, resolve_scale(scale, cache->head_dim), sink_logits,
                                  out, ws, pl, (hipStream_t)stream),
                    "decode launch");
}

int ropekv_decode_attn_noalloc(const void *q, int32_t batch, int32_t n_q_heads, const ropekv_kv_cache *cache,
                               float scale, const float *sink_logits, void *out, ropekv_stream_t stream) {
  DecodePlan pl;
  int e = check_decode(q, batch, n_q_heads, cache, scale, out, &pl);
  if (e) return e;
  if (pl.ws_bytes > kDecodeScratchBytes)
    return fail(ROPEKV_ENOSPACE, "split-K partials need %zu bytes, more than the %zu-byte scratch of the "
                "allocation-free decode (use ropekv_decode_attn with a workspace)",
                pl.ws_bytes, kDecodeScratchBytes);
  float *ws = nullptr;
  e = hip_status(decode_scratch(&ws), "decode scratch address");
  if (e) return e;
  return hip_status(launch_decode(q, batch, n_q_heads, *cache, resolve_scale(scale, cache->head_dim), sink_logits,
                                  out, ws, pl, (hipStream_t)stream),
                    "decode launch");
}

int ropekv_prefill_attn(const void *q, const void *k, const void *v, int32_t T, int32_t pos0, int32_t n_q_heads,
                        const ropekv_kv_cache *cache, int32_t seq_id, float scale, const float *sink_logits,
                        void *out, ropekv_stream_t stream) {
  int e = check_cache(cache);
  if (e) return e;
  e = check_attention_shape(cache, n_q_heads, false);
  if (e) return e;
  if (T < 0 || pos0 < 0) return fail(ROPEKV_EINVAL, "T and pos0 must be >= 0");
  if ((long)pos0 + T > 0x7fffffffL) return fail(ROPEKV_ERANGE, "positions overflow int32");
  if (!q || !k || !v || !out) return fail(ROPEKV_EINVAL, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(ROPEKV_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (!(scale >= 0.f) || !isfinite(scale)) return fail(ROPEKV_EINVAL, "scale must be finite and >= 0");
  if (pos0 > 0) {
    if (cache->layout != ROPEKV_RING && cache->layout != ROPEKV_PAGED)
      return fail(ROPEKV_ELAYOUT, "a cached prefix (pos0 > 0) needs a RING or PAGED cache");
    if (seq_id < 0 || seq_id >= cache->batch) return fail(ROPEKV_EINVAL, "seq_id outside the batch");
  }
  if (T == 0) return ok();
  return hip_status(launch_prefill(q, k, v, T, pos0, n_q_heads, *cache, seq_id,
                                   resolve_scale(scale, cache->head_dim), sink_logits, out, (hipStream_t)stream),
                    "prefill launch");
}

int ropekv_rerotate(const ropekv_rope_cfg *from, const ropekv_rope_cfg *to, const ropekv_kv_cache *cache,
                    int32_t n_layers, ropekv_stream_t stream) {
  int e = check_rope(from, "from");
  if (e) return e;
  e = check_rope(to, "to");
  if (e) return e;
  e = check_cache(cache);
  if (e) return e;
  if (cache->layout != ROPEKV_CONTIG) return fail(ROPEKV_ELAYOUT, "rerotate needs a CONTIG cache");
  if (from->head_dim != to->head_dim || from->rotary_dim != to->rotary_dim || (from->neox != 0) != (to->neox != 0))
    return fail(ROPEKV_EINVAL, "from / to differ in head_dim, rotary_dim or pairing");
  if (to->head_dim != cache->head_dim) return fail(ROPEKV_EINVAL, "cfg head_dim != cache head_dim");
  if (n_layers < 1) return fail(ROPEKV_EINVAL, "n_layers must be >= 1");
  if (cache->kv_dtype == ROPEKV_FP8) return fail(ROPEKV_EDTYPE, "rerotate supports F32, BF16, F16 and I8 keys");
  if (cache->kv_dtype == ROPEKV_I8) {
    const int d = cache->head_dim, r = to->rotary_dim;
    const int lpr = d / 16;
    if (d % 16 || (lpr & (lpr - 1)))
      return fail(ROPEKV_ERANGE, "int8 rerotate needs head_dim = 16 * 2^k (16 to 512)");
    if (to->neox ? (r % 32) : (r % 16))
      return fail(ROPEKV_ERANGE, "int8 rerotate needs rotary_dim %% %d == 0", to->neox ? 32 : 16);
    if ((cache->k_int8_mode & ROPEKV_I8_HADAMARD) && to->neox && (r < 64 || (r & (r - 1))))
      return fail(ROPEKV_ERANGE, "Hadamard-rotated NeoX keys need rotary_dim = 2^k >= 64");
  }
  return hip_status(launch_rerotate(make_rope_params(*from), make_rope_params(*to), *cache, n_layers,
                                    (hipStream_t)stream),
                    "rerotate launch");
}

int ropekv_shift_keys(const ropekv_rope_cfg *cfg, const ropekv_kv_cache *cache, int32_t delta, int32_t n_layers,
                      ropekv_stream_t stream) {
  int e = check_rope(cfg, "cfg");
  if (e) return e;
  e = check_cache(cache);
  if (e) return e;
  if (cfg->head_dim != cache->head_dim) return fail(ROPEKV_EINVAL, "cfg head_dim != cache head_dim");
  if (cache->kv_dtype != ROPEKV_F32 && cache->kv_dtype != ROPEKV_BF16 && cache->kv_dtype != ROPEKV_F16)
    return fail(ROPEKV_EDTYPE, "shift_keys supports F32, BF16 and F16 keys");
  if (cache->layout == ROPEKV_RING) {
    if (n_layers != 1) return fail(ROPEKV_EINVAL, "a RING descriptor is one layer (n_layers must be 1)");
  } else if (cache->layout == ROPEKV_CONTIG) {
    if (n_layers < 1) return fail(ROPEKV_EINVAL, "n_layers must be >= 1");
  } else {
    return fail(ROPEKV_ELAYOUT, "shift_keys needs a RING or CONTIG cache");
  }
  return hip_status(launch_shift_keys(make_rope_params(*cfg), *cache, delta, n_layers, (hipStream_t)stream),
                    "shift_keys launch");
}

int ropekv_visible_slots(const ropekv_kv_cache *cache, int32_t seq, int32_t *positions_out, int64_t *offsets_out,
                         int32_t max_out, int32_t *n_out, ropekv_stream_t stream) {
  int e = check_cache(cache);
  if (e) return e;
  if (cache->layout != ROPEKV_RING && cache->layout != ROPEKV_PAGED)
    return fail(ROPEKV_ELAYOUT, "visible_slots needs a RING or PAGED cache");
  if (seq < 0 || seq >= cache->batch) return fail(ROPEKV_EINVAL, "seq outside the batch");
  if (max_out < 0 || !n_out || (max_out > 0 && (!positions_out || !offsets_out)))
    return fail(ROPEKV_EINVAL, "output arrays missing");
  return hip_status(launch_visible_slots(*cache, seq, positions_out, offsets_out, max_out, n_out,
                                         (hipStream_t)stream),
                    "visible_slots launch");
}

}  // extern "C"
