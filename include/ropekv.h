/*
 * ropekv.h - C ABI of libropekv.so: rotary position embedding (RoPE / YaRN)
 * fused with a sink + sliding-window KV cache, the decode and prefill
 * attention that read only the visible set, and re-rotation of cached keys
 * when the YaRN factor changes.  gfx950 (MI355X) only.
 *
 * Sources, cited by page title and section:
 *   [RoPE] "RoPE, scaling, sliding window, attention sinks" (mlinterviewnotes)
 *   [GOSS] "Inference & 128K Long Context" (GPT-OSS-Lite docs)
 *   [DYN]  "#2961 rope: --rope-scaling dynamic" (strata pull request)
 *   [SINK] "Attention Sink 与 Streaming KV Cache" (llm-glossary)
 *   [VLLM] "vLLM, from the inside out"
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev or documented as "device" point to device memory
 *     the caller allocated (e.g. with torch); the library never allocates or
 *     frees device memory and keeps no state between calls, except the one
 *     fixed device array of ropekv_decode_attn_noalloc (loaded with the
 *     library's code, one per GPU).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises the host.
 *   - Arguments are validated on the host before any launch; a failing check
 *     returns a negative ROPEKV_E* code, launches nothing, and leaves a
 *     message for ropekv_last_error() (thread-local).
 *   - Conditions that only device data can show (a position outside the
 *     table, a non-consecutive position, a null block where a key must be
 *     written or read) are reported by OR-ing ROPEKV_DEV_* bits into the
 *     cache's err_word; the offending token / tile is skipped, never read or
 *     written out of bounds.  In the append, a token whose position lies
 *     outside the table is left untouched; any other flagged token still has
 *     its q and k rotated in place, but nothing of it is written to the cache;
 *     a token flagged for its sequence or position leaves the sequence's state
 *     as it was, one flagged for its block (null, or past max_blocks) still
 *     advances it.  The decode leaves a
 *     skipped tile's keys out of the softmax; the prefill's rule for a lost
 *     prefix key is given with ropekv_prefill_attn.
 */
#ifndef ROPEKV_H
#define ROPEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ropekv_stream_t; /* a hipStream_t */

/* return codes */
#define ROPEKV_OK 0
#define ROPEKV_EINVAL (-1)    /* bad size / shape / geometry argument */
#define ROPEKV_EDTYPE (-2)    /* unsupported dtype combination */
#define ROPEKV_ERANGE (-3)    /* a size exceeds what the call supports (table, head_dim...) */
#define ROPEKV_ELAYOUT (-4)   /* cache layout not supported by this call */
#define ROPEKV_ENOSPACE (-5)  /* workspace or output buffer too small */
#define ROPEKV_EHIP (-6)      /* a HIP runtime call failed */

/* element types */
#define ROPEKV_F32 0
#define ROPEKV_BF16 1
#define ROPEKV_F16 2
#define ROPEKV_I8 3
#define ROPEKV_FP8 4 /* 8-bit float E4M3 (OCP "fn": bias 7, 3 mantissa bits, max 448, no
                        infinities, S.1111.111 NaN) codes with one fp32 scale per row, like I8
                        ([VLLM] the KV cache stored as FP8) */

/* k_int8_mode bits (int8 keys only) */
#define ROPEKV_I8_KEEP_SCALE 1 /* rerotate keeps each row's scale (tail codes bitwise) unless a turned
                                  rotary code leaves [-127, 127]; then the row is requantised whole
                                  ([DYN] "Measured on this branch": without the Hadamard the dims past
                                  the rotary slice stay as written).  Not with ROPEKV_I8_HADAMARD. */
#define ROPEKV_I8_HADAMARD 2   /* K rows hold int8 codes of H k, H the orthonormal Walsh-Hadamard
                                  transform over all d dims (d a power of two): apply_append
                                  transforms before quantising, decode transforms the query (scores
                                  are unchanged: H is orthogonal), rerotate turns H (dequantised row)
                                  and transforms back ([DYN] "What it does": K with the Hadamard) */

/* cache layouts */
#define ROPEKV_RING 0   /* [batch, Hkv, C, d]: slots 0..S-1 sinks, S..C-1 a W-slot ring */
#define ROPEKV_PAGED 1  /* pool [num_blocks, Hkv, block_size, d] + block table [batch, max_blocks] */
#define ROPEKV_CONTIG 2 /* [T, Hkv, d] per layer (layers back to back), row t = position pos0 + t */

/* device error bits OR-ed into err_word */
#define ROPEKV_DEV_TABLE_RANGE 1  /* a position < 0 or >= table_len */
#define ROPEKV_DEV_POSITION 2     /* a token is not at its sequence's next position */
#define ROPEKV_DEV_NULL_BLOCK 4   /* a needed block-table entry is -1 or >= num_blocks */
#define ROPEKV_DEV_BLOCK_RANGE 8  /* position / block_size >= max_blocks, or CONTIG row out of range */
#define ROPEKV_DEV_SEQ_RANGE 16   /* a sequence id outside [0, batch) */
#define ROPEKV_DEV_PREFIX_LOST 32 /* prefill needs a prefix key the ring no longer holds */
#define ROPEKV_DEV_FREE_OVERFLOW 64 /* freed-block list capacity exceeded (nothing freed) */

/* rope_type values */
#define ROPEKV_ROPE_YARN 0        /* plain RoPE when s <= 1, else YaRN (default) */
#define ROPEKV_ROPE_LINEAR 1      /* position interpolation: angles of position m / s */
#define ROPEKV_ROPE_NTK 2         /* base b * s^(r / (r - 2)) */
#define ROPEKV_ROPE_DYNAMIC_NTK 3 /* base b * (s P / L0 - (s - 1))^(r / (r - 2)), P = served_len */
#define ROPEKV_ROPE_LLAMA3 4      /* wavelength-thresholded blend (low / high_freq_factor) */

/* Rope parameters, in the notation of [RoPE] ("YaRN, precisely" and the four
 * families of fixes): omega_i = 1 / b^(2i/r) for pair i < r/2, edited by the
 * scheme in rope_type with scaling factor s.  YaRN (s > 1) blends the
 * extrapolated and the interpolated (divided by s) frequencies over the
 * correction band of beta_fast / beta_slow rotations within L0 and scales the
 * table by mscale = 0.1 ln s + 1; the other schemes keep mscale 1.  Llama-3
 * keeps pairs with wavelength < L0 / high_freq_factor, divides those with
 * wavelength > L0 / low_freq_factor by s, and moves linearly in L0 / wavelength
 * between.  The first pruned_pairs pairs are identity (omega 0). */
typedef struct {
  int32_t head_dim;     /* d_h */
  int32_t rotary_dim;   /* r: even, 2 <= r <= d_h; dims r..d_h-1 are never touched */
  int32_t neox;         /* 1: pairs (i, i + r/2); 0: GPT-J pairs (2i, 2i+1) ([RoPE] pairing note) */
  int32_t orig_max_pos; /* L0, the trained context */
  double rope_theta;    /* b */
  double yarn_factor;   /* s, the scaling factor of every scheme */
  double beta_fast;     /* 32 */
  double beta_slow;     /* 1 */
  double extrapolation_factor; /* 1 */
  int32_t rope_type;    /* ROPEKV_ROPE_* */
  int32_t pruned_pairs; /* leading identity pairs, 0 <= pruned_pairs <= r/2 */
  int32_t served_len;   /* dynamic NTK: the served length P (> 0) */
  int32_t reserved;     /* 0 */
  double low_freq_factor;  /* Llama-3: 1 */
  double high_freq_factor; /* Llama-3: 4 (> low_freq_factor) */
} ropekv_rope_cfg;

/* One layer's KV cache.  All pointers are device pointers; k, v, k_scale and
 * v_scale must be 16-byte aligned (ROPEKV_EINVAL otherwise).
 * Visible set of the query at position p ([SINK] visible-set definition):
 * key j <= p is visible iff j < sinks or p - j < window; window 0 = full
 * attention (PAGED only).  For RING, capacity C = sinks + window. */
typedef struct {
  int32_t layout;       /* ROPEKV_RING / _PAGED / _CONTIG */
  int32_t kv_dtype;     /* F32 / BF16 / F16 / I8 / FP8 (K and V; CONTIG holds K, V optional) */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d: 64 or 128 for attention; any even size <= 512 for append / rerotate */
  int32_t batch;        /* sequences (RING, PAGED) */
  int32_t capacity;     /* RING: C slots per sequence and head; CONTIG: T rows per layer */
  int32_t sinks;        /* S */
  int32_t window;       /* W recent positions including the current one */
  int32_t block_size;   /* PAGED: tokens per block (16) */
  int32_t max_blocks;   /* PAGED: row length of block_table */
  int32_t num_blocks;   /* PAGED: blocks in the pool */
  int32_t pos0;         /* CONTIG: position of row 0 */
  void *k;              /* keys (rotated), layout as above */
  void *v;              /* values (never rotated); NULL allowed for CONTIG */
  float *k_scale;       /* I8, FP8: per-row fp32 key scale, one per K row (PAGED [num_blocks, Hkv, block_size],
                           RING [batch, Hkv, C], CONTIG [T, Hkv] per layer) */
  int32_t *ring_head;   /* RING [batch]: next ring index to write */
  int32_t *ring_count;  /* RING [batch]: valid ring entries (<= W) */
  int32_t *block_table; /* PAGED [batch, max_blocks]: physical block ids, -1 = null */
  int32_t *seq_len;     /* RING, PAGED [batch]: tokens appended so far (= next position) */
  int32_t *err_word;    /* [1]: ROPEKV_DEV_* bits, OR-ed by kernels; caller clears */
  float *v_scale;       /* I8, FP8 RING / PAGED: per-row fp32 value scale, laid out like k_scale */
  int32_t k_int8_mode;  /* I8 keys: 0 or ROPEKV_I8_* bits; must be 0 for other dtypes */
  int32_t reserved;     /* 0 */
} ropekv_kv_cache;

/* Build the cos/sin table ([RoPE] _compute_cos_sin_cache, YaRN variant):
 * cos_sin[m][i] = mu cos(m w_i), cos_sin[m][r/2 + i] = mu sin(m w_i) for
 * m < max_pos, i < r/2, angles and trig in fp64, one rounding to fp32.
 * cos_sin: device fp32 [max_pos, r], written in place (pointer-stable, so a
 * rebuild at a new factor keeps graphs that captured it valid, [DYN] "The
 * table").  mscale_dev: optional device float receiving mu.  Each cell is
 * computed independently: the result does not depend on the launch shape. */
int ropekv_build_table(const ropekv_rope_cfg *cfg, int32_t max_pos, float *cos_sin,
                       float *mscale_dev, ropekv_stream_t stream);

/* Rotate q and k in place and write the rotated k and the raw v into the
 * cache ([RoPE] "Where the positions come from" and the attention block:
 * positions and slots from one counter, rotate Q and K never V, the cache
 * stores keys-at-a-position; [GOSS] 4.8 rotate once at append).
 *   q   [n_tokens, n_q_heads, d] act_dtype, rotated in place; NULL iff n_q_heads == 0
 *   k   [n_tokens, Hkv, d] act_dtype, rotated in place
 *   v   [n_tokens, Hkv, d] act_dtype; copied unrotated (NULL only for a CONTIG cache with v == NULL)
 *   positions [n_tokens] int32 absolute positions, < table_len
 *   seq_ids   [n_tokens] int32 sequence of each token (RING, PAGED; ignored for CONTIG)
 * act_dtype: F32 / BF16 / F16.  RING and PAGED need kv_dtype == act_dtype, I8 or FP8.
 * Each sequence appears as one run of consecutive positions starting at its
 * seq_len; seq_len advances by the run length.
 * RING ([GOSS] ring buffer, 5.2 append): sinks p < S go to slot p; a chunk of
 *   k >= W non-sink tokens into an empty ring keeps its last W in order with
 *   head 0, count W; otherwise head advances per token mod W and count
 *   saturates at W.  Only the surviving (last) write to a slot is made.
 * PAGED ([RoPE] block bound and null-block freeing; [VLLM] block tables):
 *   slot = table[p / bs] * bs + p % bs, the block must be allocated (>= 0).
 *   Before the writes, blocks wholly below the edge e = max(0, seq_len - W + 1)
 *   that hold no sink are set to -1 (backward scan stopping at the first null)
 *   and their ids appended to freed_blocks (device int32 [freed_capacity]),
 *   counted in *n_freed (device int32, caller zeroes it).  freed_blocks NULL:
 *   nothing is freed.
 * CONTIG: row t = p - pos0.
 * Stored dtype: F32 / BF16 / F16 round the fp32 result to nearest; I8 stores
 *   per-row codes clamp(rne(x / scale), -127, 127) with scale = max|x| / 127,
 *   both IEEE fp32 divisions (keys after rotation, values as given; an
 *   all-zero row has scale 0).  FP8 stores the E4M3 code nearest (ties to
 *   even) to x / scale clamped to [-448, 448], with scale = max|x| / 448. */
int ropekv_apply_append(const ropekv_rope_cfg *cfg, const float *cos_sin, int32_t table_len,
                        void *q, int32_t n_q_heads, void *k, const void *v, int32_t act_dtype,
                        int32_t n_tokens, const int32_t *positions, const int32_t *seq_ids,
                        const ropekv_kv_cache *cache, int32_t *freed_blocks,
                        int32_t freed_capacity, int32_t *n_freed, ropekv_stream_t stream);

/* Bytes of fp32 workspace ropekv_decode_attn needs for this batch and cache
 * (the split-K partials of the decode plan: decode is bound by streaming the
 * KV cache, [GOSS] 4.3, so one long sequence is spread over many workgroups
 * whose partial softmax sums are then merged: [batch, Hkv, splits, n_rep,
 * d + 2]).  0 on bad input, and 0
 * for plans without partials: F32 / BF16 caches with at least 256 (sequence, KV
 * head) units of at most 512 16-row tiles each get one workgroup per unit that
 * writes its output directly. */
size_t ropekv_decode_workspace_size(int32_t batch, int32_t n_q_heads, const ropekv_kv_cache *cache);

/* Decode attention ([SINK] the incremental path; [GOSS] 4.3 decode, 4.4 GQA):
 * for each sequence b with n = seq_len[b] > 0 tokens and query head h,
 * out[b][h] = softmax(q[b][h] . K_j * scale) V_j over the keys j visible to
 * position n - 1, with K / V of KV head h / (n_q_heads / Hkv).  The keys are
 * read in place (no gather, no repeat of KV heads).  Split-K partials go to
 * ws and a second launch combines them, unless the plan has one workgroup per
 * (sequence, KV head) (see ropekv_decode_workspace_size).  n == 0 gives a zero
 * row.
 *   q   [batch, n_q_heads, d] kv_dtype (rotated), out same shape and dtype
 *   scale: 0 means 1/sqrt(d)
 *   sink_logits: NULL, or device fp32 [n_q_heads] learned sink logits ([RoPE]
 *     the learned-sink excerpt: a trained per-head logit in the softmax
 *     denominator, no cache entry): out = sum_j e^{s_j} v_j / (sum_j e^{s_j}
 *     + e^{sink_h}), the logit in the units of the scaled scores
 * Layouts RING and PAGED (block_size 16); kv_dtype F32, BF16, I8 or FP8 (for the
 * 8-bit caches q and out are BF16; keys and values are dequantised with their row
 * scales); d 64 or 128;
 * n_rep = n_q_heads / Hkv in {1, 2, 4, 8}.  ws: device, at least
 * ropekv_decode_workspace_size() bytes, caller-owned, overwritten.
 * q, out and ws must be 16-byte aligned. */
int ropekv_decode_attn(const void *q, int32_t batch, int32_t n_q_heads,
                       const ropekv_kv_cache *cache, float scale, const float *sink_logits,
                       void *out, void *ws, size_t ws_bytes, ropekv_stream_t stream);

/* ropekv_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation): the split-K partials go to a 64 MiB device array inside
 * the library, one per GPU, set up on the first call on each device and held
 * until the process ends.  Nothing is allocated per call.  Same arguments,
 * kernels and results as ropekv_decode_attn.  A batch and cache whose partials
 * (ropekv_decode_workspace_size) exceed 64 MiB return ROPEKV_ENOSPACE and
 * launch nothing.  All calls on one GPU share the array: calls that overlap in
 * time on one GPU (different streams, or different host threads) race and
 * must be ordered by the caller. */
int ropekv_decode_attn_noalloc(const void *q, int32_t batch, int32_t n_q_heads,
                               const ropekv_kv_cache *cache, float scale,
                               const float *sink_logits, void *out, ropekv_stream_t stream);

/* Prefill attention for one sequence's chunk ([GOSS] 5.5 mask alignment):
 * queries t < T at positions pos0 + t see keys j <= pos0 + t with j < S or
 * pos0 + t - j < W (W from the cache; 0 = causal).  Keys at positions
 * >= pos0 come from the chunk's own k, v ([T, Hkv, d], rotated); keys below
 * pos0 from the cache (RING or PAGED) of sequence seq_id.  For RING the
 * prefix must still be in the ring (call before appending the chunk, or keep
 * pos0 + T <= C); a missing key (not in the ring, or in a null PAGED block) sets
 * ROPEKV_DEV_PREFIX_LOST, and the output rows of the queries that see it are then
 * unspecified (the other rows stay exact; nothing is read out of bounds).
 *   q [T, n_q_heads, d], out same; dtype = kv_dtype (F32 or BF16), d 64 or 128,
 *   n_rep = n_q_heads / Hkv in {1, 2, 4, 8}; seq_id only read when pos0 > 0;
 *   sink_logits as for ropekv_decode_attn; q, k, v and out 16-byte aligned.
 * bf16 runs on MFMA with fp32 accumulation; tiles no query can see are skipped. */
int ropekv_prefill_attn(const void *q, const void *k, const void *v, int32_t T, int32_t pos0,
                        int32_t n_q_heads, const ropekv_kv_cache *cache, int32_t seq_id,
                        float scale, const float *sink_logits, void *out, ropekv_stream_t stream);

/* Re-rotate cached keys from `from` to `to` in place ([DYN] "What it does":
 * the cached keys follow a change; [SINK] R_a R_b = R_{a+b}): every pair i of
 * the row at position p turns by p (w_to,i - w_from,i) and is scaled by
 * mscale_to / mscale_from; dims r..d-1 are untouched (bitwise for F16/BF16/F32).
 * I8 rows are dequantised, turned and requantised with a new per-row scale
 * max|y| / 127, codes rne(y * (127 / max|y|)) with the reciprocal correctly
 * rounded and the product rounded once (within one fp32 rounding of y / scale);
 * a row the turn leaves unchanged keeps its codes and scale bit for bit.
 * cache: CONTIG, kv_dtype F16 / BF16 / F32 / I8, n_layers >= 1 layers back to back
 * (FP8: ROPEKV_EDTYPE).  I8 keys need head_dim = 16 * 2^k (16 to 512) and rotary_dim
 * a multiple of 32 (NeoX) or 16 (GPT-J); Hadamard-rotated NeoX keys rotary_dim = 2^k
 * >= 64; otherwise ROPEKV_ERANGE.
 * The angle p (w_to,i - w_from,i) and its reduction modulo 2 pi in fp64; cos and sin of the
 * reduced angle, and the rotation, in fp32 (cos and sin within a few 1e-7 of the exact values).
 * from / to must agree on head_dim, rotary_dim and neox. */
int ropekv_rerotate(const ropekv_rope_cfg *from, const ropekv_rope_cfg *to,
                    const ropekv_kv_cache *cache, int32_t n_layers, ropekv_stream_t stream);

/* Move cached (rotated) keys by `delta` positions in place: every rotary pair
 * turns by delta * w_i with gain 1; dims r..d-1 are untouched ([SINK] "RoPE:
 * absolute positions and local rerotation": a window implementation that
 * re-maps attention positions to [0, C-1] moves each recent key from p to
 * p - 1 per slide, R_a R_b = R_{a+b}, while sink keys keep their positions).
 *   RING: every valid ring slot (the `count` newest non-sink keys) of every
 *     sequence and KV head; sink slots, empty slots and values are not
 *     touched; n_layers must be 1.
 *   CONTIG: every row of n_layers layers.
 * kv_dtype F32 / BF16 / F16; angles in fp64, the rotation in fp32. */
int ropekv_shift_keys(const ropekv_rope_cfg *cfg, const ropekv_kv_cache *cache, int32_t delta,
                      int32_t n_layers, ropekv_stream_t stream);

/* Test-facing: the visible logical positions of sequence seq's next query
 * (position seq_len - 1) and the element offset of each key row in the
 * cache's k buffer, in chronological order, as the attention kernels address
 * them.  The visible set is the one [SINK] "可见集合与容量定义" defines (the
 * S sinks and the W most recent positions, capacity C = S + W); the order is
 * the chronological read-out of [GOSS] "5.3 get" (sinks, then the ring from
 * its oldest entry).  positions_out / offsets_out: device int32 / int64 [max_out];
 * n_out: device int32 receiving the count (entries beyond max_out dropped). */
int ropekv_visible_slots(const ropekv_kv_cache *cache, int32_t seq, int32_t *positions_out,
                         int64_t *offsets_out, int32_t max_out, int32_t *n_out,
                         ropekv_stream_t stream);

/* The message of the last failing call on this thread ("" if none).  Calls
 * fail loudly with a reason where the engines [RoPE] compares either read
 * past the cos/sin table or grow it silently with the unscaled base (the
 * passage on what happens when a position exceeds the table). */
const char *ropekv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPEKV_H */
