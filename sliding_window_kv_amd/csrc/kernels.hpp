// Host-side launchers of the ropekv kernels (called by api.cpp after validation).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ropekv {

// Launch geometry of the split-K decode, shared by the workspace query and the launch.
struct DecodePlan {
  int n_rep;
  int max_tiles;        // upper bound on 16-row tiles any sequence visits
  int tiles_per_split;  // tiles handled by one workgroup
  int splits;           // workgroups per (sequence, KV head)
  size_t ws_bytes;
  bool direct;          // one wide workgroup per (sequence, KV head) writes the output (no combine)
};

DecodePlan plan_decode(int batch, int n_q_heads, const ropekv_kv_cache &c);

// The allocation-free decode keeps its split-K partials in a file-scope device
// array of this size (one copy per GPU); decode_scratch gives the current
// device's address of it, looked up once per device.
constexpr int kMaxDecodeSplits = 1024;  // splits one combine workgroup merges
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(float **ptr);

hipError_t launch_build_table(const RopeParams &rp, int max_pos, float *out, float *mscale_dev,
                              hipStream_t s);

struct AppendArgs {
  int rotary_dim, head_dim, neox;
  const float *table;
  int table_len;
  void *q;
  int n_q_heads;
  void *k;
  const void *v;
  int act;
  int n_tokens;
  const int32_t *pos;
  const int32_t *seq;
  ropekv_kv_cache c;
  int32_t *freed;
  int freed_cap;
  int32_t *n_freed;
  int vec;  // 1: the 16-byte vector path applies (same 16-bit or fp32 dtype in and out, aligned rows)
};
hipError_t launch_apply_append(const AppendArgs &a, hipStream_t s);

hipError_t launch_decode(const void *q, int batch, int n_q_heads, const ropekv_kv_cache &c, float scale,
                         const float *sink_logits, void *out, void *ws, const DecodePlan &plan, hipStream_t s);

// 8-bit caches, int8 or E4M3 codes (bf16 q and out); sl2 = softmax scale x log2(e)
hipError_t launch_decode_8bit(const void *q, int batch, const ropekv_kv_cache &c, float sl2, const float *sinks,
                              void *out, float *ws, const DecodePlan &plan, hipStream_t s);

hipError_t launch_prefill(const void *q, const void *k, const void *v, int T, int pos0, int n_q_heads,
                          const ropekv_kv_cache &c, int seq_id, float scale, const float *sink_logits, void *out,
                          hipStream_t s);

hipError_t launch_rerotate(const RopeParams &from, const RopeParams &to, const ropekv_kv_cache &c,
                           int n_layers, hipStream_t s);

hipError_t launch_shift_keys(const RopeParams &p, const ropekv_kv_cache &c, int delta, int n_layers, hipStream_t s);

hipError_t launch_visible_slots(const ropekv_kv_cache &c, int seq, int32_t *pos_out, int64_t *off_out,
                                int max_out, int32_t *n_out, hipStream_t s);

}  // namespace ropekv
