/* Host-side argument checks of every libropekv entry point, run under the
 * address and undefined-behaviour sanitizers (tests/test_abi_sanitizers.py
 * builds it).  Every call here fails validation or only sizes a workspace:
 * nothing is launched, so no GPU is needed and none is touched. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ropekv.h"

static int failures = 0;

static void expect(int got, int want, const char *what) {
  if (got != want) {
    printf("FAIL %s: got %d want %d (%s)\n", what, got, want, ropekv_last_error());
    ++failures;
  } else if (want != ROPEKV_OK && ropekv_last_error()[0] == '\0') {
    printf("FAIL %s: no message\n", what);
    ++failures;
  }
}

#define FAKE ((void *)0x1000)

static ropekv_rope_cfg rope(int d, int r) {
  ropekv_rope_cfg c;
  memset(&c, 0, sizeof c);
  c.head_dim = d;
  c.rotary_dim = r;
  c.neox = 1;
  c.orig_max_pos = 4096;
  c.rope_theta = 1e4;
  c.yarn_factor = 1.0;
  c.beta_fast = 32.0;
  c.beta_slow = 1.0;
  c.extrapolation_factor = 1.0;
  c.low_freq_factor = 1.0;
  c.high_freq_factor = 4.0;
  return c;
}

static ropekv_kv_cache ring(int dt, int hkv, int d) {
  ropekv_kv_cache c;
  memset(&c, 0, sizeof c);
  c.layout = ROPEKV_RING;
  c.kv_dtype = dt;
  c.num_kv_heads = hkv;
  c.head_dim = d;
  c.batch = 1;
  c.capacity = 16;
  c.sinks = 4;
  c.window = 12;
  c.k = c.v = FAKE;
  c.ring_head = c.ring_count = c.seq_len = c.err_word = (int32_t *)FAKE;
  return c;
}

int main(void) {
  float *tab = (float *)FAKE;
  /* build_table */
  ropekv_rope_cfg bad[5] = {rope(64, 63), rope(64, 0), rope(32, 64), rope(64, 64), rope(64, 64)};
  bad[3].rope_theta = 1.0;
  bad[4].yarn_factor = 2.0;
  bad[4].orig_max_pos = 0;
  for (int i = 0; i < 5; ++i) expect(ropekv_build_table(&bad[i], 16, tab, NULL, NULL), ROPEKV_EINVAL, "build_table cfg");
  ropekv_rope_cfg good = rope(64, 64);
  expect(ropekv_build_table(&good, 0, tab, NULL, NULL), ROPEKV_EINVAL, "build_table max_pos");
  expect(ropekv_build_table(&good, 16, NULL, NULL, NULL), ROPEKV_EINVAL, "build_table table");
  expect(ropekv_build_table(NULL, 16, tab, NULL, NULL), ROPEKV_EINVAL, "build_table NULL cfg");
  ropekv_rope_cfg ty = rope(64, 64);
  ty.rope_type = 9;
  expect(ropekv_build_table(&ty, 16, tab, NULL, NULL), ROPEKV_EINVAL, "build_table rope_type");
  ty = rope(64, 64);
  ty.rope_type = ROPEKV_ROPE_DYNAMIC_NTK;
  ty.yarn_factor = 2.0;
  ty.served_len = 0;
  expect(ropekv_build_table(&ty, 16, tab, NULL, NULL), ROPEKV_EINVAL, "build_table dynamic NTK");
  ty.yarn_factor = NAN;
  expect(ropekv_build_table(&ty, 16, tab, NULL, NULL), ROPEKV_EINVAL, "build_table NaN factor");

  /* apply_append */
  ropekv_kv_cache c = ring(ROPEKV_F32, 4, 64);
  int32_t *ip = (int32_t *)FAKE;
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_FP8, 4, ip, ip, &c, NULL, 0, NULL, NULL),
         ROPEKV_EDTYPE, "append act fp8");
  expect(ropekv_apply_append(&good, tab, 16, NULL, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &c, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append q missing");
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, -1, ip, ip, &c, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append n_tokens");
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, NULL, &c, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append seq_ids");
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 0, ip, ip, &c, NULL, 0, NULL, NULL),
         ROPEKV_OK, "append empty");
  ropekv_kv_cache cbad = c;
  cbad.capacity = 17;
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &cbad, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append ring capacity");
  cbad = c;
  cbad.k = (char *)FAKE + 8;
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &cbad, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append alignment");
  cbad = c;
  cbad.layout = 7;
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &cbad, NULL, 0, NULL, NULL),
         ROPEKV_ELAYOUT, "append layout");
  cbad = ring(ROPEKV_I8, 4, 64);
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &cbad, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append int8 without scales");
  cbad.k_scale = cbad.v_scale = (float *)FAKE;
  cbad.k_int8_mode = ROPEKV_I8_KEEP_SCALE | ROPEKV_I8_HADAMARD;
  expect(ropekv_apply_append(&good, tab, 16, FAKE, 8, FAKE, FAKE, ROPEKV_F32, 4, ip, ip, &cbad, NULL, 0, NULL, NULL),
         ROPEKV_EINVAL, "append int8 modes");

  /* decode */
  char ws[64];
  expect(ropekv_decode_attn(FAKE, 1, 6, &c, 0.f, NULL, FAKE, FAKE, 1u << 30, NULL), ROPEKV_EINVAL, "decode heads");
  expect(ropekv_decode_attn(FAKE, 1, 64, &c, 0.f, NULL, FAKE, FAKE, 1u << 30, NULL), ROPEKV_ERANGE, "decode n_rep");
  expect(ropekv_decode_attn(FAKE, 2, 8, &c, 0.f, NULL, FAKE, FAKE, 1u << 30, NULL), ROPEKV_EINVAL, "decode batch");
  expect(ropekv_decode_attn(FAKE, 1, 8, &c, 0.f, NULL, FAKE, FAKE, 1, NULL), ROPEKV_ENOSPACE, "decode workspace");
  expect(ropekv_decode_attn(FAKE, 1, 8, &c, NAN, NULL, FAKE, FAKE, 1u << 30, NULL), ROPEKV_EINVAL, "decode scale");
  expect(ropekv_decode_attn((char *)FAKE + 2, 1, 8, &c, 0.f, NULL, FAKE, FAKE, 1u << 30, NULL), ROPEKV_EINVAL,
         "decode q alignment");
  expect(ropekv_decode_attn(FAKE, 1, 8, &c, 0.f, NULL, FAKE, NULL, 1u << 30, NULL), ROPEKV_EINVAL, "decode ws");
  ropekv_kv_cache c16 = ring(ROPEKV_F16, 4, 64);
  expect(ropekv_decode_attn(FAKE, 1, 8, &c16, 0.f, NULL, FAKE, ws, sizeof ws, NULL), ROPEKV_EDTYPE, "decode f16");
  expect(ropekv_decode_attn_noalloc(FAKE, 1, 6, &c, 0.f, NULL, FAKE, NULL), ROPEKV_EINVAL, "noalloc heads");
  expect(ropekv_decode_attn_noalloc(FAKE, 1, 8, &c, 0.f, NULL, NULL, NULL), ROPEKV_EINVAL, "noalloc out");
  ropekv_kv_cache big;
  memset(&big, 0, sizeof big);
  big.layout = ROPEKV_PAGED;
  big.kv_dtype = ROPEKV_BF16;
  big.num_kv_heads = 8;
  big.head_dim = 128;
  big.batch = 256;
  big.block_size = 16;
  big.max_blocks = 8192;
  big.num_blocks = 1 << 21;
  big.k = big.v = FAKE;
  big.block_table = big.seq_len = big.err_word = (int32_t *)FAKE;
  expect(ropekv_decode_attn_noalloc(FAKE, 256, 32, &big, 0.f, NULL, FAKE, NULL), ROPEKV_ENOSPACE, "noalloc too big");
  /* workspace sizes: the split plan of a long full-attention layer, the direct plan of many short runs */
  const size_t w1 = ropekv_decode_workspace_size(64, 32, &big);
  big.max_blocks = 2048;
  const size_t w2 = ropekv_decode_workspace_size(64, 32, &big);
  big.max_blocks = 200;
  big.batch = 64;
  const size_t w3 = ropekv_decode_workspace_size(64, 32, &big);
  if (!(w1 > 0 && w2 > 0 && w2 < w1 && w3 == 0)) {
    printf("FAIL workspace sizes %zu %zu %zu\n", w1, w2, w3);
    ++failures;
  }
  if (ropekv_decode_workspace_size(64, 30, &big) != 0) {
    printf("FAIL workspace size of a bad head count\n");
    ++failures;
  }

  /* prefill */
  expect(ropekv_prefill_attn(FAKE, FAKE, FAKE, 8, 0, 8, &c, 0, 0.f, NULL, (char *)FAKE + 4, NULL), ROPEKV_EINVAL,
         "prefill out alignment");
  expect(ropekv_prefill_attn(FAKE, FAKE, FAKE, 8, 5, 8, &c, 3, 0.f, NULL, FAKE, NULL), ROPEKV_EINVAL, "prefill seq");
  expect(ropekv_prefill_attn(FAKE, FAKE, FAKE, -1, 0, 8, &c, 0, 0.f, NULL, FAKE, NULL), ROPEKV_EINVAL, "prefill T");
  expect(ropekv_prefill_attn(FAKE, FAKE, FAKE, 0, 0, 8, &c, 0, 0.f, NULL, FAKE, NULL), ROPEKV_OK, "prefill empty");

  /* rerotate and shift */
  ropekv_rope_cfg a = rope(128, 64), b = rope(128, 64);
  b.yarn_factor = 2.0;
  b.orig_max_pos = 262144;
  ropekv_kv_cache k;
  memset(&k, 0, sizeof k);
  k.layout = ROPEKV_CONTIG;
  k.kv_dtype = ROPEKV_F16;
  k.num_kv_heads = 8;
  k.head_dim = 128;
  k.capacity = 100;
  k.k = FAKE;
  k.err_word = (int32_t *)FAKE;
  ropekv_rope_cfg b2 = b;
  b2.rotary_dim = 32;
  expect(ropekv_rerotate(&a, &b2, &k, 1, NULL), ROPEKV_EINVAL, "rerotate differing r");
  expect(ropekv_rerotate(&a, &b, &k, 0, NULL), ROPEKV_EINVAL, "rerotate layers");
  k.kv_dtype = ROPEKV_FP8;
  k.k_scale = (float *)FAKE;
  expect(ropekv_rerotate(&a, &b, &k, 1, NULL), ROPEKV_EDTYPE, "rerotate fp8");
  k.kv_dtype = ROPEKV_I8;
  k.head_dim = 120;
  a.head_dim = b.head_dim = 120;
  expect(ropekv_rerotate(&a, &b, &k, 1, NULL), ROPEKV_ERANGE, "rerotate int8 head_dim");
  expect(ropekv_shift_keys(&good, &k, -1, 1, NULL), ROPEKV_EINVAL, "shift head_dim");
  ropekv_kv_cache r8 = ring(ROPEKV_F32, 4, 64);
  expect(ropekv_shift_keys(&good, &r8, -1, 2, NULL), ROPEKV_EINVAL, "shift ring layers");
  expect(ropekv_visible_slots(&r8, 3, ip, (int64_t *)FAKE, 4, ip, NULL), ROPEKV_EINVAL, "visible seq");
  expect(ropekv_visible_slots(&r8, 0, NULL, NULL, 4, ip, NULL), ROPEKV_EINVAL, "visible outputs");

  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("all argument checks ok\n");
  return 0;
}
