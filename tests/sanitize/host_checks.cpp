// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every argument validation path, the workspace
// sizes over a range of shapes, and the error text. No kernel is launched
// (every call here is refused, or only sizes a workspace), so no GPU is
// needed. Built host-only by tests/test_host_sanitizers.py.

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "verkv.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__, \
              __LINE__, #cond, vkv_last_error());                       \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void *fake(void) { return (void *)0x1000; }

static vkv_decode_args decode_args(void) {
  vkv_decode_args a;
  memset(&a, 0, sizeof a);
  a.batch = 2; a.n_q_heads = 32; a.n_kv_heads = 8; a.head_dim = 128;
  a.n_tokens = 4096; a.sketch_dim = 32; a.cap = 600; a.fetch_cap = 4096;
  a.eps = 0.1f; a.delta = 0.05f;
  a.q = (const uint16_t *)fake(); a.resident_kv = (const uint16_t *)fake();
  a.resident_idx = (const int32_t *)fake(); a.resident_count = (const int32_t *)fake();
  a.sketch = (const uint16_t *)fake(); a.proj = (const float *)fake();
  a.r = (const float *)fake(); a.host_kv = (const uint16_t *)fake();
  a.out = (float *)fake(); a.d_hat = (float *)fake(); a.log_shift = (float *)fake();
  a.eps_hat0 = (float *)fake(); a.eps_hat = (float *)fake();
  a.k_star = (int32_t *)fake(); a.fetch_idx = (int32_t *)fake();
  a.fetch_count = (int32_t *)fake(); a.host_bytes = (uint64_t *)fake();
  a.status = (uint32_t *)fake();
  a.workspace = fake(); a.workspace_bytes = (size_t)1 << 40;
  return a;
}

static vkv_compress_args compress_args(void) {
  vkv_compress_args a;
  memset(&a, 0, sizeof a);
  a.n_layers = 2; a.n_kv_heads = 3; a.n_tokens = 5000; a.head_dim = 128;
  a.budget = 600; a.n_sink = 4; a.n_local = 32; a.seed = 1; a.cap = 1000;
  a.tau = (const float *)fake(); a.r = (float *)fake();
  a.resident_idx = (int32_t *)fake(); a.resident_count = (int32_t *)fake();
  a.status = (uint32_t *)fake();
  a.workspace = fake(); a.workspace_bytes = 1;
  return a;
}

int main(void) {
  // ---- workspace sizes over many shapes (layout arithmetic only)
  for (int b = 1; b <= 64; b *= 2)
    for (int n = 1; n <= (1 << 17); n = n * 3 + 1)
      for (int grp = 1; grp <= 8; grp *= 2) {
        vkv_decode_args a = decode_args();
        a.batch = b; a.n_tokens = n; a.fetch_cap = n; a.n_q_heads = 8 * grp;
        a.cap = n < 4096 ? n : 4096;
        const size_t ws = vkv_decode_workspace_bytes(&a);
        EXPECT(ws > 0 && ws % 256 == 0);
        a.weights = VKV_W_SKETCH2;
        a.ctx_stride = n + 7;
        EXPECT(vkv_decode_workspace_bytes(&a) > 0);
      }
  for (int n = 1; n <= (1 << 21); n = n * 5 + 3) {
    vkv_compress_args c = compress_args();
    c.n_tokens = n;
    EXPECT(vkv_compress_workspace_bytes(&c) > 0);
    vkv_sketch2_args s;
    memset(&s, 0, sizeof s);
    s.n_slices = 3; s.n_tokens = n; s.head_dim = 128; s.key_stride = 256;
    s.slice_stride = (int64_t)n * 256;
    EXPECT(vkv_sketch2_workspace_bytes(&s) > 0);
    vkv_dense_args d;
    memset(&d, 0, sizeof d);
    d.batch = 2; d.n_q_heads = 32; d.n_kv_heads = 8; d.head_dim = 128; d.n_tokens = n;
    EXPECT(vkv_dense_workspace_bytes(&d) > 0);
  }
  // ---- decode validation
  {
    vkv_decode_args a = decode_args(); a.eps = 0.0f;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL && strstr(vkv_last_error(), "eps"));
    a = decode_args(); a.delta = 1.0f;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL);
    a = decode_args(); a.n_q_heads = 24;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EUNSUPPORTED);
    a = decode_args(); a.n_tokens = (1 << 17) + 1; a.fetch_cap = 1 << 17;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EUNSUPPORTED);
    a = decode_args(); a.weights = 7;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL);
    a = decode_args(); a.weights = VKV_W_SKETCH2;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL && strstr(vkv_last_error(), "sk2"));
    a = decode_args(); a.ctx_stride = 100;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL);
    a = decode_args(); a.stage_map_prev = (const int32_t *)fake();
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL);
    a = decode_args(); a.workspace_bytes = 16;
    EXPECT(vkv_decode_step(&a, NULL) == VKV_EINVAL);
    a = decode_args();
    EXPECT(vkv_decode_step_noalloc(&a, NULL) == VKV_EINVAL);  // workspace given
    a = decode_args(); a.workspace = NULL; a.workspace_bytes = 0;
    a.batch = 16; a.n_tokens = 32768; a.fetch_cap = 32768; a.cap = 4600;
    EXPECT(vkv_decode_step_noalloc(&a, NULL) == VKV_EUNSUPPORTED);
    EXPECT(vkv_decode_step(NULL, NULL) == VKV_EINVAL);
  }
  // ---- compress validation
  {
    vkv_compress_args c = compress_args(); c.budget = 30;
    EXPECT(vkv_compress(&c, NULL) == VKV_EINVAL);
    c = compress_args(); c.head_dim = 64;
    EXPECT(vkv_compress(&c, NULL) == VKV_EINVAL);
    c = compress_args(); c.kv_stride = 100;
    EXPECT(vkv_compress(&c, NULL) == VKV_EINVAL);
    c = compress_args(); c.ctx_stride = 10;
    EXPECT(vkv_compress(&c, NULL) == VKV_EINVAL);
    c = compress_args(); c.resident_kv = (uint16_t *)fake();
    EXPECT(vkv_compress(&c, NULL) == VKV_EINVAL);
    EXPECT(vkv_compress(NULL, NULL) == VKV_EINVAL);
  }
  // ---- sketch build, append and dense validation
  {
    vkv_sketch2_args s;
    memset(&s, 0, sizeof s);
    s.n_slices = 1; s.n_tokens = 100; s.head_dim = 128; s.key_stride = 130;
    EXPECT(vkv_sketch2_build(&s, NULL) == VKV_EINVAL);
    s.key_stride = 128; s.k = (const uint16_t *)0x1008; s.codes = (uint64_t *)fake();
    s.zs = (uint16_t *)fake(); s.chan = (int32_t *)fake();
    s.workspace = fake(); s.workspace_bytes = 1 << 20;
    EXPECT(vkv_sketch2_build(&s, NULL) == VKV_EINVAL);  // misaligned k
    vkv_append_args p;
    memset(&p, 0, sizeof p);
    p.batch = 1; p.n_kv_heads = 1; p.head_dim = 128; p.pos = 5; p.cap = 4; p.ctx_stride = 5;
    EXPECT(vkv_append_token(&p, NULL) == VKV_EINVAL);  // pos == ctx_stride
    vkv_dense_args d;
    memset(&d, 0, sizeof d);
    d.batch = 1; d.n_q_heads = 4; d.n_kv_heads = 1; d.head_dim = 128; d.n_tokens = 10;
    EXPECT(vkv_dense_attention(&d, NULL) == VKV_EINVAL);
  }
  // ---- status word check and phase names
  EXPECT(vkv_check_status(NULL, NULL, NULL) == VKV_EINVAL);
  for (int i = -2; i < vkv_decode_phase_count() + 2; ++i) {
    const char *nm = vkv_decode_phase_name(i);
    EXPECT((nm != NULL) == (i >= 0 && i < vkv_decode_phase_count()));
    if (nm) EXPECT(strlen(nm) > 0);
  }
  EXPECT(strlen(vkv_last_error()) < 512);
  printf("host checks: %d failures\n", failures);
  return failures ? 1 : 0;
}
