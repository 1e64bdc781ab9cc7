/*
 * Host-side check of libtidar's argument validation and planning, meant to be
 * linked against a build of the library whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer. Every call here fails
 * validation or is a workspace query, so nothing reaches the GPU and the
 * program runs on a machine without one. Exit status 0 = every expectation
 * held and the sanitizers reported nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tidar.h"

static int failures = 0;
#define FAKE ((void*)(uintptr_t)0x10000) /* aligned, non-null, never dereferenced */
#define FAKE_OFF(n) ((void*)(uintptr_t)(0x10000 + (n)))

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, tidar_last_error());
    ++failures;
  }
}

static tidar_attn_desc base_desc(void) {
  tidar_attn_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 1;
  d.num_q_heads = 32;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.k = 16;
  d.num_blocks = 17;
  d.block_len = 16;
  d.cache_capacity = 4112;
  d.max_cache_len = 4096;
  d.sm_scale = 0.088f;
  d.dtype = TIDAR_DTYPE_BF16;
  d.num_splits = 0;
  return d;
}

static int attn(const tidar_attn_desc* d, void* ws, size_t ws_bytes) {
  return tidar_attn_step(d, FAKE, FAKE, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, NULL, NULL, ws,
                         ws_bytes, NULL);
}

static void check_attn(void) {
  struct {
    const char* what;
    int field;
    double value;
    int want;
  } bad[] = {
      {"Hq % Hkv", 1, 30, TIDAR_E_INVALID},       {"Hkv = 0", 2, 0, TIDAR_E_INVALID},
      {"dtype", 10, 7, TIDAR_E_INVALID},          {"bf16 D = 96", 3, 96, TIDAR_E_UNSUPPORTED},
      {"blocks > k+1", 5, 18, TIDAR_E_INVALID},   {"block_len 0", 6, 0, TIDAR_E_INVALID},
      {"max_len > cap", 8, 5000, TIDAR_E_CAPACITY}, {"sm_scale 0", 9, 0.0, TIDAR_E_INVALID},
      {"sm_scale nan", 9, NAN, TIDAR_E_INVALID},  {"splits -1", 11, -1, TIDAR_E_INVALID},
      {"batch 0", 0, 0, TIDAR_E_INVALID},         {"batch -3", 0, -3, TIDAR_E_INVALID},
      {"k -1", 4, -1, TIDAR_E_INVALID},           {"cap -1", 7, -1, TIDAR_E_INVALID},
      {"max_len -1", 8, -1, TIDAR_E_INVALID},     {"sm_scale inf", 9, INFINITY, TIDAR_E_INVALID},
  };
  for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    tidar_attn_desc d = base_desc();
    int32_t* f[] = {&d.batch, &d.num_q_heads, &d.num_kv_heads, &d.head_dim, &d.k, &d.num_blocks,
                    &d.block_len, &d.cache_capacity, &d.max_cache_len, NULL, &d.dtype, &d.num_splits};
    if (bad[i].field == 9)
      d.sm_scale = (float)bad[i].value;
    else
      *f[bad[i].field] = (int32_t)bad[i].value;
    expect(attn(&d, FAKE, (size_t)1 << 30), bad[i].want, bad[i].what);
    if (tidar_attn_workspace_bytes(&d) != 0) {
      fprintf(stderr, "FAIL %s: workspace query of an invalid descriptor is not 0\n", bad[i].what);
      ++failures;
    }
  }
  {
    /* bf16 fields the kernel receives packed in 16 bits: refused on the host */
    tidar_attn_desc w = base_desc();
    w.num_q_heads = 1 << 17;
    w.num_kv_heads = 1 << 17;
    w.k = 0;
    w.num_blocks = 1;
    w.block_len = 1;
    w.cache_capacity = 1;
    w.max_cache_len = 1;
    w.head_dim = 64;
    expect(attn(&w, FAKE, (size_t)1 << 30), TIDAR_E_UNSUPPORTED, "KV heads >= 2^16");
    tidar_attn_desc sp = base_desc(); /* 2^17 forced splits of a 2^24-key cache */
    sp.num_q_heads = 1;
    sp.num_kv_heads = 1;
    sp.head_dim = 64;
    sp.cache_capacity = 1 << 24;
    sp.max_cache_len = 1 << 24;
    sp.num_splits = 1 << 17;
    expect(attn(&sp, FAKE, (size_t)1 << 30), TIDAR_E_UNSUPPORTED, "splits >= 2^16");
  }
  tidar_attn_desc d = base_desc();
  expect(tidar_attn_step(NULL, FAKE, FAKE, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, NULL, NULL, FAKE,
                         1, NULL),
         TIDAR_E_INVALID, "null descriptor");
  expect(tidar_attn_step(&d, NULL, FAKE, FAKE, FAKE, FAKE, (const int32_t*)FAKE, FAKE, NULL, NULL, FAKE,
                         (size_t)1 << 30, NULL),
         TIDAR_E_INVALID, "null q");
  expect(tidar_attn_step(&d, FAKE, FAKE, FAKE, FAKE_OFF(2), FAKE, (const int32_t*)FAKE, FAKE, NULL, NULL,
                         FAKE, (size_t)1 << 30, NULL),
         TIDAR_E_INVALID, "misaligned k_cache");
  const size_t need = tidar_attn_workspace_bytes(&d);
  if (need == 0) {
    fprintf(stderr, "FAIL the Qwen3-8B step shape should need split partials\n");
    ++failures;
  } else {
    expect(attn(&d, FAKE, need - 1), TIDAR_E_WORKSPACE, "workspace one byte short");
    expect(attn(&d, NULL, 0), TIDAR_E_WORKSPACE, "no workspace");
  }

  /* Planning over a sweep of shapes, extreme ones included: every query must
   * return without undefined behaviour (the sanitizer aborts on any). */
  const int32_t batches[] = {1, 2, 8, 64, 4096, 1 << 20, INT32_MAX};
  const int32_t lens[] = {0, 1, 63, 64, 4096, 131072, 1 << 24, INT32_MAX - 64, INT32_MAX};
  const int32_t ks[] = {0, 1, 16, 64};
  const int32_t dtypes[] = {TIDAR_DTYPE_F32, TIDAR_DTYPE_BF16};
  const int32_t splits[] = {0, 1, 7, 1000};
  size_t sink = 0;
  for (size_t a = 0; a < sizeof batches / sizeof batches[0]; ++a)
    for (size_t b = 0; b < sizeof lens / sizeof lens[0]; ++b)
      for (size_t c = 0; c < sizeof ks / sizeof ks[0]; ++c)
        for (size_t e = 0; e < 2; ++e)
          for (size_t s = 0; s < sizeof splits / sizeof splits[0]; ++s) {
            tidar_attn_desc q = base_desc();
            q.batch = batches[a];
            q.cache_capacity = lens[b];
            q.max_cache_len = lens[b];
            q.k = ks[c];
            q.num_blocks = ks[c] > 0 ? ks[c] + 1 : 1;
            q.block_len = ks[c] > 0 ? ks[c] : 1;
            q.dtype = dtypes[e];
            q.num_splits = splits[s];
            const size_t need = tidar_attn_workspace_bytes(&q);
            sink += need;
            /* a descriptor that needs a workspace is refused without one,
             * before any HIP call (one that needs none would launch: skipped) */
            if (need > 0) expect(attn(&q, NULL, 0), TIDAR_E_WORKSPACE, "sweep without workspace");
          }
  printf("attn sweep done (%zu)\n", sink % 7);
}

static void check_commit(void) {
  struct {
    int32_t L, B, H, D, k, rows, cap, maxlen, dtype;
    void *ks, *kc, *acc, *lout;
    int want;
    const char* what;
  } c[] = {
      {36, 1, 8, 128, 16, 288, 4112, 4100, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_CAPACITY, "capacity"},
      {36, 1, 8, 128, 16, 288, 4112, 4096, 1, FAKE, FAKE, FAKE, FAKE, TIDAR_E_INVALID, "aliased lengths"},
      {36, 1, 8, 128, 16, 8, 4112, 4096, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_INVALID, "rows < k"},
      {36, 1, 8, 128, 16, 288, 4112, 4096, 1, FAKE, FAKE, NULL, FAKE_OFF(64), TIDAR_E_INVALID, "null accept"},
      {36, 1, 8, 128, 16, 288, 4112, 4096, 3, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_INVALID, "dtype"},
      {36, 1, 8, 4, 16, 288, 4112, 4096, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_UNSUPPORTED, "8-byte rows"},
      {36, 1, 8, 128, 16, 288, 4112, 4096, 1, FAKE, FAKE_OFF(8), FAKE, FAKE_OFF(64), TIDAR_E_INVALID,
       "misaligned cache"},
      {0, 1, 8, 128, 16, 288, 4112, 4096, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_INVALID, "no layers"},
      {INT32_MAX, INT32_MAX, INT32_MAX, 128, 16, 288, INT32_MAX, INT32_MAX - 16, 1, FAKE, FAKE, FAKE,
       FAKE_OFF(64), TIDAR_E_UNSUPPORTED, "huge grid"},
      {36, 1, 8, 128, INT32_MAX, INT32_MAX, INT32_MAX, 0, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_UNSUPPORTED,
       "k near int max"},
      {36, 1, 8, INT32_MAX - 7, 16, 288, 4112, 4096, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_UNSUPPORTED,
       "head_dim near int max"},
      {36, 1, 8, 128, 16, 288, 4112, -1, 1, FAKE, FAKE, FAKE, FAKE_OFF(64), TIDAR_E_INVALID, "max_len -1"},
  };
  for (size_t i = 0; i < sizeof c / sizeof c[0]; ++i) {
    const int st = tidar_kv_commit(c[i].L, c[i].B, c[i].H, c[i].D, c[i].k, c[i].rows, c[i].cap, c[i].maxlen,
                                   c[i].dtype, c[i].ks, FAKE, c[i].kc, FAKE, (const int32_t*)c[i].acc,
                                   (const int32_t*)FAKE, (int32_t*)c[i].lout, NULL, NULL);
    expect(st, c[i].want, c[i].what);
  }
}

static int reject(int32_t B, int32_t k, int32_t V, const void* ar, const void* drafts, float T, void* ws,
                  size_t wsb) {
  return tidar_reject_sample(B, k, V, (const float*)ar, (const float*)FAKE, (const int32_t*)drafts,
                             (const float*)FAKE, T, (int32_t*)FAKE, (int32_t*)FAKE, NULL, NULL, ws, wsb, NULL);
}

static void check_reject(void) {
  const size_t big = (size_t)1 << 30;
  expect(reject(1, 16, 151936, FAKE, FAKE, 0.f, FAKE, big), TIDAR_E_INVALID, "temperature 0");
  expect(reject(1, 16, 151936, FAKE, FAKE, -1.f, FAKE, big), TIDAR_E_INVALID, "temperature < 0");
  expect(reject(1, 16, 151936, FAKE, FAKE, NAN, FAKE, big), TIDAR_E_INVALID, "temperature nan");
  expect(reject(1, 16, 0, FAKE, FAKE, 1.f, FAKE, big), TIDAR_E_INVALID, "V 0");
  expect(reject(0, 16, 151936, FAKE, FAKE, 1.f, FAKE, big), TIDAR_E_INVALID, "B 0");
  expect(reject(1, -1, 151936, FAKE, FAKE, 1.f, FAKE, big), TIDAR_E_INVALID, "k -1");
  expect(reject(1, 16, 151936, FAKE, NULL, 1.f, FAKE, big), TIDAR_E_INVALID, "null drafts");
  expect(reject(1, 16, 151936, FAKE, FAKE, 1.f, FAKE, 16), TIDAR_E_WORKSPACE, "workspace");
  expect(reject(1, 1000, 151936, FAKE, FAKE, 1.f, FAKE, big), TIDAR_E_UNSUPPORTED, "k too large");
  expect(reject(1, 16, 151936, FAKE_OFF(4), FAKE, 1.f, FAKE, big), TIDAR_E_INVALID, "misaligned logits");
  expect(reject(INT32_MAX, 16, INT32_MAX, FAKE, FAKE, 1.f, FAKE, big), TIDAR_E_UNSUPPORTED, "huge rows");
  const size_t need = tidar_reject_workspace_bytes(1, 16, 151936);
  if (need == 0) {
    fprintf(stderr, "FAIL reject workspace query returned 0\n");
    ++failures;
  } else {
    expect(reject(1, 16, 151936, FAKE, FAKE, 1.f, FAKE, need - 1), TIDAR_E_WORKSPACE, "workspace short");
  }
  const float lams[] = {-0.25f, 1.5f, NAN, INFINITY};
  for (int i = 0; i < 4; ++i)
    expect(tidar_reject_sample_trust(1, 16, 151936, (const float*)FAKE, (const float*)FAKE,
                                     (const int32_t*)FAKE, (const float*)FAKE, 1.f, lams[i], (int32_t*)FAKE,
                                     (int32_t*)FAKE, NULL, NULL, FAKE, big, NULL),
           TIDAR_E_INVALID, "trust weight");
  const int32_t sizes[] = {0, 1, 16, 151936, 1 << 24, INT32_MAX};
  size_t sink = 0;
  for (int a = 0; a < 6; ++a)
    for (int b = 0; b < 6; ++b)
      for (int kk = 0; kk < 4; ++kk) sink += tidar_reject_workspace_bytes(sizes[a], (int32_t[]){0, 1, 16, 200}[kk], sizes[b]);
  printf("reject sweep done (%zu)\n", sink % 7);
}

static void check_logprob(void) {
  const size_t big = (size_t)1 << 30;
  struct {
    int32_t rows, V;
    void *lg, *tg, *ws;
    int want;
    const char* what;
  } c[] = {
      {0, 151936, FAKE, FAKE, FAKE, TIDAR_E_INVALID, "rows 0"},
      {4, 0, FAKE, FAKE, FAKE, TIDAR_E_INVALID, "V 0"},
      {4, 151936, NULL, FAKE, FAKE, TIDAR_E_INVALID, "null logits"},
      {4, 151936, FAKE, NULL, FAKE, TIDAR_E_INVALID, "null targets"},
      {4, 151936, FAKE_OFF(4), FAKE, FAKE, TIDAR_E_INVALID, "misaligned logits"},
      {1 << 20, 151936, FAKE, FAKE, FAKE, TIDAR_E_UNSUPPORTED, "rows * V too large"},
      {INT32_MAX, INT32_MAX, FAKE, FAKE, FAKE, TIDAR_E_UNSUPPORTED, "int max"},
      {4, 151936, FAKE, FAKE, FAKE_OFF(16), TIDAR_E_INVALID, "misaligned workspace"},
  };
  for (size_t i = 0; i < sizeof c / sizeof c[0]; ++i)
    expect(tidar_token_logprobs(c[i].rows, c[i].V, (const float*)c[i].lg, (const int32_t*)c[i].tg,
                                (float*)FAKE, NULL, c[i].ws, big, NULL),
           c[i].want, c[i].what);
  const size_t need = tidar_logprob_workspace_bytes(4, 151936);
  expect(tidar_token_logprobs(4, 151936, (const float*)FAKE, (const int32_t*)FAKE, (float*)FAKE, NULL, FAKE,
                              need - 1, NULL),
         TIDAR_E_WORKSPACE, "logprob workspace short");
  const int32_t sizes[] = {-1, 0, 1, 151936, 1 << 24, INT32_MAX};
  size_t sink = 0;
  for (int a = 0; a < 6; ++a)
    for (int b = 0; b < 6; ++b) sink += tidar_logprob_workspace_bytes(sizes[a], sizes[b]);
  printf("logprob sweep done (%zu)\n", sink % 7);
}

int main(void) {
  for (int s = 1; s >= -6; --s)
    if (tidar_status_string(s) == NULL) {
      fprintf(stderr, "FAIL status string %d\n", s);
      ++failures;
    }
  check_attn();
  check_commit();
  check_reject();
  check_logprob();
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
