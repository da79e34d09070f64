// Host-side driver of libtq's host code (tq_host.cpp: codebooks, layer
// randomness, descriptors, sizing, validation messages), built with the
// address, undefined-behaviour or thread sanitizer by
// tests/test_host_sanitize.py.  Every host entry point is called with valid
// arguments (checking properties that hold by definition) and with invalid
// ones (which must fail with a negative status and a message); several host
// threads then run the same calls at once.  Exit status 0 = every check held.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <thread>
#include <vector>

#include "tq.h"

static int g_failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      ++g_failures;                                                          \
    }                                                                        \
  } while (0)

static void codebooks() {
  const int kinds[] = {TQ_CODEBOOK_LLOYD_MAX, TQ_CODEBOOK_UNIFORM, TQ_CODEBOOK_BETA, TQ_CODEBOOK_POLAR};
  for (int kind : kinds) {
    for (int bits = 1; bits <= 8; ++bits) {
      const int L = 1 << bits;
      std::vector<float> c(L), t(L - 1);
      CHECK(tq_build_codebook(bits, kind, c.data(), t.data()) == TQ_OK);
      for (int k = 0; k + 1 < L; ++k) {
        CHECK(c[k] < c[k + 1]);
        CHECK(c[k] <= t[k] && t[k] <= c[k + 1]);
      }
      if (kind != TQ_CODEBOOK_POLAR)
        for (int k = 0; k < L; ++k) CHECK(c[k] == -c[L - 1 - k]);   // symmetric about 0
    }
    std::vector<float> table(TQ_CODEBOOK_TABLE_FLOATS);
    CHECK(tq_codebook_table(kind, table.data()) == TQ_OK);
    for (float f : table) CHECK(isfinite(f) || f == 3e38f);
  }
  float c[256], t[255];
  CHECK(tq_build_codebook(0, TQ_CODEBOOK_LLOYD_MAX, c, t) < 0);
  CHECK(tq_build_codebook(9, TQ_CODEBOOK_LLOYD_MAX, c, t) < 0);
  CHECK(tq_build_codebook(3, 17, c, t) < 0);
  CHECK(tq_build_codebook(3, TQ_CODEBOOK_LLOYD_MAX, nullptr, t) < 0);
  CHECK(strlen(tq_last_error()) > 0);
  CHECK(tq_codebook_table(TQ_CODEBOOK_FITTED, nullptr) < 0);
}

static void layer_randomness() {
  int8_t s[128];
  std::vector<float> S(128 * 128);
  CHECK(tq_layer_params(42, 0, 128, 128, s, S.data()) == TQ_OK);
  int minus = 0;
  for (int j = 0; j < 128; ++j) {
    CHECK(s[j] == 1 || s[j] == -1);
    minus += s[j] < 0;
  }
  CHECK(minus > 32 && minus < 96);
  double sum2 = 0;
  for (float f : S) {
    CHECK(isfinite(f));
    sum2 += (double)f * f;
  }
  CHECK(fabs(sum2 / S.size() - 1.0) < 0.05);   // N(0, 1) entries
  int8_t s2[128];
  CHECK(tq_layer_params(42, 0, 128, 128, s2, nullptr) == TQ_OK);
  CHECK(memcmp(s, s2, 128) == 0);
  CHECK(tq_layer_params(42, 0, 64, 128, s, nullptr) < 0);
  CHECK(tq_layer_params(42, 0, 128, 96, s, S.data()) < 0);
  uint32_t mask[4];
  CHECK(tq_sign_mask(s, 128, mask) == TQ_OK);
  for (int j = 0; j < 128; ++j) CHECK((((mask[j >> 5] >> (j & 31)) & 1u) != 0) == (s[j] < 0));
  CHECK(tq_sign_mask(s, 100, mask) < 0);
}

static void fitted() {
  int8_t s[128];
  CHECK(tq_layer_params(7, 1, 128, 128, s, nullptr) == TQ_OK);
  const size_t n = 96;
  std::vector<float> X(n * 128);
  unsigned state = 12345u;
  for (float& f : X) {   // a small LCG: uniform in [-1, 1), enough spread for the fit
    state = state * 1664525u + 1013904223u;
    f = (float)((state >> 8) * (2.0 / 16777216.0) - 1.0);
  }
  for (int bits = 1; bits <= 4; ++bits) {
    std::vector<float> c(1 << bits), t((1 << bits) - 1);
    CHECK(tq_fit_codebook(X.data(), n, s, bits, c.data(), t.data()) == TQ_OK);
    for (size_t k = 0; k + 1 < c.size(); ++k) CHECK(c[k] <= c[k + 1]);
  }
  std::vector<float> table(TQ_CODEBOOK_TABLE_FLOATS);
  const int st = tq_calibrated_table(X.data(), n, s, table.data());
  CHECK(st == TQ_OK || st == TQ_ERR_UNSUPPORTED);
  float c[2], t[1];
  CHECK(tq_fit_codebook(X.data(), 0, s, 1, c, t) < 0);
  CHECK(tq_fit_codebook(nullptr, n, s, 1, c, t) < 0);
}

static void descriptors_and_sizes() {
  CHECK(tq_page_bytes(0, 0, 0) == 2 * 64 * 128 * 2);
  CHECK(tq_page_bytes(3, 2, 0) == 1024 * 5 + 512);
  CHECK(tq_page_bytes(2, 2, 1) == 1024 * 4 + 512 + 1280);
  CHECK(tq_page_bytes(9, 2, 0) == 0);
  CHECK(tq_page_bytes(0, 2, 0) == 0);
  const uint64_t d = tq_page_descriptor(4096, 3, 2, 0);
  CHECK(d != 0 && (d & TQ_PAGE_PRESENT) && (d & TQ_PAGE_OFFSET_MASK) == 4096);
  CHECK(tq_page_descriptor(100, 3, 2, 0) == 0);           // not a multiple of 256
  CHECK(tq_page_descriptor(1ull << 48, 3, 2, 0) == 0);    // past 48 bits
  uint64_t pages[3] = {tq_page_descriptor(0, 3, 2, 0), 0, tq_page_descriptor(8192, 0, 0, 0)};
  CHECK(tq_cache_bytes(pages, 3) == tq_page_bytes(3, 2, 0) + tq_page_bytes(0, 0, 0));
  int32_t ntok[2] = {100, 7};
  tq_cache cache = {};
  cache.n_sessions = 2;
  cache.n_kv_heads = 8;
  cache.max_pages = 2;
  cache.n_tokens = ntok;
  cache.pages = pages;
  cache.pool = pages;
  cache.pool_bytes = 1 << 20;
  CHECK(tq_decode_workspace_bytes(&cache, 32) > 0);
  for (int s = -6; s <= 0; ++s) CHECK(tq_status_string(s) != nullptr);
}

static void threads() {
  // several host threads at once: per-thread error messages, no shared state
  std::vector<std::thread> pool;
  std::vector<int> bad(8, 0);
  for (int i = 0; i < 8; ++i)
    pool.emplace_back([i, &bad] {
      float c[256], t[255];
      for (int rep = 0; rep < 3; ++rep) {
        const int bits = 1 + (i + rep) % 8;
        if (tq_build_codebook(bits, i % 3, c, t) != TQ_OK) bad[i] = 1;
        if (tq_build_codebook(0, 0, c, t) >= 0) bad[i] = 1;
        if (strstr(tq_last_error(), "bits") == nullptr && strlen(tq_last_error()) == 0) bad[i] = 1;
        int8_t s[128];
        if (tq_layer_params(42 + i, rep, 128, 128, s, nullptr) != TQ_OK) bad[i] = 1;
      }
    });
  for (auto& th : pool) th.join();
  for (int b : bad) CHECK(b == 0);
}

int main() {
  codebooks();
  layer_randomness();
  fitted();
  descriptors_and_sizes();
  threads();
  if (g_failures) {
    fprintf(stderr, "%d checks failed\n", g_failures);
    return 1;
  }
  printf("host driver: all checks passed\n");
  return 0;
}
