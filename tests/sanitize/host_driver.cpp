// Host-side checks of libsaga's C ABI, built with the library's host code under
// AddressSanitizer and UndefinedBehaviorSanitizer and run on a CPU (no GPU): every
// entry point's argument checks (each returns its error before anything touches the
// GPU), the workspace-size arithmetic, and Theorem 4.2's pairing on the host
// (saga_min_weight_pairing) against a brute-force enumeration of perfect matchings.
// Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "saga.h"

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static char g_dummy[64];
static void* const FAKE = g_dummy;  // a non-null pointer that is never dereferenced

static saga_shape shape(int batch = 1, int h_q = 12, int h_k = 1, int h_v = 4, int d = 128, int d_v = 0,
                        int l_max = 131072, int dtype = SAGA_BF16) {
  saga_shape s;
  s.batch = batch;
  s.h_q = h_q;
  s.h_k = h_k;
  s.h_v = h_v;
  s.d = d;
  s.d_v = d_v;
  s.l_max = l_max;
  s.dtype = dtype;
  s.out_dtype = dtype;
  s.scale = 0.f;
  return s;
}

static int decode(const saga_shape* s, int N = 8, int period = 4, long long step = 1, size_t ws = (size_t)1 << 40,
                  int max_l = 1024, float* tau = (float*)FAKE, int32_t* sel_idx = nullptr, int cap = 0) {
  return saga_decode_attn(s, FAKE, FAKE, FAKE, (const int32_t*)FAKE, max_l, N, period, step, tau, FAKE, nullptr,
                          sel_idx, cap, nullptr, FAKE, ws, nullptr);
}

// least total weight over every perfect matching (pair the lowest free vertex first)
static double brute(int n, const std::vector<float>& w, unsigned used) {
  int i = 0;
  while (i < n && (used >> i) & 1u) ++i;
  if (i == n) return 0.0;
  double best = INFINITY;
  for (int j = i + 1; j < n; ++j)
    if (!((used >> j) & 1u)) {
      const double t = (double)w[i * n + j] + brute(n, w, used | (1u << i) | (1u << j));
      if (t < best) best = t;
    }
  return best;
}

int main() {
  // status names
  CHECK(std::strcmp(saga_status_str(SAGA_OK), "SAGA_OK") == 0);
  CHECK(std::strcmp(saga_status_str(SAGA_ERR_HIP), "SAGA_ERR_HIP") == 0);
  CHECK(std::strcmp(saga_status_str(-3), "SAGA_ERR_UNKNOWN") == 0);

  // workspace sizes: valid shapes > 0 and non-decreasing in max_l_kv; invalid ones 0
  const saga_shape shapes[] = {shape(), shape(3), shape(1, 32, 2, 8, 64), shape(1, 12, 1, 4, 128, 0, 131072, SAGA_F32),
                               shape(1, 32, 4, 8, 32, 64), shape(2, 12, 2, 4, 64, 128)};
  for (const saga_shape& s : shapes) {
    size_t prev = 0;
    for (int L : {0, 1, 127, 128, 129, 4095, 4096, 16384, 65536, 98304, 131071, 131072}) {
      const size_t n = saga_workspace_bytes(&s, 512, L);
      CHECK(n > 0);
      CHECK(n >= prev);
      prev = n;
    }
  }
  {
    saga_shape s = shape();
    CHECK(saga_workspace_bytes(nullptr, 8, 16) == 0);
    CHECK(saga_workspace_bytes(&s, 0, 16) == 0);
    CHECK(saga_workspace_bytes(&s, 8, 131073) == 0);
    s.h_k = 5;
    CHECK(saga_workspace_bytes(&s, 8, 16) == 0);
    s = shape();
    s.d = 96;
    CHECK(saga_workspace_bytes(&s, 8, 16) == 0);
    s = shape();
    s.scale = NAN;
    CHECK(saga_workspace_bytes(&s, 8, 16) == 0);
    s = shape(1 << 16);
    CHECK(saga_workspace_bytes(&s, 8, 16) == 0);
  }

  // decode step: every host-side refusal
  {
    const saga_shape s = shape();
    saga_shape bad = s;
    CHECK(decode(nullptr) == SAGA_ERR_NULL);
    CHECK(decode(&s, 8, 4, 1, (size_t)1 << 40, 1024, nullptr) == SAGA_ERR_NULL);
    bad.h_k = 5;
    CHECK(decode(&bad) == SAGA_ERR_SHAPE);
    bad = s;
    bad.batch = 0;
    CHECK(decode(&bad) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 0) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 0) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 4, -1) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 4, 1, (size_t)1 << 40, 131073) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 4, 1, (size_t)1 << 40, -1) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 4, 1, (size_t)1 << 40, 1024, (float*)FAKE, (int32_t*)FAKE, 0) == SAGA_ERR_SHAPE);
    CHECK(decode(&s, 8, 4, 1, 16) == SAGA_ERR_WORKSPACE);
    bad = s;
    bad.dtype = 7;
    CHECK(decode(&bad) == SAGA_ERR_UNSUPPORTED);
    // the no-allocation form: the same checks, and a step larger than its scratch
    CHECK(saga_decode_attn_noalloc(nullptr, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 16, 8, 4, 1, (float*)FAKE, FAKE,
                                   nullptr, nullptr, 0, nullptr, nullptr) == SAGA_ERR_NULL);
    const saga_shape big = shape(4);
    CHECK(saga_workspace_bytes(&big, 512, 131072) > SAGA_NOALLOC_SCRATCH_BYTES);
    CHECK(saga_decode_attn_noalloc(&big, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 131072, 512, 32, 0, (float*)FAKE,
                                   FAKE, nullptr, nullptr, 0, nullptr, nullptr) == SAGA_ERR_WORKSPACE);
    CHECK(saga_decode_attn_noalloc(&s, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 16, 8, 0, 1, (float*)FAKE, FAKE,
                                   nullptr, nullptr, 0, nullptr, nullptr) == SAGA_ERR_SHAPE);
  }

  // the other entry points' refusals
  {
    const saga_shape s = shape();
    CHECK(saga_refresh_threshold(&s, FAKE, FAKE, (const int32_t*)FAKE, 1024, 0, (float*)FAKE, FAKE, 1u << 30,
                                 nullptr) == SAGA_ERR_SHAPE);
    saga_shape d = shape(1, 8, 4, 2, 64);  // h_k > h_v: the dense call needs h_k | h_v
    CHECK(saga_dense_gqa_attn(&d, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 1024, FAKE, FAKE, 1u << 30, nullptr) ==
          SAGA_ERR_UNSUPPORTED);
    CHECK(saga_qk_select(&s, FAKE, FAKE, (const int32_t*)FAKE, 1024, nullptr, FAKE, 1u << 30, nullptr) ==
          SAGA_ERR_NULL);
    CHECK(saga_select_gather(&s, FAKE, FAKE, nullptr, (const int32_t*)FAKE, 1024, 8, (const float*)FAKE, FAKE,
                             1u << 30, nullptr) == SAGA_ERR_NULL);
    CHECK(saga_select_gather(&s, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 1024, 0, (const float*)FAKE, FAKE,
                             1u << 30, nullptr) == SAGA_ERR_SHAPE);
    // the gather form: late for a head keeping about 1 entry per chunk, early for dense
    // selections and rows of more than 512 chunks, -1 for invalid arguments
    CHECK(saga_gather_form(&s, 512, 131072) == 1);
    CHECK(saga_gather_form(&s, 2048, 4096) == 0);
    CHECK(saga_gather_form(&s, 0, 4096) == -1);
    CHECK(saga_gather_form(nullptr, 8, 4096) == -1);
    saga_pages pg;
    pg.table = (const int32_t*)FAKE;
    pg.max_pages = 4;
    pg.page_tokens = 24;  // not a power of two
    pg.num_pages = 8;
    CHECK(saga_decode_attn_paged(&s, &pg, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 64, 8, 4, 1, (float*)FAKE, FAKE,
                                 nullptr, nullptr, 0, nullptr, FAKE, 1u << 30, nullptr) == SAGA_ERR_SHAPE);
    pg.page_tokens = 16;
    CHECK(saga_decode_attn_paged(&s, &pg, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 65, 8, 4, 1, (float*)FAKE, FAKE,
                                 nullptr, nullptr, 0, nullptr, FAKE, 1u << 30, nullptr) == SAGA_ERR_SHAPE);
    CHECK(saga_decode_attn_paged(&s, nullptr, FAKE, FAKE, FAKE, (const int32_t*)FAKE, 64, 8, 4, 1, (float*)FAKE, FAKE,
                                 nullptr, nullptr, 0, nullptr, FAKE, 1u << 30, nullptr) == SAGA_ERR_NULL);
    CHECK(saga_linear(1, 33, 8, FAKE, FAKE, FAKE, SAGA_BF16, nullptr) == SAGA_ERR_SHAPE);
    saga_layer L;
    L.attn = shape(1, 12, 1, 4, 128, 0, 4096);
    L.d_model = 1536;
    CHECK(saga_layer_workspace_bytes(&L, 64, 4096) > saga_workspace_bytes(&L.attn, 64, 4096));
    L.d_model = 1537;
    CHECK(saga_layer_workspace_bytes(&L, 64, 4096) == 0);
    saga_merge_shape m;
    m.tokens = 512;
    m.d_model = 2048;
    m.h_q = 32;
    m.h_k = 8;
    m.d = 64;
    CHECK(saga_merge_workspace_bytes(&m) > 0);
    m.h_k = 7;
    CHECK(saga_merge_workspace_bytes(&m) == 0);
    m.h_k = 8;
    m.d = 96;
    CHECK(saga_merge_workspace_bytes(&m) == 0);
  }

  // Theorem 4.2 on the host: the pairing's total is the brute-force minimum, and the
  // partner array is a perfect matching of that total
  {
    std::mt19937 rng(1234);
    std::uniform_real_distribution<float> U(0.f, 10.f);
    for (int n = 2; n <= 16; n += 2) {
      for (int rep = 0; rep < (n <= 10 ? 20 : 3); ++rep) {
        std::vector<float> w((size_t)n * n, 0.f);
        for (int a = 0; a < n; ++a)
          for (int b = a + 1; b < n; ++b) w[a * n + b] = w[b * n + a] = rep % 5 == 0 ? std::floor(U(rng)) : U(rng);
        std::vector<int32_t> partner(n, -1);
        double total = -1.0;
        CHECK(saga_min_weight_pairing(n, w.data(), partner.data(), &total) == SAGA_OK);
        double sum = 0.0;
        for (int a = 0; a < n; ++a) {
          const int p = partner[a];
          CHECK(p >= 0 && p < n && p != a && partner[p] == a);
          if (p > a) sum += w[a * n + p];
        }
        CHECK(std::fabs(sum - total) <= 1e-9 * (1.0 + std::fabs(total)));
        if (n <= 10) CHECK(std::fabs(total - brute(n, w, 0u)) <= 1e-9 * (1.0 + std::fabs(total)));
      }
    }
    std::vector<float> w(16, 1.f);
    std::vector<int32_t> partner(16);
    CHECK(saga_min_weight_pairing(3, w.data(), partner.data(), nullptr) == SAGA_ERR_SHAPE);
    CHECK(saga_min_weight_pairing(18, w.data(), partner.data(), nullptr) == SAGA_ERR_SHAPE);
    CHECK(saga_min_weight_pairing(4, nullptr, partner.data(), nullptr) == SAGA_ERR_NULL);
    w[1] = NAN;
    CHECK(saga_min_weight_pairing(4, w.data(), partner.data(), nullptr) == SAGA_ERR_SHAPE);
  }

  std::printf("host checks: %d failed\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
