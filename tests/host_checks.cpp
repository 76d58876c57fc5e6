// Host-side checks of libmoe's argument validation, capacity and workspace carving, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the test that
// builds it passes -Xarch_host -fsanitize=...).  Makes no GPU call: every entry point is
// driven only into paths that fail validation before anything is enqueued.  Exits
// nonzero (or the sanitizers abort) on any violation.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {   // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
static int64_t pick(const int64_t* v, int n) { return v[next_u64() % (uint64_t)n]; }

int main() {
  // sizes at and beyond every limit, including values whose products overflow int64
  const int64_t Ts[] = {-1, 0, 1, 7, 4096, 16384, 1 << 20, (int64_t)INT32_MAX / 32,
                        (int64_t)INT32_MAX / 32 + 1, (int64_t)INT32_MAX, (int64_t)1 << 40,
                        INT64_MAX / 2, INT64_MAX};
  const int64_t Ds[] = {-64, 0, 1, 63, 64, 128, 4096, 7168, 65536, 65600, (int64_t)1 << 40,
                        INT64_MAX};
  const int64_t Es[] = {-1, 0, 1, 3, 8, 64, 256, 512, 513, (int64_t)1 << 40, INT64_MAX};
  const int64_t Ks[] = {-1, 0, 1, 2, 8, 16, 17, 1000, INT64_MAX};
  const int64_t Ss[] = {-1, 0, 1, 2, INT64_MAX};
  const float cfs[] = {-1.0f, 0.0f, 1e-45f, 0.01f, 0.7f, 1.0f, 1.25f, 1e10f, 3.0e38f,
                       INFINITY, -INFINITY, NAN};
  int valid = 0;
  for (int it = 0; it < 260000; ++it) {
    moe_desc_t d;
    memset(&d, 0, sizeof d);
    if (it < 200000) {   // anywhere, mostly invalid
      d.T = pick(Ts, 13);
      d.d_model = pick(Ds, 12);
      d.n_experts = pick(Es, 11);
      d.d_ff = pick(Ds, 12);
      d.top_k = pick(Ks, 9);
      d.n_shared = pick(Ss, 5);
      d.dtype = (int32_t)(next_u64() % 3);
      d.out_dtype = (int32_t)(next_u64() % 3);
    } else {             // inside the supported ranges, near their edges
      d.T = (int64_t)(next_u64() % 70000);
      if (next_u64() % 8 == 0) d.T = (int64_t)INT32_MAX / 32 - (int64_t)(next_u64() % 4);
      d.d_model = 64 * (int64_t)(1 + next_u64() % 1024);
      d.d_ff = 64 * (int64_t)(1 + next_u64() % 1024);
      d.n_experts = (int64_t)(1 + next_u64() % 512);
      const int64_t kmax = d.n_experts < 16 ? d.n_experts : 16;
      d.top_k = (int64_t)(1 + next_u64() % (uint64_t)kmax);
      d.n_shared = (int64_t)(next_u64() % 2);
      d.dtype = (int32_t)(next_u64() % 2);
      d.out_dtype = (int32_t)(next_u64() % 2);
    }
    d.capacity_factor = cfs[next_u64() % 12];
    if (next_u64() % 4 == 0) d.capacity_factor = (float)(next_u64() % 100000) / 997.0f;
    const moe_status_t st = moe_validate(&d);
    const size_t ws = moe_workspace_bytes(&d);
    const int64_t C = moe_capacity(&d);
    const size_t wse = moe_workspace_bytes_expert_choice(&d);
    const int64_t Ce = moe_capacity_expert_choice(&d);
    CHECK((st == MOE_OK) == (ws > 0));
    if (st != MOE_OK) {
      CHECK(C == -1 && ws == 0 && wse == 0 && Ce == -1);
      continue;
    }
    ++valid;
    CHECK(ws % 256 == 0);
    if (d.capacity_factor > 0.0f) {
      // k <= C <= max(T k, k)
      CHECK(C >= d.top_k && C <= (d.T * d.top_k > d.top_k ? d.T * d.top_k : d.top_k));
      if (Ce >= 0) CHECK(Ce <= d.T && Ce <= C);
    } else {
      CHECK(C == -1 && Ce == -1 && wse == 0);
    }
    // every entry point rejects a NULL descriptor, NULL required pointers, a missing,
    // misaligned or short workspace, and misaligned tensors, before any launch
    void* fake = (void*)(uintptr_t)0x100000;      // never dereferenced
    void* odd = (void*)(uintptr_t)0x100004;
    CHECK(moe_forward(nullptr, fake, fake, nullptr, fake, fake, fake, fake, nullptr, nullptr,
                      fake, ws, nullptr) == MOE_E_NULL);
    CHECK(moe_forward(&d, fake, nullptr, nullptr, fake, fake, fake, fake, nullptr, nullptr,
                      fake, ws, nullptr) == MOE_E_NULL);
    CHECK(moe_forward(&d, fake, fake, nullptr, fake, fake, fake, fake, nullptr, nullptr,
                      nullptr, ws, nullptr) == MOE_E_WORKSPACE);
    CHECK(moe_forward(&d, fake, fake, nullptr, fake, fake, fake, fake, nullptr, nullptr, fake,
                      ws - 1, nullptr) == MOE_E_WORKSPACE);
    CHECK(moe_forward(&d, fake, fake, nullptr, fake, fake, fake, fake, nullptr, nullptr, odd,
                      ws, nullptr) != MOE_OK);
    CHECK(moe_forward(&d, odd, fake, nullptr, fake, fake, fake, fake, nullptr, nullptr, fake,
                      ws, nullptr) == (d.T > 0 ? MOE_E_UNSUPPORTED : MOE_E_UNSUPPORTED));
    CHECK(moe_route(&d, fake, nullptr, nullptr, (int32_t*)fake, (float*)fake, nullptr, nullptr,
                    nullptr, fake, ws, nullptr) == MOE_E_NULL);
    CHECK(moe_dispatch(&d, (const int32_t*)fake, nullptr, (int32_t*)fake, (int32_t*)fake,
                       (int32_t*)fake, fake, ws, nullptr) == MOE_E_NULL);
    CHECK(moe_experts(&d, fake, (const int32_t*)fake, nullptr, fake, fake, fake, (float*)fake,
                      nullptr, fake, ws, nullptr) == MOE_E_NULL);
    CHECK(moe_combine(&d, (const float*)odd, (const int32_t*)fake, (const float*)fake, fake,
                      nullptr) == (d.T > 0 ? MOE_E_UNSUPPORTED : MOE_E_UNSUPPORTED));
    CHECK(moe_forward_fp8(&d, fake, fake, nullptr, (const uint8_t*)fake, (const uint8_t*)fake,
                          (const uint8_t*)fake, nullptr, nullptr, nullptr, fake, nullptr,
                          nullptr, fake, ws, nullptr) != MOE_OK);
    CHECK(moe_forward_next_best(&d, fake, nullptr, nullptr, fake, fake, fake, fake, nullptr,
                                nullptr, fake, ws, nullptr) != MOE_OK);
    if (wse > 0)
      CHECK(moe_forward_expert_choice(&d, fake, fake, fake, fake, fake, fake, nullptr, nullptr,
                                      fake, wse - 1, nullptr) == MOE_E_WORKSPACE);
    if (ws > MOE_NOALLOC_SCRATCH_BYTES)
      CHECK(moe_forward_noalloc(&d, fake, fake, nullptr, fake, fake, fake, fake, nullptr,
                                nullptr, nullptr) == MOE_E_SCRATCH);
  }
  // workspace monotone in T
  moe_desc_t a = {100, 256, 8, 512, 2, 1, 1.25f, MOE_DTYPE_BF16, MOE_DTYPE_BF16};
  size_t prev = 0;
  for (int64_t T = 0; T < 100000; T = T * 3 + 1) {
    a.T = T;
    const size_t w = moe_workspace_bytes(&a);
    CHECK(w >= prev);
    prev = w;
  }
  for (int s = 0; s <= 6; ++s) CHECK(strncmp(moe_status_str((moe_status_t)s), "MOE_", 4) == 0);
  printf("host checks: %d valid descriptors of 260000, %d failures\n", valid, failures);
  return failures ? 1 : 0;
}
