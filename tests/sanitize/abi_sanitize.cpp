// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: argument validation of every entry point (which
// answers before any HIP call), the status strings, and the draft-length
// controller (host code only) driven through many batches.  Built host-only
// (no device code), so it runs without a GPU; prints "ok" and exits 0 when
// every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "specverify.h"

static int g_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);            \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

int main() {
  void* F = reinterpret_cast<void*>(0x1000);  // never dereferenced: validation fails first
  const int32_t* FI = reinterpret_cast<const int32_t*>(F);
  const float* FF = reinterpret_cast<const float*>(F);
  int32_t* OI = reinterpret_cast<int32_t*>(F);
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();

  // sv_spec_verify
  auto V = [&](int32_t B, int32_t K, int32_t Vv, float T, int32_t tk, float tp, int32_t dt, const void* t,
               const void* d, const int32_t* x, const float* u, int32_t* ot, int32_t* on) {
    return sv_spec_verify(t, d, x, u, T, tk, tp, ot, on, B, K, Vv, dt, nullptr);
  };
  CHECK(V(-1, 3, 16, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_SHAPE);
  CHECK(V(2, SV_MAX_K + 1, 16, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_SHAPE);
  CHECK(V(2, 3, 0, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_SHAPE);
  CHECK(V(2, 3, SV_MAX_V + 1, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_SHAPE);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, 9, F, F, FI, FF, OI, OI) == SV_ERR_DTYPE);
  CHECK(V(2, 3, 16, -1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, nan, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, inf, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, 1e-45f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, 1.f, -2, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, 1.f, 0, 0.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, 1.f, 0, nan, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_PARAM);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, nullptr, F, FI, FF, OI, OI) == SV_ERR_NULL);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, F, nullptr, FI, FF, OI, OI) == SV_ERR_NULL);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, F, F, nullptr, FF, OI, OI) == SV_ERR_NULL);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, F, F, FI, nullptr, OI, OI) == SV_ERR_NULL);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, nullptr, OI) == SV_ERR_NULL);
  CHECK(V(2, 3, 16, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, nullptr) == SV_ERR_NULL);
  CHECK(V(1 << 30, 64, 1 << 20, 1.f, 0, 1.f, SV_F32, F, F, FI, FF, OI, OI) == SV_ERR_SHAPE);
  CHECK(V(0, 3, 16, 1.f, 0, 1.f, SV_F32, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SV_OK);
  CHECK(V(2, 3, 16, 0.f, 0, 1.f, SV_F32, F, nullptr, FI, nullptr, OI, OI) == SV_ERR_NULL);

  // the variants
  CHECK(sv_spec_verify_dt(F, F, FI, FF, 1.f, 0.f, 0, 1.f, OI, OI, nullptr, nullptr, nullptr, 2, 3, 16, SV_F32,
                          nullptr) == SV_ERR_PARAM);
  CHECK(sv_spec_verify_dt(F, F, FI, FF, 1.f, nan, 0, 1.f, OI, OI, nullptr, nullptr, nullptr, 2, 3, 16, SV_F32,
                          nullptr) == SV_ERR_PARAM);
  CHECK(sv_spec_verify_ragged(F, F, FI, FF, FI, 1.f, 1.f, 0, 1.f, OI, OI, nullptr, nullptr, nullptr, 2, 9, 4, 16,
                              SV_F32, nullptr) == SV_ERR_SHAPE);  // total_draft > B * max_k
  CHECK(sv_spec_verify_ragged(F, F, FI, FF, nullptr, 1.f, 1.f, 0, 1.f, OI, OI, nullptr, nullptr, nullptr, 2, 5, 4,
                              16, SV_F32, nullptr) == SV_ERR_NULL);
  CHECK(sv_spec_verify_probs(F, nullptr, FI, FF, 1.f, 0, 1.f, OI, OI, nullptr, nullptr, nullptr, 2, 3, 16, SV_F32,
                             nullptr) == SV_ERR_NULL);
  CHECK(sv_filtered_probs(F, -1, 10, SV_F32, 1.f, 0, 1.f, reinterpret_cast<float*>(F), nullptr) == SV_ERR_SHAPE);
  CHECK(sv_filtered_probs(F, 4, 10, SV_F32, 0.f, 0, 1.f, reinterpret_cast<float*>(F), nullptr) == SV_ERR_PARAM);
  CHECK(sv_sample(F, FF, 1.f, 0, 1.f, OI, nullptr, 4, 10, 5, nullptr) == SV_ERR_DTYPE);
  CHECK(sv_sample(nullptr, FF, 1.f, 0, 1.f, OI, nullptr, 4, 10, SV_F32, nullptr) == SV_ERR_NULL);
  CHECK(sv_spec_verify_noalloc(F, F, FI, FF, 1.f, 0, 1.f, OI, OI, -1, 3, 16, SV_F32, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_read_floor(F, -16, 0u, reinterpret_cast<uint32_t*>(F), nullptr) == SV_ERR_SHAPE);
  CHECK(sv_read_floor(F, 24, 0u, reinterpret_cast<uint32_t*>(F), nullptr) == SV_ERR_SHAPE);
  CHECK(sv_read_floor(nullptr, 0, 0u, nullptr, nullptr) == SV_OK);
  CHECK(sv_init(-1, nullptr, 1, 1, 16, 0) == SV_ERR_PARAM);
  CHECK(sv_init(0, nullptr, -1, 1, 16, 0) == SV_ERR_SHAPE);
  CHECK(sv_init(0, nullptr, 1, 1, 16, 99) == SV_ERR_PARAM);

  // status strings and version
  for (int c = -8; c <= 2; ++c) CHECK(sv_status_string(c) != nullptr && std::strlen(sv_status_string(c)) > 0);
  CHECK(sv_version() >= 100);

  // the draft-length controller: bad arguments, then many batches on many lanes
  CHECK(sv_dynk_create(0, 100, 0.8, 0.6, 2, 10, 5) == nullptr);
  CHECK(sv_dynk_create(4, 0, 0.8, 0.6, 2, 10, 5) == nullptr);
  CHECK(sv_dynk_observe(nullptr, nullptr, nullptr, nullptr) == SV_ERR_NULL);
  CHECK(sv_dynk_k(nullptr, 0) == -1);
  sv_dynk_destroy(nullptr);
  const int lanes = 37;
  sv_dynk* c = sv_dynk_create(lanes, 7, 0.8, 0.6, 2, 10, 5);
  CHECK(c != nullptr);
  if (c) {
    std::vector<int64_t> acc(lanes), dr(lanes);
    std::vector<int32_t> kn(lanes);
    uint64_t s = 12345;
    for (int it = 0; it < 2000; ++it) {
      for (int l = 0; l < lanes; ++l) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        const int32_t k = sv_dynk_k(c, l);
        CHECK(k >= 2 && k <= 10);
        dr[l] = (it % 11 == 0 && l % 5 == 0) ? 0 : k;  // some lanes draft nothing
        acc[l] = dr[l] ? (int64_t)((s >> 33) % (uint64_t)(dr[l] + 1)) : 0;
      }
      CHECK(sv_dynk_observe(c, acc.data(), dr.data(), (it & 1) ? kn.data() : nullptr) == SV_OK);
    }
    CHECK(sv_dynk_k(c, lanes) == -1);
    CHECK(sv_dynk_k(c, -1) == -1);
    acc[3] = dr[3] + 1;  // more accepted than drafted: rejected, nothing recorded
    CHECK(sv_dynk_observe(c, acc.data(), dr.data(), kn.data()) == SV_ERR_PARAM);
    sv_dynk_destroy(c);
  }

  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}
