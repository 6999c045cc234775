// Host-side code of the library (layout planner, placement planner) driven
// with many random and edge-case arguments, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.  Checks the
// layout invariants on the way; prints "ok" on success.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "zero_shard.h"

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

static void exercise(zero_layout* L, int32_t nt) {
  const int64_t P = zero_layout_padded(L), S = zero_layout_shard(L), nb = zero_layout_n_buckets(L);
  const int32_t nd = zero_layout_n_d(L);
  CHECK(P == (int64_t)nd * S);
  int64_t sum_p = 0, sum_s = 0;
  for (int64_t b = 0; b < nb; ++b) {
    int64_t so, len, po, pl, sh;
    CHECK(zero_layout_bucket(L, b, &so, &len, &po, &pl, &sh) == ZERO_OK);
    CHECK(pl % nd == 0 && pl - len >= 0 && po == sum_p && sh == sum_s);
    sum_p += pl;
    sum_s += pl / nd;
  }
  CHECK(sum_p == P && sum_s == S);
  CHECK(zero_layout_bucket(L, nb, nullptr, nullptr, nullptr, nullptr, nullptr) == ZERO_ERANGE);
  for (int32_t t = 0; t < nt; ++t) {
    int64_t so, lo, hi;
    CHECK(zero_layout_tensor(L, t, &so, &lo, &hi) == ZERO_OK);
    CHECK(0 <= lo && lo <= hi && hi <= S);
  }
  CHECK(zero_layout_tensor(L, nt, nullptr, nullptr, nullptr) == ZERO_ERANGE);
}

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) {
    return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
  };
  for (int it = 0; it < 3000; ++it) {
    const int32_t nt = (int32_t)uni(0, 12);
    std::vector<int64_t> numel(nt), rows(nt);
    for (int32_t t = 0; t < nt; ++t) {
      rows[t] = uni(0, 9);
      const int64_t cols = uni(1, 7);
      numel[t] = rows[t] * cols;
    }
    const int32_t nd = (int32_t)uni(1, it % 10 == 0 ? 300 : 9);
    const int32_t rank = (int32_t)uni(0, nd + 1);  // sometimes out of range
    const int64_t cap = uni(-1, 40);
    zero_layout* L = nullptr;
    const int rc = zero_layout_create(nt ? numel.data() : nullptr, nt, cap, nd, rank, &L);
    if (nd > ZERO_MAX_ND) {
      CHECK(rc == ZERO_EINVAL);
    } else if (rank >= nd) {
      CHECK(rc == ZERO_ERANGE);
    } else if (rc == ZERO_OK) {
      CHECK(zero_layout_kind(L) == 0);
      exercise(L, nt);
      zero_layout_destroy(L);
    } else {
      CHECK(nt == 0 && rc == ZERO_EINVAL);  // null numel with n_tensors 0 may be rejected
    }
    zero_layout* D = nullptr;
    const int rd = zero_layout_create_dim0(nt ? numel.data() : nullptr, nt ? rows.data() : nullptr,
                                           nt, nd, rank, &D);
    if (rd == ZERO_OK) {
      CHECK(zero_layout_kind(D) == 1);
      exercise(D, nt);
      zero_layout_destroy(D);
    }
  }
  // placement planner
  for (int it = 0; it < 2000; ++it) {
    const int32_t n = (int32_t)uni(0, 40);
    std::vector<int64_t> nb(n), off(n);
    std::vector<double> tr(n);
    for (int32_t k = 0; k < n; ++k) {
      nb[k] = uni(0, 5000);
      tr[k] = (double)uni(0, 9);
    }
    int64_t pool = -1;
    const int64_t lane = 1024 * uni(1, 4);
    const int32_t lanes = (int32_t)uni(1, 5);
    const int rc = zero_placement_plan(n, n ? nb.data() : nullptr, n ? tr.data() : nullptr, lane,
                                       lanes, 16, n ? off.data() : nullptr, &pool);
    CHECK(rc == ZERO_OK);
    for (int32_t a = 0; a < n; ++a) {
      CHECK(off[a] % 16 == 0 && off[a] + nb[a] <= pool);
      for (int32_t b = a + 1; b < n; ++b)
        CHECK(nb[a] == 0 || nb[b] == 0 || off[a] + nb[a] <= off[b] || off[b] + nb[b] <= off[a]);
    }
  }
  CHECK(zero_layout_create(nullptr, 3, 0, 2, 0, nullptr) == ZERO_EINVAL);
  zero_layout_destroy(nullptr);
  CHECK(zero_layout_padded(nullptr) == -1);
  std::printf("ok\n");
  return 0;
}
