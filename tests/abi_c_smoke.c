/* Plain C (C11) client of the library's host-side entry points: the header
 * compiles as C, the symbols link with a C toolchain, and the layout of the
 * FSDP1 worked example (page "Infra: Data Parallel", section "FSDP1": three
 * (4, 2) weights flattened, concatenated and split evenly over 2 ranks, the
 * cut passing through the second weight) comes out as the page draws it.
 * Launches nothing (no GPU needed). */
#include <stdio.h>
#include <stdlib.h>

#include "zero_shard.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  const int64_t numel[3] = {8, 8, 8};
  zero_layout* L[2] = {NULL, NULL};
  for (int r = 0; r < 2; ++r) CHECK(zero_layout_create(numel, 3, 0, 2, r, &L[r]) == ZERO_OK);
  CHECK(zero_layout_kind(L[0]) == 0);
  CHECK(zero_layout_psi(L[0]) == 24 && zero_layout_padded(L[0]) == 24);
  CHECK(zero_layout_shard(L[0]) == 12 && zero_layout_n_buckets(L[0]) == 1);
  CHECK(zero_layout_n_d(L[1]) == 2 && zero_layout_rank(L[1]) == 1);

  int64_t so, len, po, pl, sh;
  CHECK(zero_layout_bucket(L[1], 0, &so, &len, &po, &pl, &sh) == ZERO_OK);
  CHECK(so == 0 && len == 24 && po == 0 && pl == 24 && sh == 0);
  CHECK(zero_layout_bucket(L[1], 1, &so, NULL, NULL, NULL, NULL) == ZERO_ERANGE);

  /* rank 0 holds W1 and the first half of W2; rank 1 the rest of W2 and W3 */
  /* an empty range is reported as [0, 0) */
  const int64_t lo0[3] = {0, 8, 0}, hi0[3] = {8, 12, 0};
  const int64_t lo1[3] = {0, 0, 4}, hi1[3] = {0, 4, 12};
  for (int t = 0; t < 3; ++t) {
    int64_t s0, lo, hi;
    CHECK(zero_layout_tensor(L[0], t, &s0, &lo, &hi) == ZERO_OK);
    CHECK(s0 == 8 * t && lo == lo0[t] && hi == hi0[t]);
    CHECK(zero_layout_tensor(L[1], t, &s0, &lo, &hi) == ZERO_OK);
    CHECK(s0 == 8 * t && lo == lo1[t] && hi == hi1[t]);
  }

  /* FSDP2: the (8, 4) weight over 4 ranks gives local (2, 4) pieces */
  const int64_t n2[1] = {32}, rows2[1] = {8};
  zero_layout* D = NULL;
  CHECK(zero_layout_create_dim0(n2, rows2, 1, 4, 2, &D) == ZERO_OK);
  CHECK(zero_layout_kind(D) == 1 && zero_layout_shard(D) == 8);
  CHECK(zero_layout_bucket(D, 0, &so, &len, &po, &pl, &sh) == ZERO_OK);
  CHECK(pl == 32 && sh == 0);

  zero_adamw hp = {1e-3, 0.9, 0.95, 1e-8, 0.1};
  float k[8];
  CHECK(zero_step_scalars(&hp, 1, k) == ZERO_OK);
  CHECK(k[3] == 0.9f && k[5] == 0.95f && k[7] == 1e-8f);
  CHECK(zero_step_scalars(&hp, 0, k) == ZERO_EINVAL);

  int64_t nb[3] = {100, 200, 300}, off[3], pool = -1;
  double tr[3] = {1.0, 1.0, 1.0};
  CHECK(zero_placement_plan(3, nb, tr, 1024, 3, 16, off, &pool) == ZERO_OK);
  CHECK(off[0] == 0 && off[1] == 1024 && off[2] == 2048 && pool == 2348);

  /* invalid calls fail on the host before any launch */
  CHECK(zero_layout_create(NULL, 3, 0, 2, 0, &D) == ZERO_EINVAL);
  CHECK(zero_layout_create(numel, 3, 0, 2, 2, &D) == ZERO_ERANGE);
  CHECK(zero_shard_step(NULL, &hp, 1, NULL, 0, NULL, NULL, NULL, NULL, 0, NULL, NULL) ==
        ZERO_EINVAL);
  CHECK(zero_grad_accumulate(NULL, NULL, -1, 1.0f, 0, NULL, NULL) == ZERO_EINVAL);
  CHECK(zero_strerror(ZERO_EOVERLAP) != NULL);

  zero_layout_destroy(L[0]);
  zero_layout_destroy(L[1]);
  zero_layout_destroy(D);
  printf("ok\n");
  return 0;
}
