/* Plain C (C11) client that runs the shard step on the GPU without PyTorch:
 * device memory from hipMalloc, the step through the C ABI, results written
 * to a file for tests/test_abi_c.py to compare with the CPU oracle.
 * Usage: abi_c_step <output file> */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "zero_shard.h"

#define HIP_OK(x)                                               \
  do {                                                          \
    if ((x) != hipSuccess) {                                    \
      fprintf(stderr, "HIP error at line %d\n", __LINE__);      \
      return 2;                                                 \
    }                                                           \
  } while (0)

static uint32_t lcg(uint32_t* s) { return *s = *s * 1664525u + 1013904223u; }

/* a small value with a spread of exponents, as a binary32 pattern */
static float small_value(uint32_t* s, float scale) {
  const float u = (float)(lcg(s) >> 8) / 16777216.0f - 0.5f;
  return u * scale;
}

int main(int argc, char** argv) {
  if (argc != 2) return 1;
  const int64_t numel[4] = {1000, 37, 4096, 3};
  const int32_t nd = 4;
  zero_layout* L = NULL;
  if (zero_layout_create(numel, 4, 1500, nd, 3, &L) != ZERO_OK) return 1;
  const int64_t S = zero_layout_shard(L);
  uint32_t seed = 12345u;
  uint16_t* g = (uint16_t*)malloc(sizeof(uint16_t) * nd * S);
  float* st = (float*)malloc(sizeof(float) * 3 * S);
  for (int64_t i = 0; i < nd * S; ++i) {
    float x = small_value(&seed, 2e-3f);
    uint32_t b;
    memcpy(&b, &x, 4);
    g[i] = (uint16_t)(b >> 16); /* bf16 by truncation: an input convention */
  }
  for (int64_t i = 0; i < S; ++i) {
    st[i] = small_value(&seed, 0.04f);
    st[S + i] = small_value(&seed, 2e-4f);
    const float v = small_value(&seed, 2e-6f);
    st[2 * S + i] = v < 0 ? -v : v;
  }
  void *dg, *dst, *dp, *dgo;
  HIP_OK(hipMalloc(&dg, sizeof(uint16_t) * nd * S));
  HIP_OK(hipMalloc(&dst, sizeof(float) * 3 * S));
  HIP_OK(hipMalloc(&dp, sizeof(uint16_t) * S));
  HIP_OK(hipMalloc(&dgo, sizeof(float) * S));
  HIP_OK(hipMemcpy(dg, g, sizeof(uint16_t) * nd * S, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dst, st, sizeof(float) * 3 * S, hipMemcpyHostToDevice));
  const uint16_t* ranks[4];
  for (int q = 0; q < nd; ++q) ranks[q] = (const uint16_t*)dg + q * S;
  float* m = (float*)dst;
  zero_adamw hp = {1e-3, 0.9, 0.95, 1e-8, 0.1};
  for (int64_t t = 1; t <= 3; ++t)
    if (zero_shard_step(L, &hp, t, ranks, ZERO_GRAD_COMPACT, m, m + S, m + 2 * S, (uint16_t*)dp,
                        ZERO_OUT_SHARD, (float*)dgo, NULL) != ZERO_OK)
      return 3;
  HIP_OK(hipDeviceSynchronize());
  float* out_st = (float*)malloc(sizeof(float) * 3 * S);
  uint16_t* out_p = (uint16_t*)malloc(sizeof(uint16_t) * S);
  float* out_g = (float*)malloc(sizeof(float) * S);
  HIP_OK(hipMemcpy(out_st, dst, sizeof(float) * 3 * S, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_p, dp, sizeof(uint16_t) * S, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_g, dgo, sizeof(float) * S, hipMemcpyDeviceToHost));
  FILE* f = fopen(argv[1], "wb");
  if (!f) return 4;
  fwrite(&S, sizeof(S), 1, f);
  fwrite(g, sizeof(uint16_t), (size_t)(nd * S), f);
  fwrite(st, sizeof(float), (size_t)(3 * S), f);
  fwrite(out_st, sizeof(float), (size_t)(3 * S), f);
  fwrite(out_p, sizeof(uint16_t), (size_t)S, f);
  fwrite(out_g, sizeof(float), (size_t)S, f);
  fclose(f);
  hipFree(dg);
  hipFree(dst);
  hipFree(dp);
  hipFree(dgo);
  free(g);
  free(st);
  free(out_st);
  free(out_p);
  free(out_g);
  zero_layout_destroy(L);
  printf("ok\n");
  return 0;
}
