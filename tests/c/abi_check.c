/*
 * A plain C99 program that drives libpagedattn through its C ABI only: HIP
 * memory and a HIP stream from the runtime's C API, the pools described by a
 * pa_cache, one decode step (pa_kv_append, pa_decode with a workspace, and
 * pa_decode without one).  It checks results that have closed forms:
 *   - a sequence of one token attends to that token alone: out = its V row,
 *     exactly;
 *   - a zero query weighs every visible token equally: out = the mean of the
 *     V rows (float32 output, to 1e-5);
 *   - the appended rows land at their slots, bit for bit.
 * Prints "abi_check ok" and exits 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pagedattn.h"

#define CHECK_HIP(x)                                                    \
  do {                                                                  \
    if ((x) != hipSuccess) {                                            \
      fprintf(stderr, "HIP error %s at line %d\n", #x, __LINE__);       \
      return 2;                                                         \
    }                                                                   \
  } while (0)
#define CHECK_PA(x)                                                     \
  do {                                                                  \
    int st_ = (x);                                                      \
    if (st_ != PA_OK) {                                                 \
      fprintf(stderr, "%s -> %d: %s\n", #x, st_, pa_last_error());      \
      return 3;                                                         \
    }                                                                   \
  } while (0)

enum { NB = 8, HKV = 2, BS = 16, D = 128, S = 3, HQ = 8, MAXB = 4 };

static float frand(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return ((*s >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

int main(void) {
  const size_t pool_elems = (size_t)NB * HKV * BS * D;
  float* k_host = malloc(pool_elems * sizeof(float));
  float* v_host = malloc(pool_elems * sizeof(float));
  unsigned seed = 12345u;
  for (size_t i = 0; i < pool_elems; ++i) {
    k_host[i] = frand(&seed);
    v_host[i] = frand(&seed);
  }
  /* sequence lengths (the appended token included) and tables */
  const int32_t lens[S] = {1, 40, 17};
  const int32_t tables[S][MAXB] = {{5, 0, 0, 0}, {2, 7, 0, 0}, {1, 4, 0, 0}};
  int64_t slots[S];
  for (int i = 0; i < S; ++i) {
    const int p = lens[i] - 1;
    slots[i] = (int64_t)tables[i][p / BS] * BS + p % BS;
  }
  float knew[S][HKV][D], vnew[S][HKV][D], q[S][HQ][D];
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < HKV; ++h)
      for (int d = 0; d < D; ++d) {
        knew[i][h][d] = frand(&seed);
        vnew[i][h][d] = frand(&seed);
      }
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < HQ; ++h)
      for (int d = 0; d < D; ++d) q[i][h][d] = i == 0 ? frand(&seed) : 0.0f;

  void *k_pool, *v_pool, *dq, *dk, *dv, *dslots, *dtables, *dlens, *dout, *dout1, *ws;
  CHECK_HIP(hipMalloc(&k_pool, pool_elems * sizeof(float)));
  CHECK_HIP(hipMalloc(&v_pool, pool_elems * sizeof(float)));
  CHECK_HIP(hipMalloc(&dq, sizeof q));
  CHECK_HIP(hipMalloc(&dk, sizeof knew));
  CHECK_HIP(hipMalloc(&dv, sizeof vnew));
  CHECK_HIP(hipMalloc(&dslots, sizeof slots));
  CHECK_HIP(hipMalloc(&dtables, sizeof tables));
  CHECK_HIP(hipMalloc(&dlens, sizeof lens));
  CHECK_HIP(hipMalloc(&dout, sizeof q));
  CHECK_HIP(hipMalloc(&dout1, sizeof q));
  const size_t ws_bytes = pa_decode_workspace_bytes(S, HQ, D);
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemcpy(k_pool, k_host, pool_elems * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(v_pool, v_host, pool_elems * sizeof(float), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, knew, sizeof knew, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, vnew, sizeof vnew, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dslots, slots, sizeof slots, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dtables, tables, sizeof tables, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  pa_cache cache;
  memset(&cache, 0, sizeof cache);
  cache.k_pool = k_pool;
  cache.v_pool = v_pool;
  cache.num_blocks = NB;
  cache.num_kv_heads = HKV;
  cache.block_size = BS;
  cache.head_dim = D;
  cache.dtype = PA_F32;
  if (pa_abi_version() != PA_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header %d\n", pa_abi_version(), PA_ABI_VERSION);
    return 4;
  }
  const float scale = 1.0f / sqrtf((float)D);
  CHECK_PA(pa_kv_append(&cache, dk, dv, (const int64_t*)dslots, S, stream));
  CHECK_PA(pa_decode(&cache, dq, (const int32_t*)dtables, (const int32_t*)dlens, S, HQ, MAXB,
                     scale, NULL, dout, PA_F32, ws, ws_bytes, stream));
  CHECK_PA(pa_decode(&cache, dq, (const int32_t*)dtables, (const int32_t*)dlens, S, HQ, MAXB,
                     scale, NULL, dout1, PA_F32, NULL, 0, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  /* the host copy of the pools after the append */
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < HKV; ++h)
      for (int d = 0; d < D; ++d) {
        const size_t at = (((size_t)(slots[i] / BS) * HKV + h) * BS + slots[i] % BS) * D + d;
        k_host[at] = knew[i][h][d];
        v_host[at] = vnew[i][h][d];
      }
  float* k_dev = malloc(pool_elems * sizeof(float));
  float* v_dev = malloc(pool_elems * sizeof(float));
  CHECK_HIP(hipMemcpy(k_dev, k_pool, pool_elems * sizeof(float), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(v_dev, v_pool, pool_elems * sizeof(float), hipMemcpyDeviceToHost));
  if (memcmp(k_dev, k_host, pool_elems * sizeof(float)) != 0 ||
      memcmp(v_dev, v_host, pool_elems * sizeof(float)) != 0) {
    fprintf(stderr, "append: pools differ from the expected bytes\n");
    return 5;
  }
  float out[S][HQ][D], out1[S][HQ][D];
  CHECK_HIP(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out1, dout1, sizeof out1, hipMemcpyDeviceToHost));
  const int group = HQ / HKV;
  double worst = 0.0;
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < HQ; ++h) {
      const int g = h / group;
      for (int d = 0; d < D; ++d) {
        double want;
        if (i == 0) { /* one token: its V row, exactly */
          want = vnew[0][g][d];
        } else { /* zero query: the mean of the visible V rows */
          double sum = 0.0;
          for (int t = 0; t < lens[i]; ++t) {
            const int blk = tables[i][t / BS];
            sum += v_host[(((size_t)blk * HKV + g) * BS + t % BS) * D + d];
          }
          want = sum / lens[i];
        }
        const double e0 = fabs(out[i][h][d] - want), e1 = fabs(out1[i][h][d] - want);
        if (i == 0 && (e0 != 0.0 || e1 != 0.0)) {
          fprintf(stderr, "one-token sequence: out differs from its V row\n");
          return 6;
        }
        if (e0 > worst) worst = e0;
        if (e1 > worst) worst = e1;
      }
    }
  if (worst > 1e-5) {
    fprintf(stderr, "zero query: max error %g against the mean of V\n", worst);
    return 7;
  }
  printf("abi_check ok (max error %.2e)\n", worst);
  hipStreamDestroy(stream);
  return 0;
}
