/*
 * A C program that drives liblite_attn through its C ABI alone (no Python, no torch): it
 * validates a few bad configurations, then runs a short chain of bf16 steps on seeded inputs
 * and checks what holds at any size:
 *   - every output element is finite, and every output row is a convex combination of V rows,
 *     so it lies inside the per-column range of V;
 *   - the skipped-tile count never decreases along the chain (flags persist);
 *   - running the same chain twice gives bit-identical outputs and masks;
 *   - the same chain through lite_attn_step_scheduled (heaviest-first order, caller workspace)
 *     and through lite_attn_step_refresh with refresh_delta = +inf (references start as NaN)
 *     gives the plain chain's outputs and masks bit for bit;
 *   - lite_attn_output_max_abs_diff of a tensor with itself is 0;
 *   - lite_attn_calibrate with unlimited error budgets takes the loosest candidate at every step,
 *     replaying its schedule through lite_attn_step reproduces the errors it reports bit for bit
 *     (each against the same step with an empty mask), and zero budgets give exact outputs.
 * Exit status 0 means every check passed; the last line printed says "c abi smoke ok".
 * Built by tests/test_c_abi.py with gcc as C11 and linked against the library.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lite_attn.h"

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),       \
              __FILE__, __LINE__);                                            \
      return 2;                                                               \
    }                                                                         \
  } while (0)

#define CHECK_LA(x)                                                           \
  do {                                                                        \
    int s_ = (x);                                                             \
    if (s_ != LITE_ATTN_OK) {                                                 \
      fprintf(stderr, "lite_attn error %d (%s): %s at %s:%d\n", s_,           \
              lite_attn_status_string(s_), lite_attn_last_error(), __FILE__,  \
              __LINE__);                                                      \
      return 3;                                                               \
    }                                                                         \
  } while (0)

enum { B = 1, H = 4, N = 3000, D = 128, STEPS = 4 };

/* splitmix64: a published counter-based generator, used only to make inputs */
static uint64_t mix(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* float -> bf16, round to nearest even (finite inputs) */
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static float float_of(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* uniform in [-a, a), rounded to bf16 */
static void fill(uint16_t* x, size_t n, uint64_t seed, float a) {
  for (size_t i = 0; i < n; ++i) {
    const double r = (double)(mix(seed * 0x100000001ull + i) >> 11) / 9007199254740992.0;
    x[i] = bf16_of((float)((2.0 * r - 1.0) * a));
  }
}

enum { PLAIN = 0, SCHEDULED = 1, REFRESH = 2 };

static int run_chain(lite_attn_t h, int mode, const void* dq, const void* dk, const void* dv,
                     void* dout, uint32_t* dmask, uint32_t* dcounts, void* dws, float* dstats,
                     uint16_t* out_host, uint32_t* mask_host, size_t mask_bytes,
                     uint64_t* skipped) {
  static const float eps[STEPS] = {-INFINITY, -3.0f, -2.5f, -2.0f};
  CHECK_LA(lite_attn_reset_mask(h, dmask, NULL));
  if (mode == REFRESH) {
    float nan_stats[B * H * 32];   /* Tq = ceil(N / 128) = 24 query tiles per head */
    for (int i = 0; i < B * H * 32; ++i) nan_stats[i] = NAN;
    CHECK_HIP(hipMemcpy(dstats, nan_stats, sizeof(float) * B * H * ((N + 127) / 128),
                        hipMemcpyHostToDevice));
  }
  uint64_t prev = 0;
  for (int t = 0; t < STEPS; ++t) {
    if (mode == SCHEDULED)
      CHECK_LA(lite_attn_step_scheduled(h, dq, dk, dv, dout, dmask, eps[t], t, dws, NULL));
    else if (mode == REFRESH)
      CHECK_LA(lite_attn_step_refresh(h, dq, dk, dv, dout, dmask, dstats, INFINITY, eps[t], t,
                                      NULL));
    else
      CHECK_LA(lite_attn_step(h, dq, dk, dv, dout, dmask, eps[t], t, NULL));
    CHECK_LA(lite_attn_mask_popcount(h, dmask, dcounts, NULL));
    uint32_t counts[B * H];
    CHECK_HIP(hipMemcpy(counts, dcounts, sizeof counts, hipMemcpyDeviceToHost));
    uint64_t total = 0;
    for (int i = 0; i < B * H; ++i) total += counts[i];
    if (total < prev) {
      fprintf(stderr, "skipped count decreased at step %d: %llu < %llu\n", t,
              (unsigned long long)total, (unsigned long long)prev);
      return 4;
    }
    prev = total;
    printf("chain %d step %d: skipped tiles %llu\n", mode, t, (unsigned long long)total);
  }
  *skipped = prev;
  CHECK_HIP(hipMemcpy(out_host, dout, sizeof(uint16_t) * (size_t)B * H * N * D,
                      hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(mask_host, dmask, mask_bytes, hipMemcpyDeviceToHost));
  return 0;
}

/* The library's calibration loop (lite_attn_calibrate), checked against a replay of the schedule
 * it chose. Every step uses the same inputs. */
static int run_calibration(lite_attn_t h, const void* dq, const void* dk, const void* dv,
                           void* dout, uint32_t* dmask, size_t mask_bytes) {
  void *dcal, *ddense;
  uint32_t* dempty;
  float* dres;
  const size_t elems = (size_t)B * H * N * D;
  const size_t cal_bytes = lite_attn_calibrate_workspace_bytes(h);
  CHECK_HIP(hipMalloc(&dcal, cal_bytes));
  CHECK_HIP(hipMalloc(&ddense, elems * 2));
  CHECK_HIP(hipMalloc((void**)&dempty, mask_bytes));
  CHECK_HIP(hipMalloc((void**)&dres, sizeof(float)));
  float r = -1.0f;
  CHECK_LA(lite_attn_output_max_abs_diff(h, dout, dout, dres, NULL));
  CHECK_HIP(hipMemcpy(&r, dres, sizeof r, hipMemcpyDeviceToHost));
  if (r != 0.0f) {
    fprintf(stderr, "max |a - a| = %g\n", r);
    return 12;
  }
  const void *qs[STEPS], *ks[STEPS], *vs[STEPS];
  float unlimited[STEPS], zero[STEPS], log_eps[STEPS], errs[STEPS];
  for (int t = 0; t < STEPS; ++t) {
    qs[t] = dq;
    ks[t] = dk;
    vs[t] = dv;
    unlimited[t] = INFINITY;
    zero[t] = 0.0f;
  }
  const float cands[3] = {-8.0f, -2.0f, -2.5f};
  CHECK_LA(lite_attn_calibrate(h, qs, ks, vs, STEPS, unlimited, cands, 3, log_eps, errs, dcal,
                               NULL));
  for (int t = 0; t < STEPS; ++t) {
    printf("calibration step %d: log_eps %g error %g\n", t, log_eps[t], errs[t]);
    if (log_eps[t] != -2.0f) {
      fprintf(stderr, "unlimited budgets: step %d took %g, not the loosest candidate\n", t,
              log_eps[t]);
      return 13;
    }
  }
  if (errs[0] != 0.0f) {
    fprintf(stderr, "step 0 starts from an empty mask but reports error %g\n", errs[0]);
    return 13;
  }
  /* replay: the accumulated mask against an empty one, step by step */
  CHECK_LA(lite_attn_reset_mask(h, dmask, NULL));
  for (int t = 0; t < STEPS; ++t) {
    CHECK_LA(lite_attn_step(h, dq, dk, dv, dout, dmask, log_eps[t], t, NULL));
    CHECK_LA(lite_attn_reset_mask(h, dempty, NULL));
    CHECK_LA(lite_attn_step(h, dq, dk, dv, ddense, dempty, -INFINITY, t, NULL));
    CHECK_LA(lite_attn_output_max_abs_diff(h, dout, ddense, dres, NULL));
    CHECK_HIP(hipMemcpy(&r, dres, sizeof r, hipMemcpyDeviceToHost));
    if (memcmp(&r, &errs[t], sizeof r) != 0) {
      fprintf(stderr, "step %d: replayed error %g, calibration reported %g\n", t, r, errs[t]);
      return 14;
    }
  }
  CHECK_LA(lite_attn_calibrate(h, qs, ks, vs, STEPS, zero, cands, 3, log_eps, errs, dcal, NULL));
  for (int t = 0; t < STEPS; ++t)
    if (errs[t] != 0.0f) {
      fprintf(stderr, "zero budgets: step %d (log_eps %g) has error %g\n", t, log_eps[t],
              errs[t]);
      return 15;
    }
  CHECK_HIP(hipFree(dcal));
  CHECK_HIP(hipFree(ddense));
  CHECK_HIP(hipFree(dempty));
  CHECK_HIP(hipFree(dres));
  return 0;
}

int main(void) {
  /* configuration validation needs no device */
  lite_attn_config bad;
  memset(&bad, 0, sizeof bad);
  bad.abi_version = LITE_ATTN_ABI_VERSION + 1;
  lite_attn_t h = NULL;
  if (lite_attn_create(&bad, &h) != LITE_ATTN_ERR_INVALID_ARG || h != NULL) {
    fprintf(stderr, "a wrong abi_version was accepted\n");
    return 5;
  }

  lite_attn_config c;
  memset(&c, 0, sizeof c);
  c.abi_version = LITE_ATTN_ABI_VERSION;
  c.batch = B;
  c.heads = H;
  c.seq_len = N;
  c.head_dim = D;
  c.tile_q = 128;
  c.tile_k = 64;
  c.dtype = LITE_ATTN_BF16;
  c.softmax_scale = 1.0f;
  c.order = LITE_ATTN_ORDER_ALT;
  CHECK_LA(lite_attn_create(&c, &h));
  int32_t tq = 0, tk = 0, w = 0;
  CHECK_LA(lite_attn_mask_geometry(h, &tq, &tk, &w));
  const size_t mask_bytes = lite_attn_mask_bytes(h);
  if (mask_bytes != (size_t)B * H * tq * w * 4) {
    fprintf(stderr, "mask_bytes %zu does not match the geometry\n", mask_bytes);
    return 6;
  }

  const size_t elems = (size_t)B * H * N * D;
  uint16_t* q = (uint16_t*)malloc(elems * 2);
  uint16_t* k = (uint16_t*)malloc(elems * 2);
  uint16_t* v = (uint16_t*)malloc(elems * 2);
  uint16_t* out1 = (uint16_t*)malloc(elems * 2);
  uint16_t* out2 = (uint16_t*)malloc(elems * 2);
  uint32_t* m1 = (uint32_t*)malloc(mask_bytes);
  uint32_t* m2 = (uint32_t*)malloc(mask_bytes);
  if (!q || !k || !v || !out1 || !out2 || !m1 || !m2) return 7;
  if (tq > 32) {
    fprintf(stderr, "more query tiles per head than the statistics buffer holds\n");
    return 7;
  }
  fill(q, elems, 1, 2.0f);
  fill(k, elems, 2, 2.0f);
  fill(v, elems, 3, 1.0f);

  void *dq, *dk, *dv, *dout, *dws;
  uint32_t *dmask, *dcounts;
  float* dstats;
  const size_t ws_bytes = lite_attn_workspace_bytes(h);
  if (ws_bytes == 0) {
    fprintf(stderr, "lite_attn_workspace_bytes returned 0\n");
    return 6;
  }
  CHECK_HIP(hipMalloc(&dq, elems * 2));
  CHECK_HIP(hipMalloc(&dk, elems * 2));
  CHECK_HIP(hipMalloc(&dv, elems * 2));
  CHECK_HIP(hipMalloc(&dout, elems * 2));
  CHECK_HIP(hipMalloc((void**)&dmask, mask_bytes));
  CHECK_HIP(hipMalloc((void**)&dcounts, sizeof(uint32_t) * B * H));
  CHECK_HIP(hipMalloc(&dws, ws_bytes));
  CHECK_HIP(hipMalloc((void**)&dstats, sizeof(float) * B * H * tq));
  CHECK_HIP(hipMemcpy(dq, q, elems * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, k, elems * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, v, elems * 2, hipMemcpyHostToDevice));

  /* argument errors are reported, not launched */
  if (lite_attn_step(h, dq, dk, dv, dq, dmask, -1.0f, 0, NULL) != LITE_ATTN_ERR_INVALID_ARG) {
    fprintf(stderr, "out aliasing q was accepted\n");
    return 8;
  }
  if (lite_attn_step(h, dq, dk, dv, dout, dmask, 0.5f, 0, NULL) != LITE_ATTN_ERR_INVALID_ARG) {
    fprintf(stderr, "a positive log_eps was accepted\n");
    return 8;
  }

  uint64_t s1 = 0, s2 = 0;
  int rc = run_chain(h, PLAIN, dq, dk, dv, dout, dmask, dcounts, dws, dstats, out1, m1,
                     mask_bytes, &s1);
  if (rc) return rc;
  for (int mode = PLAIN; mode <= REFRESH; ++mode) {
    rc = run_chain(h, mode, dq, dk, dv, dout, dmask, dcounts, dws, dstats, out2, m2, mask_bytes,
                   &s2);
    if (rc) return rc;
    if (memcmp(out1, out2, elems * 2) != 0 || memcmp(m1, m2, mask_bytes) != 0 || s1 != s2) {
      fprintf(stderr, "chain %d differs from the plain chain\n", mode);
      return 9;
    }
  }
  if (s1 == 0) {
    fprintf(stderr, "no tile was skipped: the chain did not exercise skipping\n");
    return 10;
  }

  /* every output row lies inside the per-column range of V (of its head) */
  for (int hh = 0; hh < B * H; ++hh) {
    const uint16_t* vh = v + (size_t)hh * N * D;
    const uint16_t* oh = out1 + (size_t)hh * N * D;
    for (int d = 0; d < D; ++d) {
      float lo = INFINITY, hi = -INFINITY;
      for (int n = 0; n < N; ++n) {
        const float x = float_of(vh[(size_t)n * D + d]);
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
      }
      const float tol = 1e-2f;   /* bf16 rounding of the output */
      for (int n = 0; n < N; ++n) {
        const float o = float_of(oh[(size_t)n * D + d]);
        if (!isfinite(o) || o < lo - tol || o > hi + tol) {
          fprintf(stderr, "out[%d][%d][%d] = %g outside [%g, %g]\n", hh, n, d, o, lo, hi);
          return 11;
        }
      }
    }
  }

  rc = run_calibration(h, dq, dk, dv, dout, dmask, mask_bytes);
  if (rc) return rc;

  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dmask));
  CHECK_HIP(hipFree(dcounts));
  CHECK_HIP(hipFree(dws));
  CHECK_HIP(hipFree(dstats));
  CHECK_LA(lite_attn_destroy(h));
  free(q); free(k); free(v); free(out1); free(out2); free(m1); free(m2);
  printf("c abi smoke ok: %llu of %lld tiles skipped after %d steps\n", (unsigned long long)s1,
         (long long)B * H * tq * tk, STEPS);
  return 0;
}
