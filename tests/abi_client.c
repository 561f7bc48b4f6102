/*
 * abi_client.c - a plain C11 program that uses libadasum through include/adasum.h
 * alone: device memory comes from the HIP runtime API, never from Python.  It
 * checks results that have closed forms, so it needs no reference
 * implementation:
 *
 *   - mutually orthogonal gradients (disjoint supports): every dot product is
 *     exactly zero, so every node's coefficients are exactly (1, 1) and the
 *     combine is the plain sum, which here is exact ("Scaling Distributed
 *     Training with Adaptive Summation", the discussion before Figure 1:
 *     orthogonal gradients are summed);
 *   - K equal gradients: every pair is parallel, every coefficient is 1/2
 *     (exactly so in the tree) and the combine returns the gradient itself
 *     (same passage: parallel gradients are averaged); the orthogonality
 *     ratio is then 1/K;
 *   - adasum_sum of small integers, which is exact in every dtype;
 *   - K = 1 copies its input;
 *   - the error paths: invalid arguments return ADASUM_EINVAL with a message
 *     and leave the library usable.
 *
 * Build (host compiler only; the library carries the GPU code):
 *   gcc -std=c11 -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include -Iinclude tests/abi_client.c \
 *       -Ldistributed_sgd_gradient_amd -ladasum -L/opt/rocm/lib -lamdhip64 -o abi_client
 * Exit status 0 when every check passes; one line per check on stdout.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "adasum.h"

static int failures = 0;
static int checks = 0;

static void report(int ok, const char* name, const char* detail) {
  ++checks;
  if (!ok) ++failures;
  printf("%s %s%s%s\n", ok ? "ok  " : "FAIL", name, detail[0] ? ": " : "", detail);
  fflush(stdout);
}

#define HIP_OK(call)                                                            \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      printf("FAIL %s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

/* ---- element encodings (values used here are exact in every dtype) ---- */

static size_t elem_size(int dtype) { return dtype == ADASUM_F32 ? 4 : 2; }

static uint32_t f32_bits(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return u;
}

/* x must be zero or a normal fp16 value with at most 11 significant bits */
static uint16_t to_f16(float x) {
  if (x == 0.0f) return 0;
  const uint32_t u = f32_bits(x);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int e = (int)((u >> 23) & 0xff) - 127 + 15;
  return (uint16_t)(sign | ((uint32_t)e << 10) | ((u >> 13) & 0x3ffu));
}

static float from_f16(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const int e = (h >> 10) & 0x1f;
  const uint32_t m = h & 0x3ffu;
  float x;
  if (e == 0) {
    x = ldexpf((float)m, -24);
  } else {
    const uint32_t u = ((uint32_t)(e - 15 + 127) << 23) | (m << 13);
    memcpy(&x, &u, 4);
  }
  return sign ? -x : x;
}

/* x must have at most 8 significant bits (then truncation is exact) */
static uint16_t to_bf16(float x) { return (uint16_t)(f32_bits(x) >> 16); }

static float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}

static void store(void* buf, int dtype, int64_t i, float x) {
  if (dtype == ADASUM_F32)
    ((float*)buf)[i] = x;
  else if (dtype == ADASUM_F16)
    ((uint16_t*)buf)[i] = to_f16(x);
  else
    ((uint16_t*)buf)[i] = to_bf16(x);
}

static float load(const void* buf, int dtype, int64_t i) {
  if (dtype == ADASUM_F32) return ((const float*)buf)[i];
  if (dtype == ADASUM_F16) return from_f16(((const uint16_t*)buf)[i]);
  return from_bf16(((const uint16_t*)buf)[i]);
}

/* a nonzero value with at most 7 significant bits, varied over i */
static float value(int64_t i) {
  const float m = (float)((i * 37) % 101 + 1);
  return ldexpf((i & 1) ? -m : m, -4);
}

/* ---- the shape every combine check uses: four segments, one empty ---- */

#define NSEG 4
static const int64_t kOffsets[NSEG + 1] = {0, 4097, 4097, 5097, 75099};
#define N_ELEMS 75099

typedef struct {
  int K, dtype, schedule;
  void** dev;      /* K device buffers */
  void* host;      /* K * N host values, gradient-major */
  void* out;       /* device, N elements */
  void* ws;        /* device workspace */
  size_t ws_bytes;
  double* coeffs;  /* device [K-1][NSEG][2] */
  double* stats;   /* device [K-1][NSEG][3] */
  double* ortho;   /* device [NSEG] */
} Case;

static void case_alloc(Case* c, int K, int dtype, int schedule) {
  c->K = K;
  c->dtype = dtype;
  c->schedule = schedule;
  const size_t bytes = (size_t)N_ELEMS * elem_size(dtype);
  c->dev = (void**)calloc((size_t)K, sizeof(void*));
  c->host = malloc(bytes * (size_t)K);
  for (int k = 0; k < K; ++k) HIP_OK(hipMalloc(&c->dev[k], bytes));
  HIP_OK(hipMalloc(&c->out, bytes));
  const int64_t ws = adasum_workspace_bytes(K, kOffsets, NSEG, dtype, schedule);
  if (ws < 0) {
    printf("FAIL adasum_workspace_bytes: %s\n", adasum_last_error());
    exit(2);
  }
  c->ws_bytes = (size_t)ws;
  HIP_OK(hipMalloc(&c->ws, c->ws_bytes ? c->ws_bytes : 1));
  const size_t nodes = K > 1 ? (size_t)(K - 1) : 1;
  HIP_OK(hipMalloc((void**)&c->coeffs, nodes * NSEG * 2 * sizeof(double)));
  HIP_OK(hipMalloc((void**)&c->stats, nodes * NSEG * 3 * sizeof(double)));
  HIP_OK(hipMalloc((void**)&c->ortho, NSEG * sizeof(double)));
}

static void case_upload(Case* c) {
  const size_t bytes = (size_t)N_ELEMS * elem_size(c->dtype);
  for (int k = 0; k < c->K; ++k)
    HIP_OK(hipMemcpy(c->dev[k], (char*)c->host + (size_t)k * bytes, bytes, hipMemcpyHostToDevice));
}

static void case_free(Case* c) {
  for (int k = 0; k < c->K; ++k) HIP_OK(hipFree(c->dev[k]));
  HIP_OK(hipFree(c->out));
  HIP_OK(hipFree(c->ws));
  HIP_OK(hipFree(c->coeffs));
  HIP_OK(hipFree(c->stats));
  HIP_OK(hipFree(c->ortho));
  free(c->dev);
  free(c->host);
}

static int case_run(Case* c, hipStream_t stream) {
  return adasum_combine_ex((const void* const*)c->dev, c->K, kOffsets, NSEG, c->dtype, c->schedule, c->out,
                           c->ws, c->ws_bytes, c->coeffs, c->stats, c->ortho, stream);
}

static const char* dtype_name(int d) { return d == ADASUM_F32 ? "f32" : d == ADASUM_F16 ? "f16" : "bf16"; }

/* Orthogonal gradients: g_k is nonzero exactly where i % K == k. */
static void check_orthogonal(int K, int dtype, int schedule, hipStream_t stream) {
  char name[96], detail[256] = "";
  snprintf(name, sizeof name, "orthogonal K=%d %s %s", K, dtype_name(dtype), schedule ? "chain" : "tree");
  Case c;
  case_alloc(&c, K, dtype, schedule);
  for (int k = 0; k < K; ++k)
    for (int64_t i = 0; i < N_ELEMS; ++i)
      store((char*)c.host + (size_t)k * N_ELEMS * elem_size(dtype), dtype, i, (i % K == k) ? value(i) : 0.0f);
  case_upload(&c);
  int rc = case_run(&c, stream);
  if (rc != ADASUM_OK) {
    snprintf(detail, sizeof detail, "rc %d: %s", rc, adasum_last_error());
    report(0, name, detail);
    case_free(&c);
    return;
  }
  HIP_OK(hipStreamSynchronize(stream));
  const size_t nodes = (size_t)(K - 1) * NSEG;
  void* out = malloc((size_t)N_ELEMS * elem_size(dtype));
  double* coeffs = (double*)malloc(nodes * 2 * sizeof(double));
  double* stats = (double*)malloc(nodes * 3 * sizeof(double));
  double ortho[NSEG];
  HIP_OK(hipMemcpy(out, c.out, (size_t)N_ELEMS * elem_size(dtype), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(coeffs, c.coeffs, nodes * 2 * sizeof(double), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(stats, c.stats, nodes * 3 * sizeof(double), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ortho, c.ortho, sizeof ortho, hipMemcpyDeviceToHost));
  int ok = 1;
  for (int64_t i = 0; i < N_ELEMS && ok; ++i)
    if (load(out, dtype, i) != value(i)) {
      snprintf(detail, sizeof detail, "out[%lld] = %g, expected the sum %g", (long long)i, load(out, dtype, i),
               value(i));
      ok = 0;
    }
  for (size_t n = 0; n < nodes && ok; ++n) {
    const int seg = (int)(n % NSEG);
    const int empty = kOffsets[seg + 1] == kOffsets[seg];
    if (empty) continue;  /* an empty segment has no statistics to speak of */
    if (coeffs[2 * n] != 1.0 || coeffs[2 * n + 1] != 1.0 || stats[3 * n] != 0.0 || !(stats[3 * n + 1] > 0.0) ||
        !(stats[3 * n + 2] > 0.0)) {
      snprintf(detail, sizeof detail, "node %zu: coeffs (%.17g, %.17g) stats (%.17g, %.17g, %.17g)", n / NSEG,
               coeffs[2 * n], coeffs[2 * n + 1], stats[3 * n], stats[3 * n + 1], stats[3 * n + 2]);
      ok = 0;
    }
  }
  for (int s = 0; s < NSEG && ok; ++s) {
    const int empty = kOffsets[s + 1] == kOffsets[s];
    if (empty ? !isnan(ortho[s]) : fabs(ortho[s] - 1.0) > 1e-12) {
      snprintf(detail, sizeof detail, "ortho[%d] = %.17g, expected %s", s, ortho[s], empty ? "NaN" : "1");
      ok = 0;
    }
  }
  report(ok, name, detail);
  free(out);
  free(coeffs);
  free(stats);
  case_free(&c);
}

/* K equal gradients: the combine returns the gradient, every coefficient is 1/2. */
static void check_parallel(int K, int dtype, int schedule, hipStream_t stream) {
  char name[96], detail[256] = "";
  snprintf(name, sizeof name, "parallel K=%d %s %s", K, dtype_name(dtype), schedule ? "chain" : "tree");
  Case c;
  case_alloc(&c, K, dtype, schedule);
  for (int k = 0; k < K; ++k)
    for (int64_t i = 0; i < N_ELEMS; ++i)
      store((char*)c.host + (size_t)k * N_ELEMS * elem_size(dtype), dtype, i, value(i));
  case_upload(&c);
  int rc = case_run(&c, stream);
  if (rc != ADASUM_OK) {
    snprintf(detail, sizeof detail, "rc %d: %s", rc, adasum_last_error());
    report(0, name, detail);
    case_free(&c);
    return;
  }
  HIP_OK(hipStreamSynchronize(stream));
  const size_t nodes = (size_t)(K - 1) * NSEG;
  void* out = malloc((size_t)N_ELEMS * elem_size(dtype));
  double* coeffs = (double*)malloc(nodes * 2 * sizeof(double));
  double ortho[NSEG];
  HIP_OK(hipMemcpy(out, c.out, (size_t)N_ELEMS * elem_size(dtype), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(coeffs, c.coeffs, nodes * 2 * sizeof(double), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ortho, c.ortho, sizeof ortho, hipMemcpyDeviceToHost));
  int ok = 1;
  for (int64_t i = 0; i < N_ELEMS && ok; ++i)
    if (load(out, dtype, i) != value(i)) {
      snprintf(detail, sizeof detail, "out[%lld] = %g, expected %g", (long long)i, load(out, dtype, i), value(i));
      ok = 0;
    }
  /* Tree: every leaf of a node has the same weight 2^-level, so each
   * quadratic form of the node is an exact multiple of the common Gram entry
   * and the ratio is exactly 1/2.  Chain: the weights run from 2^-1 down to
   * 2^-(j-1), whose partial sums can need more than 53 bits; 1/2 up to
   * rounding. */
  const double tol = schedule == ADASUM_TREE ? 0.0 : 1e-15;
  for (size_t n = 0; n < nodes && ok; ++n) {
    const int seg = (int)(n % NSEG);
    if (kOffsets[seg + 1] == kOffsets[seg]) continue;
    if (fabs(coeffs[2 * n] - 0.5) > tol || fabs(coeffs[2 * n + 1] - 0.5) > tol) {
      snprintf(detail, sizeof detail, "node %zu segment %d: coeffs (%.17g, %.17g)", n / NSEG, seg, coeffs[2 * n],
               coeffs[2 * n + 1]);
      ok = 0;
    }
  }
  for (int s = 0; s < NSEG && ok; ++s) {
    if (kOffsets[s + 1] == kOffsets[s]) continue;
    if (fabs(ortho[s] - 1.0 / K) > 1e-12) {
      snprintf(detail, sizeof detail, "ortho[%d] = %.17g, expected 1/%d", s, ortho[s], K);
      ok = 0;
    }
  }
  report(ok, name, detail);
  free(out);
  free(coeffs);
  case_free(&c);
}

/* adasum_combine (library workspace) gives the same bits as adasum_combine_ex. */
static void check_cached_matches_ex(hipStream_t stream) {
  char detail[256] = "";
  const int K = 11, dtype = ADASUM_F32;
  Case c;
  case_alloc(&c, K, dtype, ADASUM_TREE);
  /* generic (neither orthogonal nor parallel) gradients */
  for (int k = 0; k < K; ++k)
    for (int64_t i = 0; i < N_ELEMS; ++i)
      store((char*)c.host + (size_t)k * N_ELEMS * 4, dtype, i, value(i * (k + 3) + k));
  case_upload(&c);
  void* out2;
  HIP_OK(hipMalloc(&out2, (size_t)N_ELEMS * 4));
  int rc = case_run(&c, stream);
  int rc2 = adasum_combine((const void* const*)c.dev, K, kOffsets, NSEG, dtype, out2, stream);
  HIP_OK(hipStreamSynchronize(stream));
  int ok = rc == ADASUM_OK && rc2 == ADASUM_OK;
  if (!ok) snprintf(detail, sizeof detail, "rc %d / %d: %s", rc, rc2, adasum_last_error());
  if (ok) {
    float* a = (float*)malloc((size_t)N_ELEMS * 4);
    float* b = (float*)malloc((size_t)N_ELEMS * 4);
    HIP_OK(hipMemcpy(a, c.out, (size_t)N_ELEMS * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(b, out2, (size_t)N_ELEMS * 4, hipMemcpyDeviceToHost));
    if (memcmp(a, b, (size_t)N_ELEMS * 4) != 0) {
      snprintf(detail, sizeof detail, "outputs differ");
      ok = 0;
    }
    free(a);
    free(b);
  }
  report(ok, "adasum_combine equals adasum_combine_ex bitwise", detail);
  HIP_OK(hipFree(out2));
  case_free(&c);
}

/* K = 1: the output is the input. */
static void check_single(hipStream_t stream) {
  char detail[256] = "";
  Case c;
  case_alloc(&c, 1, ADASUM_BF16, ADASUM_TREE);
  for (int64_t i = 0; i < N_ELEMS; ++i) store(c.host, ADASUM_BF16, i, value(i));
  case_upload(&c);
  int ok = case_run(&c, stream) == ADASUM_OK;
  if (!ok) snprintf(detail, sizeof detail, "%s", adasum_last_error());
  HIP_OK(hipStreamSynchronize(stream));
  if (ok) {
    uint16_t* out = (uint16_t*)malloc((size_t)N_ELEMS * 2);
    HIP_OK(hipMemcpy(out, c.out, (size_t)N_ELEMS * 2, hipMemcpyDeviceToHost));
    if (memcmp(out, c.host, (size_t)N_ELEMS * 2) != 0) {
      snprintf(detail, sizeof detail, "output differs from the single input");
      ok = 0;
    }
    free(out);
  }
  report(ok, "K=1 copies its input", detail);
  case_free(&c);
}

/* adasum_sum of small integers is exact; K = 70 needs a workspace. */
static void check_sum(int K, int dtype, hipStream_t stream) {
  char name[64], detail[256] = "";
  snprintf(name, sizeof name, "adasum_sum K=%d %s", K, dtype_name(dtype));
  const int64_t N = 10007;
  const size_t es = elem_size(dtype);
  void** dev = (void**)calloc((size_t)K, sizeof(void*));
  void* host = malloc((size_t)N * es);
  for (int k = 0; k < K; ++k) {
    for (int64_t i = 0; i < N; ++i) store(host, dtype, i, (float)((i + 3 * k) % 7 - 3));
    HIP_OK(hipMalloc(&dev[k], (size_t)N * es));
    HIP_OK(hipMemcpy(dev[k], host, (size_t)N * es, hipMemcpyHostToDevice));
  }
  const int64_t wsb = adasum_sum_workspace_bytes(K, N, dtype);
  void* ws = NULL;
  if (wsb > 0) HIP_OK(hipMalloc(&ws, (size_t)wsb));
  void* out;
  HIP_OK(hipMalloc(&out, (size_t)N * es));
  int ok = wsb >= 0 &&
           adasum_sum((const void* const*)dev, K, N, dtype, out, ws, wsb > 0 ? (size_t)wsb : 0, stream) == ADASUM_OK;
  if (!ok) snprintf(detail, sizeof detail, "%s", adasum_last_error());
  HIP_OK(hipStreamSynchronize(stream));
  if (ok) {
    HIP_OK(hipMemcpy(host, out, (size_t)N * es, hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < N && ok; ++i) {
      double want = 0;
      for (int k = 0; k < K; ++k) want += (double)((i + 3 * k) % 7 - 3);
      if ((double)load(host, dtype, i) != want) {
        snprintf(detail, sizeof detail, "out[%lld] = %g, expected %g", (long long)i, load(host, dtype, i), want);
        ok = 0;
      }
    }
  }
  report(ok, name, detail);
  for (int k = 0; k < K; ++k) HIP_OK(hipFree(dev[k]));
  if (ws) HIP_OK(hipFree(ws));
  HIP_OK(hipFree(out));
  free(dev);
  free(host);
}

/* Invalid arguments are rejected before any work, and the library stays usable. */
static void check_errors(hipStream_t stream) {
  Case c;
  case_alloc(&c, 4, ADASUM_F32, ADASUM_TREE);
  for (int k = 0; k < 4; ++k)
    for (int64_t i = 0; i < N_ELEMS; ++i) store((char*)c.host + (size_t)k * N_ELEMS * 4, ADASUM_F32, i, value(i + k));
  case_upload(&c);
  const void* const* g = (const void* const*)c.dev;
  char detail[256];
  struct {
    const char* what;
    int rc;
  } cases[8];
  int n = 0;
  float* host_out = (float*)malloc((size_t)N_ELEMS * 4);
  const int64_t bad_offsets[3] = {0, 10, 5};

  cases[n].what = "K = 0";
  cases[n++].rc = adasum_combine_ex(g, 0, kOffsets, NSEG, ADASUM_F32, ADASUM_TREE, c.out, c.ws, c.ws_bytes, NULL,
                                    NULL, NULL, stream);
  cases[n].what = "decreasing offsets";
  cases[n++].rc = (int)adasum_workspace_bytes(4, bad_offsets, 2, ADASUM_F32, ADASUM_TREE);
  cases[n].what = "unknown dtype";
  cases[n++].rc = adasum_combine_ex(g, 4, kOffsets, NSEG, 7, ADASUM_TREE, c.out, c.ws, c.ws_bytes, NULL, NULL,
                                    NULL, stream);
  cases[n].what = "workspace one byte short";
  cases[n++].rc = adasum_combine_ex(g, 4, kOffsets, NSEG, ADASUM_F32, ADASUM_TREE, c.out, c.ws, c.ws_bytes - 1,
                                    NULL, NULL, NULL, stream);
  cases[n].what = "misaligned out";
  cases[n++].rc = adasum_combine_ex(g, 4, kOffsets, NSEG, ADASUM_F32, ADASUM_TREE, (char*)c.out + 4, c.ws,
                                    c.ws_bytes, NULL, NULL, NULL, stream);
  cases[n].what = "out is an input";
  cases[n++].rc = adasum_combine_ex(g, 4, kOffsets, NSEG, ADASUM_F32, ADASUM_TREE, c.dev[2], c.ws, c.ws_bytes, NULL,
                                    NULL, NULL, stream);
  cases[n].what = "out in host memory";
  cases[n++].rc = adasum_combine_ex(g, 4, kOffsets, NSEG, ADASUM_F32, ADASUM_TREE, host_out, c.ws, c.ws_bytes,
                                    NULL, NULL, NULL, stream);
  for (int i = 0; i < n; ++i) {
    const char* msg = adasum_last_error();
    snprintf(detail, sizeof detail, "rc %d, message \"%s\"", cases[i].rc, msg);
    char name[96];
    snprintf(name, sizeof name, "rejects %s", cases[i].what);
    report(cases[i].rc == ADASUM_EINVAL, name, cases[i].rc == ADASUM_EINVAL ? "" : detail);
  }
  /* the last failure's message is kept for the calling thread */
  report(strlen(adasum_last_error()) > 0, "adasum_last_error describes the failure", "");
  report(strcmp(adasum_strerror(ADASUM_EINVAL), adasum_strerror(ADASUM_OK)) != 0, "adasum_strerror", "");
  /* a valid call after the failures */
  int rc = case_run(&c, stream);
  HIP_OK(hipStreamSynchronize(stream));
  snprintf(detail, sizeof detail, "rc %d: %s", rc, adasum_last_error());
  report(rc == ADASUM_OK, "valid call after rejected ones", rc == ADASUM_OK ? "" : detail);
  free(host_out);
  case_free(&c);
}

/* The kernel timing interface reports the launches of a combine: over fp16
   inputs the Gram pass, the tree walk, the exact recomputation of flagged
   pairs, the second walk over them and the weighted sum. */
static void check_profile(hipStream_t stream) {
  Case c;
  case_alloc(&c, 8, ADASUM_F16, ADASUM_TREE);
  for (int k = 0; k < 8; ++k)
    for (int64_t i = 0; i < N_ELEMS; ++i) store((char*)c.host + (size_t)k * N_ELEMS * 2, ADASUM_F16, i, value(i + k));
  case_upload(&c);
  adasum_kernel_time_t rows[8];
  int ok = adasum_profile_begin() == ADASUM_OK && case_run(&c, stream) == ADASUM_OK;
  const int nrows = adasum_profile_end(rows, 8);
  int seen = 0;
  for (int r = 0; r < nrows; ++r) {
    const int want = !strcmp(rows[r].kernel, "tree") ? 2
                     : (!strcmp(rows[r].kernel, "gram") || !strcmp(rows[r].kernel, "wsum") ||
                        !strcmp(rows[r].kernel, "exact")) ? 1 : 0;
    if (want && rows[r].launches == want && rows[r].milliseconds > 0 && rows[r].bytes > 0) ++seen;
  }
  char detail[80];
  snprintf(detail, sizeof detail, "%d rows, %d of gram/tree/exact/wsum as expected", nrows, seen);
  report(ok && nrows == 4 && seen == 4, "adasum_profile reports gram, tree (twice), exact, wsum",
         ok && seen == 4 ? "" : detail);
  case_free(&c);
}

int main(void) {
  int ndev = 0;
  HIP_OK(hipGetDeviceCount(&ndev));
  if (ndev < 1) {
    printf("FAIL no HIP device\n");
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  printf("libadasum version %d\n", adasum_version());
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  const int dtypes[3] = {ADASUM_F32, ADASUM_F16, ADASUM_BF16};
  for (int d = 0; d < 3; ++d)
    for (int schedule = 0; schedule < 2; ++schedule) {
      check_orthogonal(5, dtypes[d], schedule, stream);
      check_orthogonal(20, dtypes[d], schedule, stream);
      check_parallel(8, dtypes[d], schedule, stream);
      check_parallel(33, dtypes[d], schedule, NULL);  /* default stream; more than one stage */
    }
  check_cached_matches_ex(stream);
  check_single(stream);
  check_sum(3, ADASUM_F16, stream);
  check_sum(70, ADASUM_F32, stream);
  check_sum(9, ADASUM_BF16, stream);
  check_errors(stream);
  check_profile(stream);

  HIP_OK(hipStreamDestroy(stream));
  printf("%d checks, %d failed\n", checks, failures);
  return failures ? 1 : 0;
}
