/*
 * c_consumer.c -- the C ABI of libh3attn.so used from plain C (TEST INFRASTRUCTURE).
 *
 * A C caller with no Python and no torch: device buffers come from the HIP runtime
 * (hipMalloc / hipMemcpy), the library's entry points are resolved by name from the shared
 * object with dlsym and typed from include/h3attn.h (which must therefore compile as C),
 * and the outputs are checked against the fp64 oracle (oracle/liboracle.so, also resolved
 * with dlsym), with the parity tolerances of the other GPU tests: O relative L2 <= 5e-3,
 * max |dO| <= 2e-2, max |dLSE| <= 1e-3.  Rejected calls must return their status without
 * writing an output byte.
 *
 * Built by the repository's build step into a shared object whose one function,
 * h3attn_c_consumer_run, a GPU test calls through ctypes (in its own process, so the HIP
 * runtime is the one the test process already has).
 */
#include <dlfcn.h>
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "h3attn.h"

typedef int (*oracle_causal_fn)(const uint16_t*, const uint16_t*, const uint16_t*, int64_t,
                                int64_t, int64_t, int64_t, float, const int64_t*, int64_t,
                                double*, double*, int);
typedef int (*oracle_varlen_fn)(const uint16_t*, const uint16_t*, const uint16_t*,
                                const int64_t*, int64_t, int64_t, int64_t, int64_t, float,
                                const int64_t*, int64_t, double*, double*, int);

static char* g_report;
static int g_report_len;

static void say(const char* fmt, ...) {
  const size_t used = strlen(g_report);
  if ((int)used >= g_report_len - 1) return;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_report + used, (size_t)g_report_len - used, fmt, ap);
  va_end(ap);
}

/* xorshift32 values in [-2, 2), rounded to bf16 (nearest, ties to even) */
static uint32_t g_state = 2463534242u;
static uint16_t next_bf16(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 17;
  g_state ^= g_state << 5;
  float x = ((float)(g_state >> 8) * (1.0f / 16777216.0f)) * 4.0f - 2.0f;
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static void* dev_alloc(size_t n) {
  void* p = NULL;
  if (hipMalloc(&p, n ? n : 16) != hipSuccess) return NULL;
  return p;
}

/* compare a GPU result (bf16 O, fp32 LSE, copied back) with the oracle's */
static int check(const char* what, const uint16_t* o, const float* lse, const double* o_ref,
                 const double* lse_ref, size_t n_o, size_t n_lse) {
  double num = 0.0, den = 0.0, mx = 0.0, lmx = 0.0;
  for (size_t i = 0; i < n_o; ++i) {
    const double d = bf16_to_double(o[i]) - o_ref[i];
    num += d * d;
    den += o_ref[i] * o_ref[i];
    if (!(fabs(d) <= mx)) mx = fabs(d);
  }
  for (size_t i = 0; i < n_lse; ++i) {
    const double d = fabs((double)lse[i] - lse_ref[i]);
    if (!(d <= lmx)) lmx = d;
  }
  const double rel = den > 0.0 ? sqrt(num / den) : sqrt(num);
  const int ok = rel <= 5e-3 && mx <= 2e-2 && lmx <= 1e-3;
  say("%s: rel_l2=%.3e max_abs=%.3e lse_abs=%.3e %s\n", what, rel, mx, lmx, ok ? "ok" : "FAIL");
  return ok ? 0 : 1;
}

/* One causal call (fixed length, or packed when nseq > 0) through the library and the
 * oracle.  Returns 0 when it matches. */
static int run_case(void* lib, void* orc, int S, int Hq, int Hkv, int D, const int* lens,
                    int nseq) {
  __typeof__(&h3attn_gqa_causal_fwd) fwd =
      (__typeof__(&h3attn_gqa_causal_fwd))dlsym(lib, "h3attn_gqa_causal_fwd");
  __typeof__(&h3attn_gqa_causal_varlen_fwd) varlen =
      (__typeof__(&h3attn_gqa_causal_varlen_fwd))dlsym(lib, "h3attn_gqa_causal_varlen_fwd");
  oracle_causal_fn ocausal = (oracle_causal_fn)dlsym(orc, "oracle_gqa_causal");
  oracle_varlen_fn ovarlen = (oracle_varlen_fn)dlsym(orc, "oracle_gqa_causal_varlen");
  if (!fwd || !varlen || !ocausal || !ovarlen) {
    say("missing symbol\n");
    return 2;
  }
  int max_len = S;
  int32_t cu32[16];
  int64_t cu64[16];
  if (nseq > 0) {
    S = 0;
    max_len = 0;
    cu32[0] = 0;
    cu64[0] = 0;
    for (int i = 0; i < nseq; ++i) {
      S += lens[i];
      cu32[i + 1] = S;
      cu64[i + 1] = S;
      if (lens[i] > max_len) max_len = lens[i];
    }
  }
  const size_t nq = (size_t)S * Hq * D, nk = (size_t)S * Hkv * D, nl = (size_t)Hq * S;
  uint16_t* q = malloc(nq * 2);
  uint16_t* k = malloc(nk * 2);
  uint16_t* v = malloc(nk * 2);
  uint16_t* o = malloc(nq * 2);
  float* lse = malloc(nl * 4);
  double* o_ref = malloc(nq * 8);
  double* lse_ref = malloc(nl * 8);
  int64_t* tokens = malloc((size_t)(S > 0 ? S : 1) * 8);   /* every query token */
  void *dq = dev_alloc(nq * 2), *dk = dev_alloc(nk * 2), *dv = dev_alloc(nk * 2);
  void *dout = dev_alloc(nq * 2), *dlse = dev_alloc(nl * 4), *dcu = dev_alloc(sizeof cu32);
  int rc = 2;
  if (!q || !k || !v || !o || !lse || !o_ref || !lse_ref || !tokens || !dq || !dk || !dv ||
      !dout || !dlse || !dcu) {
    say("allocation failed\n");
    goto done;
  }
  for (int i = 0; i < S; ++i) tokens[i] = i;
  for (size_t i = 0; i < nq; ++i) q[i] = next_bf16();
  for (size_t i = 0; i < nk; ++i) k[i] = next_bf16();
  for (size_t i = 0; i < nk; ++i) v[i] = next_bf16();
  if (hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dk, k, nk * 2, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dv, v, nk * 2, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dcu, cu32, sizeof cu32, hipMemcpyHostToDevice) != hipSuccess) {
    say("copy to the device failed\n");
    goto done;
  }
  const float scale = 1.0f / sqrtf((float)D);
  int st;
  if (nseq > 0)
    st = varlen(dq, dk, dv, dout, dlse, (const int32_t*)dcu, nseq, S, max_len, Hq, Hkv, D, scale,
                NULL);
  else
    st = fwd(dq, dk, dv, dout, dlse, S, Hq, Hkv, D, scale, NULL);
  if (st != H3ATTN_OK) {
    say("call failed: %s\n", ((__typeof__(&h3attn_status_string))dlsym(lib,
                                 "h3attn_status_string"))(st));
    goto done;
  }
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(o, dout, nq * 2, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(lse, dlse, nl * 4, hipMemcpyDeviceToHost) != hipSuccess) {
    say("copy back failed\n");
    goto done;
  }
  if ((nseq > 0 ? ovarlen(q, k, v, cu64, nseq, Hq, Hkv, D, scale, tokens, S, o_ref, lse_ref, 0)
                : ocausal(q, k, v, S, Hq, Hkv, D, scale, tokens, S, o_ref, lse_ref, 0)) != 0) {
    say("oracle failed\n");
    goto done;
  }
  {
    char what[96];
    snprintf(what, sizeof what, "%s S=%d %d/%d D=%d", nseq > 0 ? "packed" : "fixed", S, Hq,
             Hkv, D);
    rc = check(what, o, lse, o_ref, lse_ref, nq, nl);
  }
done:
  free(q), free(k), free(v), free(o), free(lse), free(o_ref), free(lse_ref), free(tokens);
  hipFree(dq), hipFree(dk), hipFree(dv), hipFree(dout), hipFree(dlse), hipFree(dcu);
  return rc;
}

/* Rejected calls: each returns its status and leaves a device canary untouched. */
static int run_rejections(void* lib) {
  __typeof__(&h3attn_gqa_causal_fwd) fwd =
      (__typeof__(&h3attn_gqa_causal_fwd))dlsym(lib, "h3attn_gqa_causal_fwd");
  __typeof__(&h3attn_status_string) status_string =
      (__typeof__(&h3attn_status_string))dlsym(lib, "h3attn_status_string");
  if (!fwd || !status_string) return 2;
  const size_t n = 64 * 8 * 128 * 2 + 64;
  uint8_t* canary = malloc(n);
  uint8_t* back = malloc(n);
  void* d = dev_alloc(n);
  int rc = 0;
  if (!canary || !back || !d) {
    rc = 2;
    goto done;
  }
  memset(canary, 0xA5, n);
  if (hipMemcpy(d, canary, n, hipMemcpyHostToDevice) != hipSuccess) {
    rc = 2;
    goto done;
  }
  struct {
    const char* what;
    int D, Hq, Hkv, offset, expect;
    int null_q;
  } cases[] = {
      {"head dim 96", 96, 8, 2, 0, H3ATTN_ERR_UNSUPPORTED, 0},
      {"Hq not a multiple of Hkv", 128, 6, 4, 0, H3ATTN_ERR_SHAPE, 0},
      {"NULL q", 128, 8, 2, 0, H3ATTN_ERR_NULL, 1},
      {"misaligned output", 128, 8, 2, 2, H3ATTN_ERR_ALIGN, 0},
  };
  for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i) {
    uint8_t* base = (uint8_t*)d;
    const int st = fwd(cases[i].null_q ? NULL : base, base, base, base + cases[i].offset,
                       (float*)base, 64, cases[i].Hq, cases[i].Hkv, cases[i].D, 0.125f, NULL);
    const char* s = status_string(st);
    const int ok = st == cases[i].expect && s != NULL && s[0] != '\0';
    say("rejection %s: status %d (%s) %s\n", cases[i].what, st, s ? s : "(null)",
        ok ? "ok" : "FAIL");
    if (!ok) rc = 1;
  }
  if (hipMemcpy(back, d, n, hipMemcpyDeviceToHost) != hipSuccess) {
    rc = 2;
    goto done;
  }
  if (memcmp(back, canary, n) != 0) {
    say("a rejected call wrote device memory FAIL\n");
    rc = 1;
  }
done:
  free(canary), free(back);
  if (d) hipFree(d);
  return rc;
}

/* Runs every case; returns 0 when all pass, and writes one line per case to report. */
int h3attn_c_consumer_run(const char* lib_path, const char* oracle_path, char* report,
                          int report_len) {
  g_report = report;
  g_report_len = report_len;
  if (report_len > 0) report[0] = '\0';
  void* lib = dlopen(lib_path, RTLD_NOW | RTLD_LOCAL);
  void* orc = dlopen(oracle_path, RTLD_NOW | RTLD_LOCAL);
  if (!lib || !orc) {
    say("dlopen failed: %s\n", dlerror());
    return 2;
  }
  int rc = 0;
  const int lens[3] = {100, 0, 77};
  rc |= run_case(lib, orc, 333, 16, 2, 128, NULL, 0);
  rc |= run_case(lib, orc, 200, 8, 8, 64, NULL, 0);
  rc |= run_case(lib, orc, 0, 8, 2, 128, lens, 3);
  rc |= run_rejections(lib);
  return rc;
}
