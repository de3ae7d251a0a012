/* Host-only driver of the C ABI for the address / undefined-behaviour
 * sanitizer build (tests/test_abi_sanitize.py).  Every call below must be
 * turned away by argument validation before any HIP call, so it runs on a
 * machine without a GPU; the size queries are swept over extreme values so
 * that an overflowing product or an out-of-range shift in the host code is
 * reported by the sanitizers.  Exit status 0 means every call returned what
 * it should; the sanitizers abort the process on any finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sdpa.h"

static int failures = 0, calls = 0;
static char fake_bytes[64];
#define FAKE ((void*)fake_bytes)
#define FAKEF ((float*)fake_bytes)
#define FAKEU ((uint32_t*)fake_bytes)

static void expect(int got, int want, const char* what) {
  ++calls;
  if (got != want) {
    ++failures;
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, sdpa_last_error());
    return;
  }
  if (want != SDPA_OK && sdpa_last_error()[0] == '\0') {
    ++failures;
    fprintf(stderr, "FAIL %s: status %d without a message\n", what, got);
  }
}

/* sdpa_fwd and sdpa_fwd_noalloc with one argument changed from a valid call. */
typedef struct {
  const void *q, *k, *v;
  void* o;
  int dtype, out_dtype, layout;
  int64_t B, Hq, Hkv, Tq, Tkv, D;
  float scale;
  const sdpa_mask* mask;
  void* ws;
  size_t wsn;
} fwd_args;

static fwd_args fwd_base(void) {
  fwd_args a = {FAKE, FAKE, FAKE, FAKE, SDPA_BF16, SDPA_BF16, SDPA_BHSD, 1, 2, 2, 8, 8, 64, NAN, NULL, NULL, 0};
  return a;
}

static void fwd_both(fwd_args a, int want, const char* what) {
  char name[160];
  snprintf(name, sizeof(name), "sdpa_fwd %s", what);
  expect(sdpa_fwd(a.q, a.k, a.v, a.o, a.dtype, a.out_dtype, a.layout, a.B, a.Hq, a.Hkv, a.Tq, a.Tkv, a.D, a.scale,
                  a.mask, NULL, a.ws, a.wsn, NULL), want, name);
  snprintf(name, sizeof(name), "sdpa_fwd_noalloc %s", what);
  expect(sdpa_fwd_noalloc(a.q, a.k, a.v, a.o, a.dtype, a.out_dtype, a.layout, a.B, a.Hq, a.Hkv, a.Tq, a.Tkv, a.D,
                          a.scale, a.mask, NULL, NULL), want, name);
}

static const int64_t extremes[] = {-1, 0, 1, 3, 64, 4096, 65535, 65536, INT32_MAX, (int64_t)INT32_MAX + 1,
                                   (int64_t)1 << 40, INT64_MAX / 2, INT64_MAX, INT64_MIN};
#define NX ((int)(sizeof(extremes) / sizeof(extremes[0])))

static void fwd_cases(void) {
  fwd_args a;
  a = fwd_base(); a.q = NULL; fwd_both(a, SDPA_ERR_INVALID, "null q");
  a = fwd_base(); a.k = NULL; fwd_both(a, SDPA_ERR_INVALID, "null k");
  a = fwd_base(); a.v = NULL; fwd_both(a, SDPA_ERR_INVALID, "null v");
  a = fwd_base(); a.o = NULL; fwd_both(a, SDPA_ERR_INVALID, "null o");
  a = fwd_base(); a.B = 0; fwd_both(a, SDPA_ERR_INVALID, "B=0");
  a = fwd_base(); a.Tq = -3; fwd_both(a, SDPA_ERR_INVALID, "Tq<0");
  a = fwd_base(); a.Tkv = INT64_MIN; fwd_both(a, SDPA_ERR_INVALID, "Tkv=min");
  a = fwd_base(); a.D = 0; fwd_both(a, SDPA_ERR_INVALID, "D=0");
  a = fwd_base(); a.Hq = 3; fwd_both(a, SDPA_ERR_INVALID, "Hq%Hkv");
  a = fwd_base(); a.dtype = 7; fwd_both(a, SDPA_ERR_INVALID, "dtype");
  a = fwd_base(); a.out_dtype = -1; fwd_both(a, SDPA_ERR_INVALID, "out_dtype");
  a = fwd_base(); a.dtype = SDPA_F32; fwd_both(a, SDPA_ERR_INVALID, "fp32 in, bf16 out");
  a = fwd_base(); a.layout = 9; fwd_both(a, SDPA_ERR_INVALID, "layout");
  a = fwd_base(); a.D = 48; fwd_both(a, SDPA_ERR_UNSUPPORTED, "D=48");
  a = fwd_base(); a.D = INT64_MAX; fwd_both(a, SDPA_ERR_UNSUPPORTED, "D=max");
  a = fwd_base(); a.B = INT64_MAX; fwd_both(a, SDPA_ERR_UNSUPPORTED, "B=max");
  a = fwd_base(); a.Hq = a.Hkv = INT64_MAX; fwd_both(a, SDPA_ERR_UNSUPPORTED, "H=max");
  a = fwd_base(); a.Tq = a.Tkv = INT64_MAX; fwd_both(a, SDPA_ERR_UNSUPPORTED, "T=max");
  /* in the grid limits one by one, but more elements than any device holds */
  a = fwd_base(); a.B = 65535; a.Hq = a.Hkv = 65535; a.Tq = a.Tkv = INT32_MAX; a.D = 128;
  fwd_both(a, SDPA_ERR_UNSUPPORTED, "elements beyond memory");
  /* split-KV route without a workspace (sdpa_fwd only; the fixed scratch covers it) */
  a = fwd_base(); a.D = 16; a.Tq = 1; a.Tkv = 4096; a.Hq = a.Hkv = 4;
  expect(sdpa_fwd(a.q, a.k, a.v, a.o, a.dtype, a.out_dtype, a.layout, a.B, a.Hq, a.Hkv, a.Tq, a.Tkv, a.D, a.scale,
                  NULL, NULL, NULL, 0, NULL), SDPA_ERR_WORKSPACE, "sdpa_fwd split-KV without workspace");
  /* split-KV partials larger than the allocation-free entry point's scratch */
  a = fwd_base(); a.D = 16; a.Tq = 8; a.Tkv = 1 << 20; a.Hq = a.Hkv = 64; a.B = 1;
  expect(sdpa_set_tuning("num_splits", 1024), SDPA_OK, "set num_splits");
  expect(sdpa_fwd_noalloc(a.q, a.k, a.v, a.o, a.dtype, a.out_dtype, a.layout, a.B, a.Hq, a.Hkv, a.Tq, a.Tkv, a.D,
                          a.scale, NULL, NULL, NULL), SDPA_ERR_UNSUPPORTED, "sdpa_fwd_noalloc beyond scratch");
  expect(sdpa_set_tuning("num_splits", 0), SDPA_OK, "reset num_splits");

  sdpa_mask m;
  memset(&m, 0, sizeof(m));
  a = fwd_base(); a.mask = &m;
  m.kind = SDPA_MASK_SLIDING; m.window = 0; fwd_both(a, SDPA_ERR_INVALID, "window 0");
  m.kind = SDPA_MASK_ADDITIVE; m.data = NULL; fwd_both(a, SDPA_ERR_INVALID, "additive without data");
  m.kind = SDPA_MASK_BOOL; fwd_both(a, SDPA_ERR_INVALID, "bool without data");
  m.kind = SDPA_MASK_ADDITIVE; m.data = FAKE; m.data_dtype = SDPA_F16;
  fwd_both(a, SDPA_ERR_INVALID, "additive fp16 data");
  m.data_dtype = SDPA_F32; m.stride[2] = -1; fwd_both(a, SDPA_ERR_INVALID, "negative mask stride");
  m.stride[2] = 0; m.kind = 42; fwd_both(a, SDPA_ERR_INVALID, "mask kind");
  m.kind = -5; fwd_both(a, SDPA_ERR_INVALID, "negative mask kind");
}

static void relpos_cases(void) {
  float th[4], tw[4];
  /* sdpa_relpos_fwd */
  expect(sdpa_relpos_fwd(NULL, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 4, 4, 64, FAKE, FAKE, NAN, NULL, NULL, 0, NULL),
         SDPA_ERR_INVALID, "relpos null q");
  expect(sdpa_relpos_fwd(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 4, 4, 64, NULL, FAKE, NAN, NULL, NULL, 0, NULL),
         SDPA_ERR_INVALID, "relpos null table");
  for (int i = 0; i < NX; ++i)
    for (int j = 0; j < NX; ++j) {
      const int64_t gh = extremes[i], gw = extremes[j];
      const int ok_grid = gh > 0 && gw > 0;
      if (ok_grid && gh <= 1024 && gw <= 1024) continue;   /* a grid in range would launch */
      const int st = sdpa_relpos_fwd(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, gh, gw, 64, FAKE, FAKE, NAN, NULL, NULL,
                                     0, NULL);
      ++calls;
      if (!ok_grid && st != SDPA_ERR_INVALID) {
        ++failures;
        fprintf(stderr, "FAIL relpos grid %lld x %lld: status %d\n", (long long)gh, (long long)gw, st);
      }
      if (ok_grid && (gh > 1024 || gw > 1024) && st != SDPA_ERR_UNSUPPORTED) {
        ++failures;
        fprintf(stderr, "FAIL relpos large grid %lld x %lld: status %d\n", (long long)gh, (long long)gw, st);
      }
      (void)sdpa_relpos_fused(1, 64, gh, gw);
      (void)sdpa_relpos_fused(1, extremes[i], 64, 64);
    }
  expect(sdpa_relpos_fwd(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 4, 4, 48, FAKE, FAKE, NAN, NULL, NULL, 0, NULL),
         SDPA_ERR_UNSUPPORTED, "relpos D=48");
  expect(sdpa_relpos_fwd(FAKE, FAKE, FAKE, FAKE, 0, 0, 1, 1, 2, 1000, 1000, 128, FAKE, FAKE, NAN, NULL, NULL, 0,
                         NULL), SDPA_ERR_UNSUPPORTED, "relpos grid beyond the term staging");
  /* relpos_terms */
  expect(relpos_terms(FAKE, 1, 1, 1, 2, 4, 4, 64, FAKE, FAKE, NULL, tw, NULL), SDPA_ERR_INVALID, "terms null out");
  expect(relpos_terms(FAKE, 1, 1, 0, 2, 4, 4, 64, FAKE, FAKE, th, tw, NULL), SDPA_ERR_INVALID, "terms B=0");
  expect(relpos_terms(FAKE, 5, 1, 1, 2, 4, 4, 64, FAKE, FAKE, th, tw, NULL), SDPA_ERR_INVALID, "terms dtype");
  expect(relpos_terms(FAKE, 1, 3, 1, 2, 4, 4, 64, FAKE, FAKE, th, tw, NULL), SDPA_ERR_INVALID, "terms layout");
  for (int i = 0; i < NX; ++i) {
    const int64_t x = extremes[i];
    const int want = x <= 0 ? SDPA_ERR_INVALID : SDPA_ERR_UNSUPPORTED;
    if (x > 0 && x <= 1024) continue;           /* a valid size would launch */
    expect(relpos_terms(FAKE, 1, 1, 1, 2, x, 4, 64, FAKE, FAKE, th, tw, NULL), want, "terms grid_h extreme");
    expect(relpos_terms(FAKE, 1, 1, 1, 2, 4, x, 64, FAKE, FAKE, th, tw, NULL), want, "terms grid_w extreme");
    if (x > 65535 || x <= 0)
      expect(relpos_terms(FAKE, 1, 1, x, x, 4, 4, 64, FAKE, FAKE, th, tw, NULL), want, "terms B,H extreme");
  }
}

static void train_cases(void) {
  /* dropout keep bits */
  expect(sdpa_dropout_mask(1, 0, 0.2f, 1, 1, 8, 8, NULL, NULL), SDPA_ERR_INVALID, "keep null");
  expect(sdpa_dropout_mask(1, 0, 1.0f, 1, 1, 8, 8, FAKEU, NULL), SDPA_ERR_INVALID, "rate 1");
  expect(sdpa_dropout_mask(1, 0, NAN, 1, 1, 8, 8, FAKEU, NULL), SDPA_ERR_INVALID, "rate nan");
  expect(sdpa_dropout_mask(1, 0, -0.1f, 1, 1, 8, 8, FAKEU, NULL), SDPA_ERR_INVALID, "rate < 0");
  expect(sdpa_dropout_mask(1, 0, 0.2f, INT64_MAX, INT64_MAX, 8, 8, FAKEU, NULL), SDPA_ERR_UNSUPPORTED, "keep B*H max");
  expect(sdpa_dropout_mask(1, 0, 0.2f, 1, 1, INT64_MAX, 8, FAKEU, NULL), SDPA_ERR_UNSUPPORTED, "keep Tq max");
  /* dropout forward */
  expect(sdpa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL, NULL, 0.2f, NULL, NULL, 0,
                          NULL), SDPA_ERR_INVALID, "dropout fwd keep null");
  expect(sdpa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL, FAKEU, 2.0f, NULL, NULL, 0,
                          NULL), SDPA_ERR_INVALID, "dropout fwd rate");
  expect(sdpa_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, INT64_MAX, 2, 2, 8, 8, 64, NAN, NULL, FAKEU, 0.2f, NULL,
                          NULL, 0, NULL), SDPA_ERR_UNSUPPORTED, "dropout fwd B max");
  /* backward */
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, NULL, 1, 1, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL,
                  NULL, 0.f, NULL, 0, NULL), SDPA_ERR_INVALID, "bwd null dv");
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, 1, 1, 2, 1, 1, 2, 2, 8, 8, 64, NAN, NULL,
                  NULL, 0.f, NULL, 0, NULL), SDPA_ERR_INVALID, "bwd grad dtype");
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, 1, 1, 1, 1, 1, 2, 2, 8, 8, 64, INFINITY,
                  NULL, NULL, 0.f, NULL, 0, NULL), SDPA_ERR_INVALID, "bwd scale inf");
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, 0, 0, 0, 1, 1, 2, 2, 8, 8, 64, NAN, NULL,
                  NULL, 0.f, NULL, 0, NULL), SDPA_ERR_UNSUPPORTED, "bwd fp32");
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, 1, 1, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL,
                  NULL, 0.f, NULL, 0, NULL), SDPA_ERR_WORKSPACE, "bwd without workspace");
  expect(sdpa_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, 1, 1, 1, 1, INT64_MAX, 2, 2, 8, 8, 64, NAN,
                  NULL, NULL, 0.f, NULL, 0, NULL), SDPA_ERR_UNSUPPORTED, "bwd B max");
  /* rel-pos backward */
  expect(sdpa_relpos_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, NULL, FAKEF, 1, 1, 1, 1, 1, 2, 8, 8,
                         64, FAKE, FAKE, NAN, NULL, 0, NULL), SDPA_ERR_INVALID, "relpos bwd null table grad");
  for (int i = 0; i < NX; ++i) {
    const int64_t x = extremes[i];
    const int st = sdpa_relpos_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, FAKEF, FAKEF, 1, 1, 1, 1, 1,
                                   2, x, x, 64, FAKE, FAKE, NAN, NULL, 0, NULL);
    ++calls;
    if (st == SDPA_OK) {
      ++failures;
      fprintf(stderr, "FAIL relpos bwd grid %lld: accepted without a workspace\n", (long long)x);
    }
  }
  /* rel-pos with dropout: forward and backward */
  expect(sdpa_relpos_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 8, 8, 64, FAKE, FAKE, NAN, NULL, 0.2f, NULL,
                                 NULL, 0, NULL), SDPA_ERR_INVALID, "relpos dropout fwd keep null");
  expect(sdpa_relpos_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 8, 8, 64, FAKE, FAKE, NAN, FAKEU, 1.0f, NULL,
                                 NULL, 0, NULL), SDPA_ERR_INVALID, "relpos dropout fwd rate");
  expect(sdpa_relpos_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 1, 2, 8, 8, 64, FAKE, FAKE, NAN, FAKEU, 0.2f, NULL,
                                 NULL, 0, NULL), SDPA_ERR_WORKSPACE, "relpos dropout fwd without workspace");
  expect(sdpa_relpos_fwd_dropout(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, INT64_MAX, 2, 8, 8, 64, FAKE, FAKE, NAN, FAKEU,
                                 0.2f, NULL, NULL, 0, NULL), SDPA_ERR_UNSUPPORTED, "relpos dropout fwd B max");
  expect(sdpa_relpos_bwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, FAKEF, FAKEF, 1, 1, 1, 1, 1, 2,
                                 8, 8, 64, FAKE, FAKE, NAN, NULL, 0.2f, NULL, 0, NULL), SDPA_ERR_INVALID,
         "relpos dropout bwd keep null");
  expect(sdpa_relpos_bwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, FAKEF, FAKEF, 1, 1, 1, 1, 1, 2,
                                 8, 8, 64, FAKE, FAKE, NAN, FAKEU, -0.5f, NULL, 0, NULL), SDPA_ERR_INVALID,
         "relpos dropout bwd rate");
  expect(sdpa_relpos_bwd_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, FAKEF, FAKE, FAKE, FAKE, FAKEF, FAKEF, 1, 1, 1, 1, 1, 2,
                                 8, 8, 64, FAKE, FAKE, NAN, FAKEU, 0.2f, NULL, 0, NULL), SDPA_ERR_WORKSPACE,
         "relpos dropout bwd without workspace");
  /* attention weights */
  expect(sdpa_attention_weights(FAKE, FAKE, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL, NULL, NULL, 0.f, FAKEF, NULL),
         SDPA_ERR_INVALID, "weights null lse");
  expect(sdpa_attention_weights(FAKE, FAKE, 1, 1, 1, 2, 2, 8, 8, 64, NAN, NULL, FAKEF, FAKEU, 1.5f, FAKEF, NULL),
         SDPA_ERR_INVALID, "weights rate");
  expect(sdpa_attention_weights(FAKE, FAKE, 1, 1, 4096, 64, 64, 8, 8, 64, NAN, NULL, FAKEF, NULL, 0.f, FAKEF, NULL),
         SDPA_ERR_UNSUPPORTED, "weights B*H beyond grid");
}

/* Size queries: every combination of extreme arguments returns a value (or
   the (size_t)-1 refusal) without undefined behaviour on the way. */
static void size_sweeps(void) {
  size_t sink = 0;
  for (int i = 0; i < NX; ++i)
    for (int j = 0; j < NX; ++j)
      for (int d = 0; d < 3; ++d) {
        const int64_t x = extremes[i], y = extremes[j];
        const int64_t D = d == 0 ? 16 : (d == 1 ? 64 : y);
        sink ^= sdpa_workspace_size(1, x, 4, 4, 8, y, D, NAN, 0, 0, 0);
        sink ^= sdpa_workspace_size(1, 1, x, 1, y, 4096, 16, NAN, 0, 0, 0);
        sink ^= sdpa_workspace_size(0, 1, 2, 2, x * 0 + 16, 16, D, 0.f, 1, x, y);
        sink ^= sdpa_workspace_size(1, x, 2, 2, 4096, 4096, 64, NAN, 1, 64, 64);
        sink ^= sdpa_workspace_size(2, 1, 12, 12, 196, 196, D, NAN, 1, x, y);
        sink ^= sdpa_bwd_workspace_size(x, y, 4096);
        sink ^= sdpa_bwd_workspace_size(1, x, y);
        sink ^= sdpa_relpos_bwd_workspace_size(x, 12, 64, 64, 64);
        sink ^= sdpa_relpos_bwd_workspace_size(1, 1, x, y, 64);
        sink ^= sdpa_relpos_bwd_workspace_size(1, 1, 14, 14, x);
        sink ^= sdpa_relpos_fwd_dropout_workspace_size(x, y, 64, 64);
        sink ^= sdpa_relpos_fwd_dropout_workspace_size(1, 2, x, y);
        calls += 12;
      }
  /* the documented refusal and a few exact values */
  expect(sdpa_workspace_size(1, 0, 2, 2, 8, 8, 64, NAN, 0, 0, 0) == (size_t)-1, 1, "ws B=0 refused");
  expect(sdpa_workspace_size(1, 1, 2, 2, 16, 16, 64, NAN, 1, 4, 5) == (size_t)-1, 1, "ws grid != T refused");
  expect(sdpa_workspace_size(1, 1, 2, 2, 8, 8, 64, NAN, 0, 0, 0) == 0, 1, "ws no split");
  expect(sdpa_bwd_workspace_size(1, 2, 8) == 256, 1, "bwd ws rounded to 256");
  if (sink == 0x5eed) puts("");               /* keep the sweep from being optimised out */
}

static void misc_cases(void) {
  const int codes[] = {SDPA_OK, SDPA_ERR_INVALID, SDPA_ERR_UNSUPPORTED, SDPA_ERR_WORKSPACE, SDPA_ERR_HIP, 7, -99,
                       INT32_MIN, INT32_MAX};
  for (unsigned i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
    const char* s = sdpa_status_string(codes[i]);
    ++calls;
    if (!s || !s[0]) {
      ++failures;
      fprintf(stderr, "FAIL status string %d\n", codes[i]);
    }
  }
  expect(sdpa_set_tuning(NULL, 1), SDPA_ERR_INVALID, "tuning null key");
  expect(sdpa_set_tuning("no_such_knob", 1), SDPA_ERR_INVALID, "tuning unknown key");
  expect(sdpa_set_tuning("num_splits", -1), SDPA_ERR_INVALID, "tuning negative");
  expect(sdpa_set_tuning("num_splits", INT64_MAX), SDPA_ERR_INVALID, "tuning huge");
  expect(sdpa_set_tuning("num_splits", 0), SDPA_OK, "tuning reset");
  (void)sdpa_last_kernel();
  /* a long message is cut to the buffer, not written past it */
  expect(sdpa_fwd(FAKE, FAKE, FAKE, FAKE, 1, 1, 1, INT64_MIN, INT64_MIN, INT64_MIN, INT64_MIN, INT64_MIN, INT64_MIN,
                  NAN, NULL, NULL, NULL, 0, NULL), SDPA_ERR_INVALID, "long error message");
}

int main(void) {
  fwd_cases();
  relpos_cases();
  train_cases();
  size_sweeps();
  misc_cases();
  printf("%d calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
