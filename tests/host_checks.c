/* Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code of the library
 * (tests/test_host_sanitizers.py builds and runs this).  Every call here
 * returns before any kernel launch: parameter validation, null arguments,
 * the span bound, a context on a device that may not exist, and a sweep of
 * random and extreme parameter values through the validation arithmetic.
 * With a device present it also imports a small ragged index from host
 * arrays into each tier, reads it back and compares every array bit for bit,
 * and checks use after free: the host packing and unpacking code runs under
 * the sanitizers (no kernel is launched).
 * Prints "host checks passed: N" and exits 0, or lists the failures and
 * exits 1; a sanitizer report aborts the run. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sekv.h"

static int n_checks = 0, n_fail = 0;

#define CHECK(cond, what)                                               \
  do {                                                                  \
    ++n_checks;                                                         \
    if (!(cond)) {                                                      \
      ++n_fail;                                                         \
      printf("FAIL line %d: %s (%s)\n", __LINE__, what, sekv_last_error()); \
    }                                                                   \
  } while (0)

/* the 32K single-layer 8B-shaped workload */
static sekv_build_params valid_params(void) {
  sekv_build_params p;
  memset(&p, 0, sizeof p);
  p.B = 1; p.L = 1; p.Hq = 32; p.Hkv = 8; p.d = 128; p.T = 32768;
  p.R = 32; p.dprime = 64; p.alpha_sp = 2.0f; p.l_min = 8;
  p.oversample = 8; p.power_iters = 2; p.seed = 0;
  p.tier = SEKV_TIER_HBM; p.ring_bytes = 0; p.gate_eps = 0.0f;
  return p;
}

/* 64-bit linear congruential generator (Knuth's MMIX constants) */
static uint64_t lcg = 88172645463325252ull;
static uint32_t next_u32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}
static int32_t pick_i32(void) {
  static const int32_t edge[] = {0, 1, -1, 2, 7, 8, 16, 17, 31, 32, 48, 63, 64, 65, 96, 127, 128,
                                 256, 65535, 65536, 131072, 1 << 20, 1 << 30, INT32_MAX, INT32_MIN};
  const uint32_t r = next_u32();
  if (r & 1u) return edge[(r >> 1) % (sizeof edge / sizeof edge[0])];
  return (int32_t)next_u32();
}

static void check_validation(void) {
  sekv_build_params p = valid_params();
  CHECK(sekv_validate_params(&p) == SEKV_OK, "the 32K workload validates");
  p.T = 131072; p.L = 32; p.R = 16;
  CHECK(sekv_validate_params(&p) == SEKV_OK, "the 128K 32-layer workload validates");
  p = valid_params(); p.B = 32; p.Hq = 64; p.T = 65536; p.R = 64;
  CHECK(sekv_validate_params(&p) == SEKV_OK, "the 70B-shaped batch validates");

  struct { const char* what; int32_t* field; int32_t value; sekv_status status; } ic[] = {
      {"Hkv not dividing Hq", &p.Hkv, 7, SEKV_EINVAL},
      {"d = 96", &p.d, 96, SEKV_EUNSUPPORTED},
      {"R above d", &p.R, 256, SEKV_EINVAL},
      {"R = 48", &p.R, 48, SEKV_EUNSUPPORTED},
      {"G = 16", &p.Hkv, 2, SEKV_EUNSUPPORTED},
      {"l_min = 0", &p.l_min, 0, SEKV_EINVAL},
      {"oversample 17", &p.oversample, 17, SEKV_EINVAL},
      {"power_iters -1", &p.power_iters, -1, SEKV_EINVAL},
      {"dprime 0", &p.dprime, 0, SEKV_EUNSUPPORTED},
      {"dprime 65", &p.dprime, 65, SEKV_EUNSUPPORTED},
      {"T = 0", &p.T, 0, SEKV_EINVAL},
      {"B = 0", &p.B, 0, SEKV_EINVAL},
      {"tier 5", &p.tier, 5, SEKV_EINVAL},
      {"T = 2M", &p.T, 2000000, SEKV_EUNSUPPORTED},
  };
  for (size_t i = 0; i < sizeof ic / sizeof ic[0]; ++i) {
    p = valid_params();
    /* the field pointers above point into p, which is rebuilt in place */
    *ic[i].field = ic[i].value;
    const sekv_status st = sekv_validate_params(&p);
    CHECK(st == ic[i].status, ic[i].what);
    CHECK(st == SEKV_OK || sekv_last_error()[0] != '\0', "a refusal leaves a message");
  }
  p = valid_params(); p.alpha_sp = NAN;
  CHECK(sekv_validate_params(&p) == SEKV_EINVAL, "alpha_sp NaN");
  p = valid_params(); p.alpha_sp = INFINITY;
  CHECK(sekv_validate_params(&p) == SEKV_EINVAL, "alpha_sp inf");
  p = valid_params(); p.gate_eps = NAN;
  CHECK(sekv_validate_params(&p) == SEKV_EINVAL, "gate_eps NaN");
  p = valid_params(); p.ring_bytes = -1;
  CHECK(sekv_validate_params(&p) == SEKV_EINVAL, "ring_bytes -1");

  /* extreme sizes: refused, or accepted only when every product fits */
  const int32_t big[] = {INT32_MAX, INT32_MAX / 2, 1 << 30, 1 << 24};
  for (size_t i = 0; i < sizeof big / sizeof big[0]; ++i) {
    int32_t* fields[] = {&p.B, &p.L, &p.Hq, &p.T};
    for (size_t f = 0; f < 4; ++f) {
      p = valid_params();
      *fields[f] = big[i];
      (void)sekv_validate_params(&p);   /* any status; the sanitizers watch the arithmetic */
    }
  }
  p = valid_params(); p.B = INT32_MAX; p.L = INT32_MAX; p.T = INT32_MAX;
  CHECK(sekv_validate_params(&p) != SEKV_OK, "B = L = T = INT32_MAX refused");

  /* random fields through the validation arithmetic */
  for (int it = 0; it < 200000; ++it) {
    p = valid_params();
    switch (next_u32() % 10) {
      case 0: p.B = pick_i32(); break;
      case 1: p.L = pick_i32(); break;
      case 2: p.Hq = pick_i32(); p.Hkv = pick_i32(); break;
      case 3: p.d = pick_i32(); p.R = pick_i32(); break;
      case 4: p.T = pick_i32(); p.l_min = pick_i32(); break;
      case 5: p.dprime = pick_i32(); break;
      case 6: p.oversample = pick_i32(); p.power_iters = pick_i32(); break;
      case 7: p.tier = pick_i32(); p.ring_bytes = (int64_t)pick_i32() * 1048576; break;
      case 8: p.B = pick_i32(); p.L = pick_i32(); p.Hq = pick_i32(); p.T = pick_i32(); break;
      default: p.alpha_sp = (float)(int32_t)next_u32() * 1e-9f; p.gate_eps = (float)(int32_t)next_u32(); break;
    }
    const sekv_status st = sekv_validate_params(&p);
    if (st != SEKV_OK && st != SEKV_EINVAL && st != SEKV_EUNSUPPORTED) {
      CHECK(0, "validation returns OK, EINVAL or EUNSUPPORTED");
      break;
    }
  }
}

static void check_span_bound(void) {
  CHECK(sekv_max_spans(0, 8) == 0 && sekv_max_spans(10, 0) == 0, "degenerate span bounds");
  CHECK(sekv_max_spans(131072, 8) == 14563, "spans of a 128K context");
  for (int T = 1; T < 60; ++T)
    for (int lm = 1; lm < 10; ++lm) {
      int best = 0;
      for (int k = 0; k <= T; ++k)
        if (k * lm + (k > 0 ? k - 1 : 0) <= T) best = k;
      if (sekv_max_spans(T, lm) != best) {
        CHECK(0, "span bound against brute force");
        return;
      }
    }
  for (int it = 0; it < 100000; ++it) {
    const int32_t T = pick_i32(), lm = pick_i32();
    const int32_t k = sekv_max_spans(T, lm);
    if (k < 0 || (T > 0 && lm > 0 && (int64_t)k * lm + (k > 0 ? k - 1 : 0) > T)) {
      CHECK(0, "span bound within the context");
      return;
    }
  }
}

static void check_null_arguments(void) {
  sekv_build_params p = valid_params();
  sekv_index* out = NULL;
  float f = 0.f;
  uint64_t w = 0;
  CHECK(sekv_build_index(NULL, &p, &f, &f, &f, &f, NULL, &out) == SEKV_EINVAL, "build without a context");
  CHECK(sekv_index_import(NULL, &p, NULL, &out) == SEKV_EINVAL, "import without a context");
  CHECK(sekv_route(NULL, NULL, 0, 1, &f, &f, 0, &w, NULL) == SEKV_EINVAL, "route without a context");
  CHECK(sekv_route_pooled(NULL, NULL, 0, 1, &f, &f, 5, &w, NULL) == SEKV_EINVAL, "pooled route without a context");
  CHECK(sekv_decode_attend(NULL, NULL, 0, 1, &f, &w, &f, NULL) == SEKV_EINVAL, "decode without a context");
  CHECK(sekv_decode_attend_noalloc(NULL, NULL, 0, 1, &f, &w, &f, NULL) == SEKV_EINVAL,
        "no-allocation decode without a context");
  CHECK(sekv_calibrate_tau(NULL, NULL, 0, 1, &f, 0.1f, &f) == SEKV_EINVAL, "calibration without a context");
  CHECK(sekv_index_get_info(NULL, NULL) == SEKV_EINVAL, "info of no index");
  CHECK(sekv_index_counts(NULL, NULL, NULL) == SEKV_EINVAL, "counts of no index");
  CHECK(sekv_validate_params(NULL) == SEKV_EINVAL, "validate nothing");
  CHECK(strstr(sekv_last_error(), "null") != NULL, "the message names the null argument");
  CHECK(sekv_timing_enable(NULL, 1) == SEKV_EINVAL, "timing without a context");
  sekv_destroy(NULL);
  sekv_index_free(NULL);
}

/* bf16 bit pattern of a value in [-1, 1) (exactly representable) */
static uint16_t rand_bf16(void) {
  const float f = (float)((int32_t)next_u32()) * (1.0f / 2147483648.0f);
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static float rand_sigma(void) { return 0.25f + (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }

/* import -> export round trip of a two-sequence, two-layer index (G = 2,
 * d = 64, R = 16, d' = 8, T = 100) with random span partitions */
static void check_roundtrip(sekv_ctx* c, int tier) {
  enum { B = 2, L = 2, HQ = 4, HKV = 2, D = 64, R = 16, DP = 8, T = 100 };
  int32_t n_spans[B], n_raw[B];
  int32_t span_start[2 * T], span_len[2 * T], raw_pos[2 * T];
  int ns_all = 0, nr_all = 0, ntok_all = 0, nres_all = 0;
  for (int b = 0; b < B; ++b) {
    int ns = 0, nr = 0;
    for (int t = 0; t < T;) {
      const int len = (next_u32() % 3 == 0 || t == 0) ? 0 : 1 + (int)(next_u32() % 12);
      if (len == 0 || t + len > T) {
        raw_pos[nr_all + nr++] = t++;
      } else {
        span_start[ns_all + ns] = t;
        span_len[ns_all + ns++] = len;
        ntok_all += len;
        t += len;
      }
    }
    n_spans[b] = ns;
    n_raw[b] = nr;
    ns_all += ns;
    nr_all += nr;
    nres_all += ns + nr;
  }
  const size_t n_kres = (size_t)L * HKV * nres_all * D, n_s = (size_t)L * HQ * DP * ns_all;
  const size_t n_u = (size_t)L * HKV * ntok_all * R, n_vt = (size_t)L * HKV * ns_all * R * D;
  const size_t n_sm = (size_t)L * HKV * ns_all * R, n_w = (size_t)L * HQ * DP * D;
  uint16_t* kres = malloc(2 * n_kres); uint16_t* vres = malloc(2 * n_kres);
  float* sk = malloc(4 * n_s);
  uint16_t* uk = malloc(2 * n_u); uint16_t* uv = malloc(2 * n_u);
  uint16_t* vkt = malloc(2 * n_vt); uint16_t* vvt = malloc(2 * n_vt);
  float* smk = malloc(4 * n_sm); float* smv = malloc(4 * n_sm);
  float* W = malloc(4 * n_w);
  for (size_t i = 0; i < n_kres; ++i) { kres[i] = rand_bf16(); vres[i] = rand_bf16(); }
  for (size_t i = 0; i < n_s; ++i) sk[i] = (float)(int32_t)next_u32() * 1e-9f;
  for (size_t i = 0; i < n_u; ++i) { uk[i] = rand_bf16(); uv[i] = rand_bf16(); }
  for (size_t i = 0; i < n_vt; ++i) { vkt[i] = rand_bf16(); vvt[i] = rand_bf16(); }
  for (size_t i = 0; i < n_sm; ++i) { smk[i] = rand_sigma(); smv[i] = rand_sigma(); }
  for (size_t i = 0; i < n_w; ++i) W[i] = (float)(int32_t)next_u32() * 1e-9f;

  sekv_build_params p;
  memset(&p, 0, sizeof p);
  p.B = B; p.L = L; p.Hq = HQ; p.Hkv = HKV; p.d = D; p.T = T; p.R = R; p.dprime = DP;
  p.alpha_sp = 2.0f; p.l_min = 1; p.oversample = 8; p.power_iters = 2; p.tier = tier;
  sekv_host_index h = {n_spans, n_raw, span_start, span_len, raw_pos, kres, vres, sk,
                       uk, uv, vkt, vvt, smk, smv, W};
  sekv_index* x = NULL;
  const sekv_status st = sekv_index_import(c, &p, &h, &x);
  CHECK(st == SEKV_OK && x != NULL, "import of a ragged two-sequence index");
  if (st == SEKV_OK) {
    sekv_index_info info;
    CHECK(sekv_index_get_info(x, &info) == SEKV_OK && info.total_spans == ns_all &&
              info.total_raw == nr_all && info.total_span_tokens == ntok_all && info.tier == tier,
          "index info after import");
    int32_t cs[B], cr[B];
    CHECK(sekv_index_counts(x, cs, cr) == SEKV_OK && cs[0] == n_spans[0] && cs[1] == n_spans[1] &&
              cr[0] == n_raw[0] && cr[1] == n_raw[1], "span and raw counts after import");
    int32_t* o_ss = calloc(ns_all, 4); int32_t* o_sl = calloc(ns_all, 4); int32_t* o_rp = calloc(nr_all, 4);
    uint16_t* o_kres = calloc(n_kres, 2); uint16_t* o_vres = calloc(n_kres, 2);
    float* o_s = calloc(n_s, 4);
    uint16_t* o_uk = calloc(n_u, 2); uint16_t* o_uv = calloc(n_u, 2);
    uint16_t* o_vkt = calloc(n_vt, 2); uint16_t* o_vvt = calloc(n_vt, 2);
    float* o_smk = calloc(n_sm, 4); float* o_smv = calloc(n_sm, 4);
    int32_t* o_rank = calloc(2 * n_sm / R, 4);
    sekv_host_index_out o = {o_ss, o_sl, o_rp, o_kres, o_vres, o_s, o_uk, o_uv, o_vkt, o_vvt, o_smk, o_smv, o_rank};
    CHECK(sekv_index_export(c, x, &o) == SEKV_OK, "export");
    CHECK(!memcmp(o_ss, span_start, 4 * ns_all) && !memcmp(o_sl, span_len, 4 * ns_all) &&
              !memcmp(o_rp, raw_pos, 4 * nr_all), "span tables round trip");
    CHECK(!memcmp(o_kres, kres, 2 * n_kres) && !memcmp(o_vres, vres, 2 * n_kres), "resident rows round trip");
    CHECK(!memcmp(o_s, sk, 4 * n_s), "summary keys round trip");
    CHECK(!memcmp(o_uk, uk, 2 * n_u) && !memcmp(o_uv, uv, 2 * n_u), "left factors round trip");
    CHECK(!memcmp(o_vkt, vkt, 2 * n_vt) && !memcmp(o_vvt, vvt, 2 * n_vt), "right factors round trip");
    CHECK(!memcmp(o_smk, smk, 4 * n_sm) && !memcmp(o_smv, smv, 4 * n_sm), "sigma m round trip");
    int ranks_ok = 1;
    for (size_t i = 0; i < 2 * n_sm / R; ++i) ranks_ok &= o_rank[i] == R;
    CHECK(ranks_ok, "every blob stores R components");
    CHECK(sekv_index_export_part(c, x, 1, 1, 1, 1, &o) == SEKV_OK, "partial export");
    CHECK(sekv_index_export_part(c, x, 1, 2, 0, 1, &o) == SEKV_EINVAL, "partial export past B");
    CHECK(sekv_index_export_part(c, x, 0, 1, 1, 2, &o) == SEKV_EINVAL, "partial export past L");
    free(o_ss); free(o_sl); free(o_rp); free(o_kres); free(o_vres); free(o_s); free(o_uk); free(o_uv);
    free(o_vkt); free(o_vvt); free(o_smk); free(o_smv); free(o_rank);
    sekv_index_free(x);
    CHECK(sekv_index_get_info(x, &info) == SEKV_ESTATE, "info of a freed index");
    CHECK(sekv_index_export(c, x, &o) == SEKV_ESTATE, "export of a freed index");
    sekv_index_free(x);   /* a second free is a no-op */
  }
  /* a partition with a gap is refused before any device work */
  span_len[0] += 1;
  x = NULL;
  CHECK(sekv_index_import(c, &p, &h, &x) == SEKV_EINVAL && x == NULL, "import of overlapping spans refused");
  span_len[0] -= 1;
  free(kres); free(vres); free(sk); free(uk); free(uv); free(vkt); free(vvt); free(smk); free(smv); free(W);
}

static void check_context(void) {
  sekv_ctx* c = NULL;
  const sekv_status st = sekv_create(0, NULL, &c);
  if (st == SEKV_OK) {
    CHECK(c != NULL, "a created context");
    check_roundtrip(c, SEKV_TIER_HBM);
    check_roundtrip(c, SEKV_TIER_PINNED_HOST);
    sekv_destroy(c);
    CHECK(sekv_index_import(c, NULL, NULL, NULL) != SEKV_OK, "a destroyed context is refused");
  } else {
    CHECK(st == SEKV_EHIP && c == NULL, "no device: EHIP and no context");
    CHECK(sekv_last_error()[0] != '\0', "no device: a message");
  }
  CHECK(sekv_create(-1, NULL, &c) != SEKV_OK, "device -1 refused");
  CHECK(sekv_create(0, NULL, NULL) == SEKV_EINVAL, "create without an output");
}

int main(void) {
  check_validation();
  check_span_bound();
  check_null_arguments();
  check_context();
  if (n_fail) {
    printf("host checks failed: %d of %d\n", n_fail, n_checks);
    return 1;
  }
  printf("host checks passed: %d\n", n_checks);
  return 0;
}
