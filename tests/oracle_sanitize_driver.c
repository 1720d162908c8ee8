/* Drives every entry point of the oracle over ragged sizes, all modes and
 * flag combinations, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py). The oracle
 * source is compiled into this translation unit; inputs come from a small
 * linear congruential generator. Prints "ok" when every call returned. */
#include <stdio.h>

#include "../oracle/ps_oracle.c"

static uint64_t lcg = 88172645463325252ull;
static uint32_t rnd32(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(lcg >> 32);
}
static float rndf(float scale) { return ((float)(rnd32() >> 8) / 16777216.0f - 0.5f) * 2.0f * scale; }
static uint16_t rnd_bf16(float scale) {
  float x = rndf(scale);
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

static void fill_bf16(uint16_t* a, int64_t n, float s) { for (int64_t i = 0; i < n; ++i) a[i] = rnd_bf16(s); }
static void fill_u16(uint16_t* a, int64_t n) { for (int64_t i = 0; i < n; ++i) a[i] = (uint16_t)rnd32(); }
static void zero_moments(uint16_t* mc, float* ms, uint16_t* vc, float* vs, int64_t n) {
  for (int64_t i = 0; i < n; ++i) { mc[i] = 32768; vc[i] = 0; }
  for (int64_t b = 0; b < (n + ORC_BLOCK - 1) / ORC_BLOCK; ++b) { ms[b] = 0.0f; vs[b] = 0.0f; }
}

static void split_join_codec(void) {
  const int64_t sizes[] = {1, 7, 255, 256, 257, 1000};
  for (size_t k = 0; k < sizeof(sizes) / sizeof(sizes[0]); ++k) {
    int64_t n = sizes[k], nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
    float* w = malloc(n * sizeof(float));
    float* w2 = malloc(n * sizeof(float));
    uint16_t* hi = malloc(n * 2);
    uint16_t* lo = malloc(n * 2);
    uint16_t* code = malloc(n * 2);
    float* scale = malloc(nb * sizeof(float));
    uint8_t* b24 = malloc(n * 3);
    for (int64_t i = 0; i < n; ++i) w[i] = rndf(1e-3f);
    for (int mode = 0; mode < 2; ++mode) {
      orc_split(w, hi, lo, n, mode);
      orc_join(hi, lo, w2, n, mode);
    }
    for (int kind = 0; kind < 2; ++kind) {
      orc_encode(w, n, kind, code, scale);
      orc_decode(code, scale, n, kind, w2);
    }
    orc_f24_encode(w, n, b24);
    orc_f24_decode(b24, n, w2);
    orc_sr_rand16_array(3, 4, 5, 6, n, hi);
    uint32_t* km = malloc(n * sizeof(uint32_t));
    for (int64_t i = 0; i < n; ++i) w2[i] = (float)(i % 65536);
    orc_dec_mag_array(w2, n, ORC_UNSIGNED, w);
    for (int64_t i = 0; i < n; ++i) w[i] = (float)i / (float)n;
    orc_code_mag_array(w, n, ORC_SIGNED, km);
    free(km); free(w); free(w2); free(hi); free(lo); free(code); free(scale); free(b24);
  }
}

static void adam_steps(void) {
  const int64_t sizes[] = {1, 9, 256, 257, 1023, 3000};
  for (size_t k = 0; k < sizeof(sizes) / sizeof(sizes[0]); ++k) {
    int64_t n = sizes[k], nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
    uint16_t *hi = malloc(n * 2), *lo = malloc(n * 2), *g = malloc(n * 2), *mc = malloc(n * 2), *vc = malloc(n * 2);
    float *ms = malloc(nb * 4), *vs = malloc(nb * 4);
    for (int algo = 0; algo < 2; ++algo)
      for (int split = 0; split < 3; ++split)
        for (int wd = 0; wd < 2; ++wd) {
          orc_hparams hp = {algo, split, 1e-3, 0.9, 0.999, 1e-8, wd ? 0.01 : 0.0, 4e-3, 7, (int64_t)k, 0};
          fill_bf16(hi, n, 0.02f);
          fill_u16(lo, n);
          zero_moments(mc, ms, vc, vs, n);
          for (int t = 1; t <= 3; ++t) {
            fill_bf16(g, n, 1e-3f);
            orc_opt_step(hi, lo, g, mc, ms, vc, vs, n, &hp, t);
          }
          orc_opt_step(hi, lo, NULL, mc, ms, vc, vs, n, &hp, 4);
        }
    /* storage flags */
    float *w32 = malloc(n * 4), *g32 = malloc(n * 4), *m32 = malloc(n * 4), *v32 = malloc(n * 4);
    uint8_t *m24 = malloc(n * 3), *v24 = malloc(n * 3);
    const uint32_t flag_sets[] = {1, 2, 4, 3, 6};
    for (size_t f = 0; f < sizeof(flag_sets) / sizeof(flag_sets[0]); ++f) {
      uint32_t fl = flag_sets[f];
      orc_hparams hp = {1, 0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 4e-3, 0, 0, 0};
      for (int64_t i = 0; i < n; ++i) { w32[i] = rndf(0.02f); g32[i] = rndf(1e-3f); m32[i] = 0.0f; v32[i] = 0.0f; }
      memset(m24, 0, n * 3);
      memset(v24, 0, n * 3);
      fill_bf16(hi, n, 0.02f);
      fill_u16(lo, n);
      fill_bf16(g, n, 1e-3f);
      zero_moments(mc, ms, vc, vs, n);
      void* w = (fl & 2) ? (void*)w32 : (void*)hi;
      const void* gg = (fl & 2) ? (const void*)g32 : (const void*)g;
      void* m = (fl & 1) ? (void*)m32 : (fl & 4) ? (void*)m24 : (void*)mc;
      void* v = (fl & 1) ? (void*)v32 : (fl & 4) ? (void*)v24 : (void*)vc;
      for (int t = 1; t <= 2; ++t) orc_opt_step_flags(w, (fl & 2) ? NULL : lo, gg, m, ms, v, vs, n, fl, &hp, t);
    }
    float* cw = malloc(n * 4);
    for (int64_t i = 0; i < n; ++i) { cw[i] = rndf(0.02f); g32[i] = rndf(1e-3f); m32[i] = 0.0f; v32[i] = 0.0f; }
    orc_hparams hp = {0, 0, 1e-3, 0.9, 0.999, 1e-8, 0.0, 4e-3, 0, 0, 0};
    orc_core_step(cw, m32, v32, g32, n, &hp, 1);
    free(cw); free(w32); free(g32); free(m32); free(v32); free(m24); free(v24);
    free(hi); free(lo); free(g); free(mc); free(vc); free(ms); free(vs);
  }
}

static void factored_steps(void) {
  const int64_t shapes[][2] = {{1, 1}, {3, 5}, {17, 40}, {64, 300}, {1, 1000}, {700, 1}};
  for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k) {
    int64_t R = shapes[k][0], C = shapes[k][1], n = R * C, nb = (n + ORC_BLOCK - 1) / ORC_BLOCK;
    uint16_t *hi = malloc(n * 2), *lo = malloc(n * 2), *g = malloc(n * 2), *mc = malloc(n * 2), *vc = malloc(n * 2);
    float *ms = malloc(nb * 4), *vs = malloc(nb * 4), *row = malloc(R * 4), *col = malloc(C * 4);
    for (int split = 0; split < 3; split += 2)
      for (int fm = 0; fm < 2; ++fm)
        for (int sched = 0; sched < 2; ++sched) {
          orc_fhparams hp = {split, 0, 1e-3, 0.999, 1e-30, 1.0, 0.01, sched ? -0.8 : 0.0, fm ? 0.9 : 0.0, 11,
                             (int64_t)k};
          fill_bf16(hi, n, 0.02f);
          fill_u16(lo, n);
          zero_moments(mc, ms, vc, vs, n);
          for (int64_t i = 0; i < R; ++i) row[i] = 0.0f;
          for (int64_t j = 0; j < C; ++j) col[j] = 0.0f;
          for (int t = 1; t <= 3; ++t) {
            if (t == 2)
              memset(g, 0, n * 2); /* an all-zero gradient step */
            else
              fill_bf16(g, n, 1e-3f);
            orc_factored_2d(hi, lo, g, row, col, mc, ms, R, C, &hp, t);
            orc_factored_1d(hi, lo, g, vc, vs, mc, ms, n, &hp, t);
          }
          orc_factored_2d(hi, lo, NULL, row, col, mc, ms, R, C, &hp, 4);
          orc_factored_1d(hi, lo, NULL, vc, vs, mc, ms, n, &hp, 4);
        }
    free(hi); free(lo); free(g); free(mc); free(vc); free(ms); free(vs); free(row); free(col);
  }
}

int main(void) {
  split_join_codec();
  adam_steps();
  factored_steps();
  orc_coeffs c;
  orc_hparams hp = {1, 0, 3.5e-6, 0.9, 0.999, 1e-8, 0.0, 4e-3, 0, 0, 0};
  for (int64_t t = 1; t < 2000; t += 97) orc_coeffs_for(&hp, t, &c);
  printf("ok\n");
  return 0;
}
