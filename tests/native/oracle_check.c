/*
 * oracle_check.c — the C oracle (oracle/kamera_oracle.c) driven on small cases of every kind,
 * built with gcc under AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure:
 * it looks for memory and undefined-behaviour errors in the oracle's own code paths, and checks
 * a few closed forms on the way).
 *
 * Cases: fp32, bf16 and fp64 inputs; half-split and interleaved pairs; partial rotary widths;
 * a frequency table and per-pair shifts; patches of rank 0, 1 and 7 with padded row strides;
 * the bf16 rounding of specials and ties; page-table slots, including a table overrun.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kamera_oracle_segment_ex(int32_t dtype, const void* src, int64_t src_row_stride,
                             int32_t n_tokens, int32_t width, int32_t rotate, int32_t layout,
                             int32_t rot_dim, const double* inv_freq, const int64_t* pair_delta,
                             int64_t delta, double theta, int32_t m, const void* U,
                             int64_t u_row_stride, const void* V, int64_t v_row_stride,
                             double* out, double* abs_sum);
int kamera_oracle_segment(int32_t dtype, const void* src, int64_t src_row_stride,
                          int32_t n_tokens, int32_t width, int32_t rotate, int32_t layout,
                          int64_t delta, double theta, int32_t m, const void* U,
                          int64_t u_row_stride, const void* V, int64_t v_row_stride,
                          double* out, double* abs_sum);
void kamera_oracle_inv_freq(double theta, int32_t rot_dim, double* out);
void kamera_oracle_phase(int64_t delta, double theta, int32_t rot_dim, double* c, double* s);
void kamera_oracle_to_f32(const double* in, int64_t n, float* out);
void kamera_oracle_to_bf16(const double* in, int64_t n, uint16_t* out);
int kamera_oracle_slots(const int32_t* table, int32_t n_table, int32_t page_size,
                        int64_t dst_offset, int32_t n_tokens, int64_t* out);

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);               \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static uint64_t rng_state = 88172645463325252ull;
static double uniform(void) { /* xorshift64 in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 4503599627370496.0 - 1.0;
}
static uint16_t bf16_of(float f) { /* truncation: any bf16 pattern serves as an input */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* One head through every element type, with padded row strides (buffers sized exactly, so an
 * index past a row shows under the sanitizer). */
static void run_case(int dtype, int n_tokens, int width, int rotate, int layout, int rot_dim,
                     int use_table, int per_pair, int m) {
  const int ss = width + 3, us = m + 2, vs = m + 1;
  const size_t es = dtype == 0 ? 4 : (dtype == 1 ? 2 : 8);
  const size_t n_src = (size_t)(n_tokens > 0 ? (n_tokens - 1) * ss + width : 0);
  const size_t n_u = (size_t)(m > 0 && n_tokens > 0 ? (n_tokens - 1) * us + m : 0);
  const size_t n_v = (size_t)(m > 0 ? (width - 1) * vs + m : 0);
  void* src = malloc(n_src * es + 1);
  void* U = malloc(n_u * es + 1);
  void* V = malloc(n_v * es + 1);
  for (size_t i = 0; i < n_src; ++i) {
    const double x = uniform();
    if (dtype == 0) ((float*)src)[i] = (float)x;
    else if (dtype == 1) ((uint16_t*)src)[i] = bf16_of((float)x);
    else ((double*)src)[i] = x;
  }
  for (size_t i = 0; i < n_u; ++i) {
    const double x = 0.1 * uniform();
    if (dtype == 0) ((float*)U)[i] = (float)x;
    else if (dtype == 1) ((uint16_t*)U)[i] = bf16_of((float)x);
    else ((double*)U)[i] = x;
  }
  for (size_t i = 0; i < n_v; ++i) {
    const double x = 0.1 * uniform();
    if (dtype == 0) ((float*)V)[i] = (float)x;
    else if (dtype == 1) ((uint16_t*)V)[i] = bf16_of((float)x);
    else ((double*)V)[i] = x;
  }
  const int pairs = rot_dim / 2;
  double* table = use_table ? malloc(sizeof(double) * pairs) : NULL;
  int64_t* pd = per_pair ? malloc(sizeof(int64_t) * pairs) : NULL;
  for (int i = 0; i < pairs; ++i) {
    if (table) table[i] = pow(10.0, -6.0 * i / (pairs > 1 ? pairs - 1 : 1));
    if (pd) pd[i] = (i % 3) * 1000 - 777;
  }
  const size_t n_out = (size_t)n_tokens * width;
  double* out = malloc(sizeof(double) * n_out + 1);
  double* mag = malloc(sizeof(double) * n_out + 1);
  const int rc = kamera_oracle_segment_ex(dtype, src, ss, n_tokens, width, rotate, layout,
                                          rot_dim, table, pd, 4242, 1e4, m, U, us, V, vs, out,
                                          mag);
  CHECK(rc == 0);
  /* closed forms: |out| <= S; unrotated, unpatched elements are the input */
  for (size_t i = 0; i < n_out; ++i) CHECK(fabs(out[i]) <= mag[i] * (1 + 1e-15) + 1e-300);
  if (!rotate && m == 0 && dtype == 2)
    for (int t = 0; t < n_tokens; ++t)
      for (int f = 0; f < width; ++f)
        CHECK(out[(size_t)t * width + f] == ((double*)src)[(size_t)t * ss + f]);
  free(src);
  free(U);
  free(V);
  free(table);
  free(pd);
  free(out);
  free(mag);
}

int main(void) {
  for (int dtype = 0; dtype < 3; ++dtype)
    for (int layout = 0; layout < 2; ++layout)
      for (int m = 0; m <= 7; m += 7) {
        run_case(dtype, 33, 128, 1, layout, 128, 0, 0, m);
        run_case(dtype, 17, 96, 1, layout, 64, 1, 1, m);   /* partial rotary, table, sections */
        run_case(dtype, 5, 64, 0, layout, 64, 0, 0, m);
        run_case(dtype, 1, 2, 1, layout, 2, 0, 1, m ? 1 : 0);
        run_case(dtype, 0, 128, 1, layout, 128, 0, 0, m);   /* no tokens */
      }

  /* invalid arguments are refused, not read */
  double o[4], s[4];
  float one = 1.0f;
  CHECK(kamera_oracle_segment(0, &one, 1, 1, 1, 1, 0, 0, 1e4, 0, NULL, 0, NULL, 0, o, s) != 0);
  CHECK(kamera_oracle_segment_ex(0, &one, 1, 1, 2, 1, 2, 2, NULL, NULL, 0, 1e4, 0, NULL, 0,
                                 NULL, 0, o, s) != 0);
  CHECK(kamera_oracle_segment(0, &one, 1, 1, 1, 0, 0, 0, 1e4, 1, NULL, 0, NULL, 0, o, s) != 0);

  /* ladder and phases: pair 0 turns by exactly delta radians */
  double f[64], c[64], sn[64];
  kamera_oracle_inv_freq(1e4, 128, f);
  CHECK(f[0] == 1.0 && f[63] < f[1]);
  kamera_oracle_phase(3, 1e4, 128, c, sn);
  CHECK(c[0] == cos(3.0) && sn[0] == sin(3.0));

  /* bf16 rounding: ties to even, NaN stays NaN, infinities and signed zeros kept */
  const double in[7] = {1.0 + 1.0 / 256, 1.0 + 3.0 / 256, NAN, INFINITY, -INFINITY, -0.0, 0.0};
  uint16_t b[7];
  kamera_oracle_to_bf16(in, 7, b);
  CHECK(b[0] == 0x3F80 && b[1] == 0x3F82);
  CHECK((b[2] & 0x7F80) == 0x7F80 && (b[2] & 0x7F) != 0);
  CHECK(b[3] == 0x7F80 && b[4] == 0xFF80 && b[5] == 0x8000 && b[6] == 0x0000);
  float f32[2];
  kamera_oracle_to_f32(in, 2, f32);
  CHECK(f32[0] == (float)in[0]);

  /* slots through a table, and a table overrun refused */
  const int32_t table[3] = {2, 0, 1};
  int64_t sl[40];
  CHECK(kamera_oracle_slots(table, 3, 16, 10, 30, sl) == 0);
  CHECK(sl[0] == 2 * 16 + 10 && sl[6] == 0 * 16 + 0 && sl[29] == 1 * 16 + 7);
  CHECK(kamera_oracle_slots(table, 3, 16, 40, 10, sl) != 0);
  CHECK(kamera_oracle_slots(NULL, 0, 16, 5, 3, sl) == 0 && sl[2] == 7);

  printf("oracle checks: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
