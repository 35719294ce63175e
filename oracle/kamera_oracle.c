/*
 * kamera_oracle.c — plain fp64 CPU oracle of the Kamera reuse operator.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code with the GPU path (no headers, no helpers, no
 * tables) and is deliberately slow: every output element is formed from the definition, in
 * fp64, one term at a time.
 *
 * What it computes (technical summary of "Kamera: Unified Position-Invariant Multimodal KV
 * Cache for Training-Free Reuse", §2 Methodology, reuse equation):
 *
 *     out(t, f) = [R(delta) x](t, f) + sum_{r < m} U(t, r) V(f, r)
 *
 * R(delta) is the RoPE phase shift (same section: exact re-rotation, not a forward pass).
 * Pair i of a rotated head turns by delta * theta^(-2i/width); the rotation is applied first
 * and the patch is added afterwards, unrotated (the equation's order). Unrotated channels
 * (GQA/MHA values, MLA c_KV — "Unified Architecture Support" in §2) pass x through unchanged.
 *
 * Alongside each output the oracle returns S(t, f), the sum of the absolute values of all the
 * terms that make it up; the comparison rules scale their tolerance by it where the result
 * cancels.
 *
 * Inputs are decoded exactly: bf16 -> binary32 -> binary64 and binary32 -> binary64 are exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_HALF_SPLIT = 0, OR_INTERLEAVED = 1 };

static double decode(int dtype, const void* base, int64_t index) {
  if (dtype == OR_F64) return ((const double*)base)[index];
  if (dtype == OR_F32) return (double)((const float*)base)[index];
  /* bf16: the 16 stored bits are the high half of a binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[index] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int kamera_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* theta_i = theta^(-2i/rot_dim), i < rot_dim/2: the standard RoPE frequency ladder. */
void kamera_oracle_inv_freq(double theta, int32_t rot_dim, double* out) {
  for (int32_t i = 0; i < rot_dim / 2; ++i) out[i] = pow(theta, -2.0 * (double)i / (double)rot_dim);
}

/* cos and sin of the angle delta * theta_i of every pair, in fp64. */
void kamera_oracle_phase(int64_t delta, double theta, int32_t rot_dim, double* cos_out,
                         double* sin_out) {
  for (int32_t i = 0; i < rot_dim / 2; ++i) {
    double angle = (double)delta * pow(theta, -2.0 * (double)i / (double)rot_dim);
    cos_out[i] = cos(angle);
    sin_out[i] = sin(angle);
  }
}

/*
 * One head of one chunk, one layer, one channel, with the RoPE variants real backbones use.
 *   src      rows of `width` elements, row t at src + t*src_row_stride (elements, dtype)
 *   rotate   1: turn the pairs of the first rot_dim features; 0: identity
 *   rot_dim  features that carry RoPE (even, <= width); the rest pass through unchanged
 *            (partial rotary, as GPT-NeoX-style models apply it)
 *   inv_freq rot_dim/2 frequencies, or NULL for the ladder theta^(-2i/rot_dim)
 *   pair_delta  the shift of each pair (multimodal sections: each pair turns by the shift of
 *            its position component), or NULL for `delta` on every pair
 *   U        n_tokens x m, row t at U + t*u_row_stride (dtype); V width x m, row f at
 *            V + f*v_row_stride; ignored when m == 0
 *   out, abs_sum   n_tokens x width, dense, fp64
 * Pair i of the rotated block turns by angle pair_delta[i] * inv_freq[i]:
 * (x, y) -> (x cos - y sin, y cos + x sin).
 * Returns 0, or -1 on an invalid argument.
 */
int kamera_oracle_segment_ex(int32_t dtype, const void* src, int64_t src_row_stride,
                             int32_t n_tokens, int32_t width, int32_t rotate, int32_t layout,
                             int32_t rot_dim, const double* inv_freq, const int64_t* pair_delta,
                             int64_t delta, double theta, int32_t m, const void* U,
                             int64_t u_row_stride, const void* V, int64_t v_row_stride,
                             double* out, double* abs_sum) {
  if (n_tokens < 0 || width <= 0 || m < 0) return -1;
  if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_F64) return -1;
  if (rotate && (rot_dim <= 0 || rot_dim % 2 != 0 || rot_dim > width ||
                 (layout != OR_HALF_SPLIT && layout != OR_INTERLEAVED)))
    return -1;
  if (m > 0 && (U == NULL || V == NULL)) return -1;

  const int32_t half = rot_dim / 2;
  double c[1024], s[1024];
  if (rotate) {
    if (half > 1024) return -1;
    for (int32_t i = 0; i < half; ++i) {
      const double inv = inv_freq ? inv_freq[i] : pow(theta, -2.0 * (double)i / (double)rot_dim);
      const double angle = (double)(pair_delta ? pair_delta[i] : delta) * inv;
      c[i] = cos(angle);
      s[i] = sin(angle);
    }
  }

#pragma omp parallel for schedule(static)
  for (int32_t t = 0; t < n_tokens; ++t) {
    for (int32_t f = 0; f < width; ++f) {
      const double x = decode(dtype, src, (int64_t)t * src_row_stride + f);
      double value, mag;
      if (rotate && f < rot_dim) {
        /* pair index i, the partner feature, and whether f is the pair's first element */
        int32_t i, partner, first;
        if (layout == OR_HALF_SPLIT) {
          first = f < half;
          i = first ? f : f - half;
          partner = first ? f + half : f - half;
        } else {
          first = (f % 2) == 0;
          i = f / 2;
          partner = first ? f + 1 : f - 1;
        }
        const double y = decode(dtype, src, (int64_t)t * src_row_stride + partner);
        if (first) {
          value = x * c[i] - y * s[i]; /* x cos - y sin */
        } else {
          value = x * c[i] + y * s[i]; /* y' = y cos + x sin, here x is the second element */
        }
        mag = fabs(x * c[i]) + fabs(y * s[i]);
      } else {
        value = x;
        mag = fabs(x);
      }
      for (int32_t r = 0; r < m; ++r) {
        const double term = decode(dtype, U, (int64_t)t * u_row_stride + r) *
                            decode(dtype, V, (int64_t)f * v_row_stride + r);
        value += term;
        mag += fabs(term);
      }
      out[(int64_t)t * width + f] = value;
      abs_sum[(int64_t)t * width + f] = mag;
    }
  }
  return 0;
}

/* The plain operator: every feature of the head rotates, the theta ladder, one shift. */
int kamera_oracle_segment(int32_t dtype, const void* src, int64_t src_row_stride,
                          int32_t n_tokens, int32_t width, int32_t rotate, int32_t layout,
                          int64_t delta, double theta, int32_t m, const void* U,
                          int64_t u_row_stride, const void* V, int64_t v_row_stride,
                          double* out, double* abs_sum) {
  return kamera_oracle_segment_ex(dtype, src, src_row_stride, n_tokens, width, rotate, layout,
                                  width, NULL, NULL, delta, theta, m, U, u_row_stride, V,
                                  v_row_stride, out, abs_sum);
}

/* fp64 -> binary32, round to nearest even (the C conversion under the default FP mode). */
void kamera_oracle_to_f32(const double* in, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)in[i];
}

/* fp64 -> binary32 (RNE) -> bf16 (RNE on the binary32 bits): the fp32 oracle rounded to bf16.
 * NaN stays NaN (quiet bit set); infinities and signed zeros are kept. */
void kamera_oracle_to_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    float f = (float)in[i];
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) {
      out[i] = (uint16_t)((u >> 16) | 0x0040u);
      continue;
    }
    /* add half an ulp of the kept part, plus one more if the kept part is odd (ties to even) */
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

/* Physical slot of each token of a chunk placed at logical cache token dst_offset:
 * slot(t) = table[p / page_size] * page_size + p % page_size with p = dst_offset + t.
 * table == NULL means the identity table. Returns 0, or -1 if a table index runs past
 * n_table. */
int kamera_oracle_slots(const int32_t* table, int32_t n_table, int32_t page_size,
                        int64_t dst_offset, int32_t n_tokens, int64_t* out) {
  if (page_size <= 0 || n_tokens < 0 || dst_offset < 0) return -1;
  for (int32_t t = 0; t < n_tokens; ++t) {
    int64_t p = dst_offset + t;
    int64_t page = p / page_size;
    if (table != NULL && page >= n_table) return -1;
    int64_t phys = table ? (int64_t)table[page] : page;
    out[t] = phys * page_size + p % page_size;
  }
  return 0;
}
