// kamera_compile.hip — the patch compile of the Kamera reuse operator on gfx950 (CDNA4).
//
// Per chunk, channel, layer and head the deficit is
//     Delta = KV(B|A) - R(delta) KV(B|empty)                      (n_tokens x width)
// (Kamera technical summary: §1 names the deficit a chunk's context leaves in its KV; §2
// Methodology forms the patch once from one conditioned pass over [A, B] and keeps its top-m
// SVD factors). The library takes KV(B|A) and KV(B|empty) and returns
//     V (width x m)     an orthonormal basis of Delta's dominant right singular subspace,
//     U (n_tokens x m)  = Delta V,
// so that U V^T is the rank-m truncation of Delta once the subspace has converged.
//
// Kernels (one launch per class of tile / LDS size present in the batch):
//   gram      partial Gram tiles Delta_s^T Delta_s over token splits s with fp32 MFMA
//             16x16x4 (unrotated bf16 heads of one ordering, the MLA latent: bf16 MFMA
//             16x16x32 on an exact high/low bf16 split of Delta); one tile pair (bi <= bj) of G
//             per block; Delta is formed on the fly (canonical rows rotated in fp32 with cos/sin
//             from fp64, as the reuse kernels do);
//   subspace  one wave per head (widths up to 128) or one block of four waves per head (the
//             wide MLA latent): sums the partials into G where there are several, then block
//             power iteration X <- orth(G X) from a fixed +-1 start, G X on fp32 MFMA. orth() is
//             a Cholesky QR: S = Y^T Y on fp64 MFMA, its Cholesky factor L in fp64, X = Y L^-T,
//             the factorisation and the substitution in 16 x 16 blocks on fp64 MFMA
//             (chol_blocked, subst_blocked). Columns that
//             collapse (Y rank deficient) are re-seeded between rounds
//             and zero after the last; a final orth() of X alone restores orthonormality to
//             fp32 rounding;
//   project   U = Delta X with the fp32 X kept in the workspace (a second pass over the inputs).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "kamera_host.h"
#include "kamera_internal.h"

using namespace kamera::host;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Eight fp32 values as bf16 high parts (round to nearest) and the bf16 of what is left.
__device__ __forceinline__ void split8_bf16(const float* x, bf16x8* hi, bf16x8* lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = bf16_rne(x[2 * e]), h1 = bf16_rne(x[2 * e + 1]);
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = (uint32_t)bf16_rne(x[2 * e] - __uint_as_float((uint32_t)h0 << 16)) |
           ((uint32_t)bf16_rne(x[2 * e + 1] - __uint_as_float((uint32_t)h1 << 16)) << 16);
  }
  *hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  *lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}


// Subspace iteration: Y = G X on fp32 MFMA (1) or fp32 VALU FMA (0).
#ifndef KAMERA_SUBSPACE_MFMA
#define KAMERA_SUBSPACE_MFMA 1
#endif

constexpr int kThreads = 256;
constexpr int kStepTokens = 32;      // tokens of Delta staged in LDS per step
constexpr int kProjTokens = 128;     // tokens per projection block
constexpr int kMinSplitTokens = 1024; // Gram split never shorter than this (except the tail)
constexpr int kGramTilesPerJob = 64;   // jobs with fewer Gram tiles split their tokens
constexpr double kDeadTol = 1e-12;   // pivot^2 / column norm^2 below this: column collapsed

// One ordering of a chunk (an orbit member; a plain compile has one): its conditioned rows of
// one channel and its shifts.
struct alignas(16) CMember {
  const void* cond;
  int64_t cond_ls, cond_ts;
  int64_t delta;    // shift of section 0 (of every pair without sections)
  int64_t delta_s1; // shifts of sections 1 and 2
  int64_t delta_s2;
};

// One chunk, one channel, all layers and heads (a "unit" is one layer and head).
struct alignas(16) CJob {
  const void* canon;
  void* U;
  void* V;
  int64_t canon_ls, canon_ts;
  int64_t u_ls, u_hs, v_ls, v_hs;
  int64_t gpart;   // float offset of the partial Gram tiles [unit][pair][split][te][te]
  int64_t gfull;   // float offset of the assembled G [unit][width][width], or -1 (partial is G)
  int64_t xbase;   // float offset of the fp32 bases [unit][width][mp]
  int32_t n_tokens, m, mp, width, heads, rotate, te, nb, n_pairs, splits, split_tokens, n_units;
  int32_t rot_dim;  // features of each head that turn (the rest pass through); pairs rot_dim/2
  int32_t member_off, n_members;   // this job's orderings in the member table
  int32_t gperm;   // 1: G is stored with its rows and columns permuted (gram_stream_kernel)
  int32_t gsplit;  // 1: G by gram_split_kernel (128-wide bf16 heads, natural order)
  int32_t ptok;    // tokens per block of the streamed projection (a multiple of 16)
};

struct CParams {
  const CJob* jobs;
  const CMember* members;
  const int32_t* starts;   // first block of each entry, ascending
  const int32_t* job_of;   // job index of each entry
  float* ws;               // float view of the workspace's data region
  const double* inv_freq;  // device: frequency table, or NULL (theta ladder)
  const uint8_t* pair_section;  // device: section of each pair, or NULL
  double theta;
  int32_t n_entries;
  int32_t layout;
  int32_t n_iter;
  int32_t n_total;         // units covered by a per-wave launch
};

// ---------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int find_entry(const CParams& P, int b) {
  int lo = 0, hi = P.n_entries - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (P.starts[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// cos/sin(shift * frequency) per pair: angle and reduction in fp64, one rounding. The
// frequency is the table entry when the model gives one, else theta^(-2i/rot_dim); the shift
// is that of the pair's position component (multimodal sections), else the chunk's.
// With several orderings (an orbit) the table holds the mean of their cos and sin: the mean
// of the rotations R(delta_k) acts on each pair as [[cbar, -sbar], [sbar, cbar]].
__device__ __forceinline__ void fill_phases(float2* cs, const CJob& J, const CParams& P) {
  const int rot_dim = J.rot_dim;
  const CMember* mem = P.members + J.member_off;
  for (int i = threadIdx.x; i < rot_dim / 2; i += kThreads) {
    const double inv = P.inv_freq ? P.inv_freq[i]
                                  : pow(P.theta, -2.0 * (double)i / (double)rot_dim);
    const int sec = P.pair_section ? (int)P.pair_section[i] : 0;
    double cbar = 0.0, sbar = 0.0;
    for (int k = 0; k < J.n_members; ++k) {
      const int64_t delta = sec == 0 ? mem[k].delta : (sec == 1 ? mem[k].delta_s1 : mem[k].delta_s2);
      double s, c;
      sincos((double)delta * inv, &s, &c);
      cbar += c;
      sbar += s;
    }
    cs[i] = make_float2((float)(cbar / J.n_members), (float)(sbar / J.n_members));
  }
}

__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(w[k] << 16);
    o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

__device__ __forceinline__ void store_elem(uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);   // RNE
}
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

// Mean over the job's orderings of the conditioned elements [f, f + 8) of one token row (one
// ordering: the row itself, exactly).
template <typename T>
__device__ __forceinline__ void load_cond8(const CMember* mem, int n_members, int layer,
                                           int64_t head_off, int tok, int f, float* o) {
  load8(static_cast<const T*>(mem[0].cond) + layer * mem[0].cond_ls + head_off +
            tok * mem[0].cond_ts + f, o);
  if (n_members == 1) return;
  for (int k = 1; k < n_members; ++k) {
    float x[8];
    load8(static_cast<const T*>(mem[k].cond) + layer * mem[k].cond_ls + head_off +
              tok * mem[k].cond_ts + f, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += x[e];
  }
  const float scale = 1.0f / (float)n_members;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= scale;
}

// Rows [tok0, tok0 + ROWS) of Delta, columns [col0, col0 + ncols), into dst (fp32, row stride
// ds); rows at or past tok_end are zero. A rotated head is always staged whole (col0 = 0,
// ncols = width) so that both members of every pair are at hand; its pairs lie in the first
// rot_dim features, the others pass through. With several orderings Delta is their mean:
// mean conditioned rows minus the mean rotation (cs) applied to the canonical rows.
template <typename T, int ROWS>
__device__ __forceinline__ void stage_delta(const CJob& J, const CParams& P, const float2* cs, int layer,
                            int head, int tok0, int tok_end, int col0, int ncols, float* dst,
                            int ds) {
  const int layout = P.layout;
  const int W = J.width;
  const int64_t head_off = (int64_t)head * W;
  const T* canon = static_cast<const T*>(J.canon) + layer * J.canon_ls + head_off;
  const CMember* mem = P.members + J.member_off;
  const int K = J.n_members;
  if (J.rotate) {
    // groups of 8 pairs over the turning features [0, R), then groups of 8 features passing
    // through over [R, W)
    const int R = J.rot_dim;
    const int gr = R / 16, gpr = gr + (W - R) / 8;
    for (int g = threadIdx.x; g < ROWS * gpr; g += kThreads) {
      const int r = g / gpr, q = g - r * gpr;
      const int tok = tok0 + r;
      float* d = dst + r * ds;
      if (q >= gr) {
        const int f = R + 8 * (q - gr);
        if (tok >= tok_end) {
#pragma unroll
          for (int k = 0; k < 8; ++k) d[f + k] = 0.f;
          continue;
        }
        float x[8], c[8];
        load8(canon + tok * J.canon_ts + f, x);
        load_cond8<T>(mem, K, layer, head_off, tok, f, c);
#pragma unroll
        for (int k = 0; k < 8; ++k) d[f + k] = c[k] - x[k];
        continue;
      }
      const int fa = layout == KAMERA_ROPE_HALF_SPLIT ? 8 * q : 16 * q;
      const int fb = layout == KAMERA_ROPE_HALF_SPLIT ? R / 2 + 8 * q : 16 * q + 8;
      if (tok >= tok_end) {
#pragma unroll
        for (int k = 0; k < 8; ++k) d[fa + k] = d[fb + k] = 0.f;
        continue;
      }
      float xa[8], xb[8], ca[8], cb[8];
      load8(canon + tok * J.canon_ts + fa, xa);
      load8(canon + tok * J.canon_ts + fb, xb);
      load_cond8<T>(mem, K, layer, head_off, tok, fa, ca);
      load_cond8<T>(mem, K, layer, head_off, tok, fb, cb);
      if (layout == KAMERA_ROPE_HALF_SPLIT) {
        // pair 8q+k = (feature fa+k, feature fb+k)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float c = cs[8 * q + k].x, s = cs[8 * q + k].y;
          const float x = xa[k], y = xb[k];
          d[fa + k] = ca[k] - (x * c - y * s);
          d[fb + k] = cb[k] - (y * c + x * s);
        }
      } else {
        // pairs 8q..8q+3 are adjacent features in piece a, 8q+4..8q+7 in piece b
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float c = cs[8 * q + k].x, s = cs[8 * q + k].y;
          const float x = xa[2 * k], y = xa[2 * k + 1];
          d[fa + 2 * k] = ca[2 * k] - (x * c - y * s);
          d[fa + 2 * k + 1] = ca[2 * k + 1] - (y * c + x * s);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float c = cs[8 * q + 4 + k].x, s = cs[8 * q + 4 + k].y;
          const float x = xb[2 * k], y = xb[2 * k + 1];
          d[fb + 2 * k] = cb[2 * k] - (x * c - y * s);
          d[fb + 2 * k + 1] = cb[2 * k + 1] - (y * c + x * s);
        }
      }
    }
  } else {
    const int gpr = ncols / 8;
    for (int g = threadIdx.x; g < ROWS * gpr; g += kThreads) {
      const int r = g / gpr, q = g - r * gpr;
      const int tok = tok0 + r;
      float* d = dst + r * ds + 8 * q;
      if (tok >= tok_end) {
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = 0.f;
        continue;
      }
      float x[8], c[8];
      load8(canon + tok * J.canon_ts + col0 + 8 * q, x);
      load_cond8<T>(mem, K, layer, head_off, tok, col0 + 8 * q, c);
#pragma unroll
      for (int k = 0; k < 8; ++k) d[k] = c[k] - x[k];
    }
  }
}

#define CGLOBAL __attribute__((address_space(1)))

// Eight consecutive features of a row, as loaded (16 bytes per bf16 piece).
template <typename T>
struct Piece {
  u32x4 w[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ void load_piece(const T* p, Piece<T>& o) {
  const CGLOBAL u32x4* q = (const CGLOBAL u32x4*)p;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(T) / 2); ++k) o.w[k] = q[k];
}

__device__ __forceinline__ void piece_floats(const Piece<uint16_t>& a, float* o) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(a.w[0][k] << 16);
    o[2 * k + 1] = __uint_as_float(a.w[0][k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void piece_floats(const Piece<float>& a, float* o) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = __uint_as_float(a.w[0][k]);
    o[4 + k] = __uint_as_float(a.w[1][k]);
  }
}

// Tile pair index -> (bi, bj), bi <= bj, row-major over the upper triangle of nb x nb tiles.
__device__ __forceinline__ void pair_tiles(int pair, int nb, int* bi, int* bj) {
  int p = pair;
  for (int r = 0; r < nb; ++r) {
    const int len = nb - r;
    if (p < len) {
      *bi = r;
      *bj = r + p;
      return;
    }
    p -= len;
  }
  *bi = *bj = 0;
}

// ---------------------------------------------------------------------------------------
// gram: partial G tiles. Tile edge TE = 32*NB; four waves own the 2x2 quadrants of the tile,
// each NB x NB MFMA blocks of 16x16. MFMA 16x16x4 fp32 operands: lane l gives A[l%16][l/16]
// (feature i, token k) and B[l/16][l%16] (token k, feature j); it receives C rows
// 4(l/16)..4(l/16)+3 of column l%16.
// ---------------------------------------------------------------------------------------

// Compiled for 3 waves per SIMD: the bf16 path of NB = 4 then keeps its accumulators and
// operands in 162 VGPRs (the compiler's own choice, 2 waves, was 4.6 % slower on the MLA batch).
template <typename T, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void gram_kernel(CParams P) {
  constexpr int TE = 32 * NB;
  constexpr int DS = TE + 16;   // row stride: the four token rows of an operand fall in
                                // different LDS banks
  __shared__ float di[kStepTokens * DS];
  __shared__ float dj[kStepTokens * DS];
  __shared__ float2 cs[64];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  int local = blockIdx.x - P.starts[e];
  const int split = local % J.splits;
  local /= J.splits;
  const int pair = local % J.n_pairs;
  const int unit = local / J.n_pairs;
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  int bi, bj;
  pair_tiles(pair, J.nb, &bi, &bj);
  if (J.rotate) fill_phases(cs, J, P);

  const int t_lo = split * J.split_tokens;
  const int t_hi = min(J.n_tokens, t_lo + J.split_tokens);
  const float* A = di;
  const float* B = bi == bj ? di : dj;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = (wave >> 1) * (TE / 2), c0 = (wave & 1) * (TE / 2);

  f32x4 acc[NB][NB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_step = [&]() {
#pragma unroll 2
    for (int kk = 0; kk < kStepTokens / 4; ++kk) {
      const int row = (kk * 4 + (lane >> 4)) * DS + (lane & 15);
      float a[NB], b[NB];
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        a[x] = A[row + r0 + 16 * x];
        b[x] = B[row + c0 + 16 * x];
      }
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int y = 0; y < NB; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[y], acc[x][y], 0, 0, 0);
    }
  };

  bool done = false;
  if constexpr (NB == 4) {
    if (!J.rotate && J.n_members == 1) {
      // Unrotated head, one ordering (the MLA latent): Delta = conditioned - canonical needs
      // no phase table, so the next step's rows are loaded into registers while this step's
      // MFMAs run. Thread item k < 2 of a tile: row (tid + 256 k) / 16 of the step, features
      // 8 ((tid + 256 k) % 16) .. + 7 of the tile.
      const int64_t head_off = (int64_t)head * J.width;
      const T* canon = static_cast<const T*>(J.canon) + layer * J.canon_ls + head_off;
      const CMember& m0 = P.members[J.member_off];
      const T* cond = static_cast<const T*>(m0.cond) + layer * m0.cond_ls + head_off;
      const int ntile = bi == bj ? 1 : 2;
      // Row loads are unconditional (a token past the split reads the split's first row, and
      // a diagonal pair loads its one tile twice; both are zeroed or ignored when staged) and
      // the row strides sit in registers: a load under a branch, or a field read through J
      // after a barrier (a memory fence), would make the compiler wait for every load in
      // flight instead of this step's.
      const int64_t canon_ts = J.canon_ts, cond_ts = m0.cond_ts;
      Piece<T> px[2][2], pc[2][2];
      bool pok[2];
      auto load_rows = [&](int tok0) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = threadIdx.x + kThreads * k;
          const int tok = tok0 + (g >> 4);
          pok[k] = tok < t_hi;
          const int64_t tk = pok[k] ? tok : t_lo;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int col = (tt ? bj : bi) * TE + 8 * (g & 15);
            load_piece(canon + tk * canon_ts + col, px[tt][k]);
            load_piece(cond + tk * cond_ts + col, pc[tt][k]);
          }
        }
      };
      if (t_lo < t_hi) load_rows(t_lo);
      if constexpr (sizeof(T) == 2) {
        // bf16 rows: Delta = conditioned - canonical (exact in fp32) is cut into bf16 high and
        // low parts, h = RNE(Delta), l = RNE(Delta - h), and the Gram is summed on
        // v_mfma_f32_16x16x32_bf16 as l l + l h + h l + h h (products exact in fp32, fp32 sums).
        // The difference of two bf16 values needs at most 16 significant bits when their
        // exponents differ by less than 8, and h + l is then Delta exactly; otherwise l is
        // rounded (at most 2^-18 of |Delta|). A 32-token step is one K step. The parts sit in
        // LDS as [token][feature]; an operand (eight tokens of one feature per lane) is two LDS
        // transpose reads (ds_read_b64_tr_b16: lane s of a 16-lane group points at row s / 4,
        // features 4 (s % 4) .. + 3, and lane i receives feature i of the four rows).
        constexpr int RS = TE + 16;   // bf16 row stride of a part
        uint16_t* dih = reinterpret_cast<uint16_t*>(di);
        uint16_t* dil = dih + kStepTokens * RS;
        uint16_t* djh = reinterpret_cast<uint16_t*>(dj);
        uint16_t* djl = djh + kStepTokens * RS;
        const uint16_t* bh = bi == bj ? dih : djh;
        const uint16_t* bl = bi == bj ? dil : djl;
        const int li = lane & 15, kg = lane >> 4;
        const int tro = (8 * kg + (li >> 2)) * RS + 4 * (li & 3);   // this lane's transpose-read offset
        auto operand = [&](const uint16_t* part, int f0) {
          const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(part + tro + f0));
          const s16x4 b =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(part + tro + 4 * RS + f0));
          return __builtin_bit_cast(bf16x8, s16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
        };
        for (int tok0 = t_lo; tok0 < t_hi; tok0 += kStepTokens) {
          __syncthreads();   // the previous step's MFMAs are done with the parts
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              if (tt < ntile) {
                const int g = threadIdx.x + kThreads * k;
                float x[8], c[8], d[8];
                piece_floats(px[tt][k], x);
                piece_floats(pc[tt][k], c);
#pragma unroll
                for (int e = 0; e < 8; ++e) d[e] = pok[k] ? c[e] - x[e] : 0.f;
                bf16x8 h, l;
                split8_bf16(d, &h, &l);
                const int at = (g >> 4) * RS + 8 * (g & 15);
                *reinterpret_cast<bf16x8*>((tt ? djh : dih) + at) = h;
                *reinterpret_cast<bf16x8*>((tt ? djl : dil) + at) = l;
              }
            }
          __syncthreads();
          load_rows(tok0 + kStepTokens);   // past the split: clamped, never staged
          // keep the next rows' loads here, ahead of this step's products (left to itself the
          // compiler moves them to the next step, just before their use)
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 bhv[NB], blv[NB];
#pragma unroll
          for (int y = 0; y < NB; ++y) {
            bhv[y] = operand(bh, c0 + 16 * y);
            blv[y] = operand(bl, c0 + 16 * y);
          }
#pragma unroll
          for (int x = 0; x < NB; ++x) {
            const bf16x8 ah = operand(dih, r0 + 16 * x), al = operand(dil, r0 + 16 * x);
#pragma unroll
            for (int y = 0; y < NB; ++y) {
              acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, blv[y], acc[x][y], 0, 0, 0);
              acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bhv[y], acc[x][y], 0, 0, 0);
              acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, blv[y], acc[x][y], 0, 0, 0);
              acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bhv[y], acc[x][y], 0, 0, 0);
            }
          }
        }
      } else {
        for (int tok0 = t_lo; tok0 < t_hi; tok0 += kStepTokens) {
          __syncthreads();   // the previous step's MFMAs are done with di / dj
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              if (tt < ntile) {
                const int g = threadIdx.x + kThreads * k;
                float x[8], c[8];
                piece_floats(px[tt][k], x);
                piece_floats(pc[tt][k], c);
                float* d = (tt ? dj : di) + (g >> 4) * DS + 8 * (g & 15);
#pragma unroll
                for (int e = 0; e < 8; ++e) d[e] = pok[k] ? c[e] - x[e] : 0.f;
              }
            }
          __syncthreads();
          load_rows(tok0 + kStepTokens);   // past the split: clamped, never staged
          mfma_step();
        }
      }
      done = true;
    }
  }
  if (!done) {
    for (int tok0 = t_lo; tok0 < t_hi; tok0 += kStepTokens) {
      __syncthreads();
      stage_delta<T, kStepTokens>(J, P, cs, layer, head, tok0, t_hi, bi * TE, TE, di, DS);
      if (bi != bj)
        stage_delta<T, kStepTokens>(J, P, cs, layer, head, tok0, t_hi, bj * TE, TE, dj, DS);
      __syncthreads();
      mfma_step();
    }
  }

  float* out = P.ws + J.gpart +
               ((int64_t)(unit * J.n_pairs + pair) * J.splits + split) * (TE * TE);
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(r0 + 16 * x + 4 * (lane >> 4) + i) * TE + c0 + 16 * y + (lane & 15)] = acc[x][y][i];
}

// Piece (8 features) held by lane group g in slot p of slab c.
__host__ __device__ inline int stream_piece(int g, int p, int c, int S, int unit_layout, int hp) {
  if (!unit_layout) return 16 * c + 4 * p + g;
  const int pos = g * S + p;
  if (pos < 2 * hp) return (pos & 1) ? hp + (pos >> 1) : (pos >> 1);
  return pos;
}

// LDS row stride (floats) of the permuted X: the four rows one MFMA step reads (16 floats
// each) land in distinct banks; wider heads take the plain stride to bound the LDS.
__host__ __device__ inline int stream_sv(int width, int mp) {
  if (width > 128) return mp;
  return mp == 16 ? 16 : (mp == 64 ? 80 : 48);
}

// ---------------------------------------------------------------------------------------
// gram_stream: G = Delta^T Delta for 128-wide heads with Delta formed in registers.
// The sum runs over tokens in any order and G may be stored in any symmetric permutation, so
// each lane multiplies what it loaded itself: at step s lane 16g + n holds token
// t + 4s + g, features 8n .. 8n + 7 (the 16 lanes of a group read one whole 256-byte row).
// Stored order: row 16b + i of G' is feature 8i + b, so element b of every lane's piece is
// the MFMA operand of 16-feature block b (A[i][k] = Delta[token k][8i + b] and
// B[k][j] = Delta[token k][8j + b']), and one v_mfma_f32_16x16x4f32 per block pair
// b <= b' (36 of 64: G is symmetric) adds four tokens. Half-split RoPE partners sit R/16
// lanes apart in the group and are fetched with a lane permute. The four waves take
// contiguous quarters of the block's tokens and their partial sums are added in LDS in wave
// order, so the result does not depend on timing.
// ---------------------------------------------------------------------------------------

constexpr int kGramPrefetch = 4;   // steps of 4 tokens kept in flight per wave

__host__ __device__ inline int gperm_row(int f) { return 16 * (f & 7) + (f >> 3); }

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 8)))
void gram_stream_kernel(CParams P) {
  __shared__ float red[36 * 256];
  __shared__ float2 cs[64];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  int local = blockIdx.x - P.starts[e];
  const int split = local % J.splits;
  const int unit = local / J.splits;
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int t_lo = split * J.split_tokens;
  const int t_hi = min(J.n_tokens, t_lo + J.split_tokens);
  // this wave's quarter of the tokens, in steps of 4
  const int q4 = ((t_hi - t_lo + 15) / 16) * 4;
  const int w_lo = t_lo + wave * q4, w_hi = min(t_hi, w_lo + q4);
  const int nsteps = w_hi > w_lo ? (w_hi - w_lo + 3) / 4 : 0;

  // this lane's piece of the row: features 8n .. 8n + 7; its RoPE role
  const int R = J.rotate ? J.rot_dim : 0;
  const bool inter = P.layout != KAMERA_ROPE_HALF_SPLIT;
  const int hp = R / 16;
  int kind = 0, pair0 = 0, src_lane = lane;
  if (J.rotate && n < R / 8) {
    if (inter) {
      kind = 3;
      pair0 = 4 * n;
    } else if (n < hp) {
      kind = 1;
      pair0 = 8 * n;
      src_lane = (lane & ~15) | (n + hp);
    } else {
      kind = 2;
      pair0 = 8 * (n - hp);
      src_lane = (lane & ~15) | (n - hp);
    }
  }

  const CMember* mem = P.members + J.member_off;
  const int K = J.n_members;
  const int64_t head_off = (int64_t)head * 128;
  const T* canon = static_cast<const T*>(J.canon) + layer * J.canon_ls + head_off + 8 * n;
  const T* cond0 = static_cast<const T*>(mem[0].cond) + layer * mem[0].cond_ls + head_off + 8 * n;

  Piece<T> px[kGramPrefetch], pc[kGramPrefetch];
  auto load_step = [&](int st, Piece<T>& x, Piece<T>& c) {
    const int tok = w_lo + 4 * st + g;
    if (st < nsteps && tok < w_hi) {
      load_piece(canon + (int64_t)tok * J.canon_ts, x);
      load_piece(cond0 + (int64_t)tok * mem[0].cond_ts, c);
    } else {
#pragma unroll
      for (int k = 0; k < (int)(sizeof(T) / 2); ++k) {
        x.w[k] = u32x4{0u, 0u, 0u, 0u};
        c.w[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
#pragma unroll
  for (int k = 0; k < kGramPrefetch; ++k) load_step(k, px[k], pc[k]);
  // the phase table after the first loads, so their latency overlaps it
  if (J.rotate) {
    fill_phases(cs, J, P);
    __syncthreads();
  }

  f32x4 acc[36];
#pragma unroll
  for (int k = 0; k < 36; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float inv_k = 1.0f / (float)K;

  for (int st0 = 0; st0 < nsteps; st0 += kGramPrefetch) {
#pragma unroll
    for (int k = 0; k < kGramPrefetch; ++k) {
      const int st = st0 + k;
      if (st >= nsteps) break;
      // the partner piece (half-split pairs), then this step's slot refilled
      Piece<T> py;
#pragma unroll
      for (int w = 0; w < (int)(sizeof(T) / 2); ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          py.w[w][q] = (uint32_t)__shfl((int)px[k].w[w][q], src_lane);
      float x[8], y[8], d[8];
      piece_floats(px[k], x);
      piece_floats(py, y);
      piece_floats(pc[k], d);
      const int tok = w_lo + 4 * st + g;
      load_step(st + kGramPrefetch, px[k], pc[k]);
      if (K > 1) {
        if (tok < w_hi) {
          for (int mk = 1; mk < K; ++mk) {
            Piece<T> pm;
            load_piece(static_cast<const T*>(mem[mk].cond) + layer * mem[mk].cond_ls + head_off +
                           8 * n + (int64_t)tok * mem[mk].cond_ts, pm);
            float z[8];
            piece_floats(pm, z);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += z[q];
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] *= inv_k;
      }
      if (kind == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = d[q] - x[q];
      } else if (kind == 3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 r = cs[pair0 + j];
          const float a = x[2 * j], b = x[2 * j + 1];
          d[2 * j] = d[2 * j] - (a * r.x - b * r.y);
          d[2 * j + 1] = d[2 * j + 1] - (b * r.x + a * r.y);
        }
      } else {
        const float sg = kind == 1 ? -1.f : 1.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float2 r = cs[pair0 + q];
          d[q] = d[q] - (x[q] * r.x + (sg * y[q]) * r.y);
        }
      }
      int blk = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int b2 = b; b2 < 8; ++b2) {
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x4f32(d[b], d[b2], acc[blk], 0, 0, 0);
          ++blk;
        }
    }
  }

  // partial sums of the four waves, added in wave order
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int k = 0; k < 36; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = red + k * 256 + (4 * g + r) * 16 + n;
          *dst = w == 0 ? acc[k][r] : *dst + acc[k][r];
        }
    }
    __syncthreads();
  }
  // G' (permuted order) to the workspace, both triangles
  float* gout = P.ws + J.gpart + ((int64_t)unit * J.splits + split) * (128 * 128);
  int blk = 0;
  for (int b = 0; b < 8; ++b)
    for (int b2 = b; b2 < 8; ++b2, ++blk) {
      const float* src = red + blk * 256;
      const int i = tid >> 4, j = tid & 15;
      gout[(16 * b + i) * 128 + 16 * b2 + j] = src[i * 16 + j];
      if (b2 != b) gout[(16 * b2 + i) * 128 + 16 * b + j] = src[j * 16 + i];
    }
}

// ---------------------------------------------------------------------------------------
// gram_split_kernel: the Gram of 128-wide bf16 heads on bf16 MFMA. Delta (fp32, formed as
// stage_delta forms it) is cut into bf16 high and low parts by round to nearest, h = RNE(Delta),
// l = RNE(Delta - h) (the subtraction is exact), and each 16 x 16 block pair (a <= b) of G sums
// l l, l h, h l, h h on v_mfma_f32_16x16x32_bf16 (products exact in fp32, fp32 sums). For an
// unrotated head of one ordering Delta is the difference of two bf16 values, and h + l is
// Delta exactly unless their exponents differ by 8 or more; otherwise (and for rotated heads,
// whose Delta has 24 significant bits) l is rounded, by at most 2^-18 of |Delta|, an error that
// varies in sign from token to token and so mostly cancels in the sum over tokens (a third part
// made the products exact to fp32 but the whole compile 4 % slower). A step stages 32 tokens of
// the parts in LDS as [token][feature] (a thread forms 16 features of one token: both members
// of its RoPE pairs, or 16 features passing through) and is one K step; wave w takes the 9
// block pairs (w, w..7) and (7 - w, 7 - w..7), its operands (eight tokens of one feature per
// lane) by LDS transpose reads (ds_read_b64_tr_b16). Rows are loaded two steps ahead (three
// register buffers in rotation, so no register copy waits for a load). G is written in natural
// feature order, both triangles, exactly symmetric (gperm = 0).
// ---------------------------------------------------------------------------------------

constexpr int kSplitStep = 32;   // tokens per step: one K step of the bf16 MFMA

// MULTI: several orderings (their conditioned rows are averaged); a separate instantiation, so
// that the plain one has no load under a branch in its step loop.
template <typename T, bool MULTI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void gram_split_kernel(CParams P) {
  static_assert(sizeof(T) == 2, "bf16 rows");
  constexpr int RS = 128 + 16;   // bf16 row stride of a part
  __shared__ __align__(16) uint16_t parts[2][kSplitStep * RS];
  __shared__ float2 cs[64];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  const int local = blockIdx.x - P.starts[e];
  const int split = local % J.splits;
  const int unit = local / J.splits;
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t_lo = split * J.split_tokens;
  const int t_hi = min(J.n_tokens, t_lo + J.split_tokens);
  const int nsteps = t_hi > t_lo ? (t_hi - t_lo + kSplitStep - 1) / kSplitStep : 0;

  // this thread's item of a step: token row r, feature group q (features fa..fa+7, fb..fb+7)
  const int r = tid >> 3, q = tid & 7;
  const int R = J.rotate ? J.rot_dim : 0;   // a multiple of 16 (host)
  const bool half = P.layout == KAMERA_ROPE_HALF_SPLIT;
  const int gr = R / 16;
  const bool turn = q < gr;
  const int fa = turn ? (half ? 8 * q : 16 * q) : R + 16 * (q - gr);
  const int fb = turn ? (half ? R / 2 + 8 * q : 16 * q + 8) : fa + 8;
  const CMember* mem = P.members + J.member_off;
  const int K = J.n_members;
  const int64_t head_off = (int64_t)head * 128;
  const T* canon = static_cast<const T*>(J.canon) + layer * J.canon_ls + head_off;
  const T* cond0 = static_cast<const T*>(mem[0].cond) + layer * mem[0].cond_ls + head_off;
  // row strides in registers: a barrier is a memory fence, after which fields read through J
  // would be loaded again (and a load's wait would also wait for the rows in flight)
  const int64_t canon_ts = J.canon_ts, cond_ts = mem[0].cond_ts;

  // The row loads are issued unconditionally (a token past the split reads the split's first
  // row and is zeroed when staged): the compiler can then wait for one buffer's loads with a
  // partial count, where a load under a branch makes it wait for every load in flight.
  struct Rows {
    Piece<T> xa, xb, ca, cb;
    bool ok;
  };
  auto load_rows = [&](int st, Rows& b) {
    const int tok0 = t_lo + kSplitStep * st + r;
    b.ok = st < nsteps && tok0 < t_hi;
    const int64_t tok = b.ok ? tok0 : t_lo;
    load_piece(canon + tok * canon_ts + fa, b.xa);
    load_piece(canon + tok * canon_ts + fb, b.xb);
    load_piece(cond0 + tok * cond_ts + fa, b.ca);
    load_piece(cond0 + tok * cond_ts + fb, b.cb);
  };
  auto stage = [&](int st, const Rows& b) {
    const int tok = t_lo + kSplitStep * st + r;
    float xa[8], xb[8], da[8], db[8];
    piece_floats(b.xa, xa);
    piece_floats(b.xb, xb);
    piece_floats(b.ca, da);
    piece_floats(b.cb, db);
    if (!b.ok) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xa[i] = xb[i] = da[i] = db[i] = 0.f;
    }
    if (MULTI && b.ok) {
      // several orderings: the mean of their conditioned rows
      for (int k = 1; k < K; ++k) {
        const T* ck = static_cast<const T*>(mem[k].cond) + layer * mem[k].cond_ls + head_off +
                      (int64_t)tok * mem[k].cond_ts;
        float ya[8], yb[8];
        load8(ck + fa, ya);
        load8(ck + fb, yb);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          da[i] += ya[i];
          db[i] += yb[i];
        }
      }
      const float inv_k = 1.0f / (float)K;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        da[i] *= inv_k;
        db[i] *= inv_k;
      }
    }
    if (!turn) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        da[i] = da[i] - xa[i];
        db[i] = db[i] - xb[i];
      }
    } else if (half) {
      // pair 8 q + i = (feature fa + i, feature fb + i)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float c = cs[8 * q + i].x, sn = cs[8 * q + i].y;
        const float x = xa[i], y = xb[i];
        da[i] = da[i] - (x * c - y * sn);
        db[i] = db[i] - (y * c + x * sn);
      }
    } else {
      // pairs 8 q .. 8 q + 3 are adjacent features of piece a, 8 q + 4 .. 8 q + 7 of piece b
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = cs[8 * q + i].x, sn = cs[8 * q + i].y;
        const float x = xa[2 * i], y = xa[2 * i + 1];
        da[2 * i] = da[2 * i] - (x * c - y * sn);
        da[2 * i + 1] = da[2 * i + 1] - (y * c + x * sn);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = cs[8 * q + 4 + i].x, sn = cs[8 * q + 4 + i].y;
        const float x = xb[2 * i], y = xb[2 * i + 1];
        db[2 * i] = db[2 * i] - (x * c - y * sn);
        db[2 * i + 1] = db[2 * i + 1] - (y * c + x * sn);
      }
    }
    bf16x8 h, l;
    split8_bf16(da, &h, &l);
    *reinterpret_cast<bf16x8*>(parts[0] + r * RS + fa) = h;
    *reinterpret_cast<bf16x8*>(parts[1] + r * RS + fa) = l;
    split8_bf16(db, &h, &l);
    *reinterpret_cast<bf16x8*>(parts[0] + r * RS + fb) = h;
    *reinterpret_cast<bf16x8*>(parts[1] + r * RS + fb) = l;
  };

  const int li = lane & 15, kg = lane >> 4;
  const int tro = (8 * kg + (li >> 2)) * RS + 4 * (li & 3);   // transpose-read offset
  auto operand = [&](int p, int blk) {
    const uint16_t* src = parts[p] + tro + 16 * blk;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 4 * RS));
    return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  const int first = 8 - wave;   // slots of row block `wave`; the rest are row block 7 - wave
  f32x4 acc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto products = [&]() {
    bf16x8 ah, al;
#pragma unroll
    for (int sl = 0; sl < 9; ++sl) {
      const int a = sl < first ? wave : 7 - wave;
      const int b = sl < first ? wave + sl : 7 - wave + (sl - first);
      if (sl == 0 || sl == first) {
        ah = operand(0, a);
        al = operand(1, a);
      }
      const bf16x8 bh = operand(0, b), bl = operand(1, b);
      acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bl, acc[sl], 0, 0, 0);
      acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[sl], 0, 0, 0);
      acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[sl], 0, 0, 0);
      acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[sl], 0, 0, 0);
    }
  };

  if (nsteps == 0) {   // an empty split (no rows to read): its partial G is zero
    float* gz = P.ws + J.gpart + ((int64_t)unit * J.splits + split) * (128 * 128);
    for (int i = tid; i < 128 * 128; i += kThreads) gz[i] = 0.f;
    return;
  }
  Rows b0, b1, b2;
  load_rows(0, b0);
  load_rows(1, b1);
  // the phase table after the first loads, so their latency overlaps it (the first step's
  // barrier publishes it)
  if (J.rotate) fill_phases(cs, J, P);
  auto step = [&](int st, const Rows& cur, Rows& ahead) {
    __syncthreads();   // the previous step's products are done with the parts
    stage(st, cur);
    __syncthreads();
    load_rows(st + 2, ahead);   // into the buffer staged one step ago
    products();
  };
  // whole rounds of three steps (steps past the split stage zeros): no branch in the loop
  for (int st = 0; st < nsteps; st += 3) {
    step(st, b0, b2);
    step(st + 1, b1, b0);
    step(st + 2, b2, b1);
  }

  // both triangles of each block pair, mirrored so that G is exactly symmetric
  float* gout = P.ws + J.gpart + ((int64_t)unit * J.splits + split) * (128 * 128);
#pragma unroll
  for (int sl = 0; sl < 9; ++sl) {
    const int a = sl < first ? wave : 7 - wave;
    const int b = sl < first ? wave + sl : 7 - wave + (sl - first);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * a + 4 * kg + v, col = 16 * b + li;
      if (a != b || row >= col) {
        gout[row * 128 + col] = acc[sl][v];
        gout[col * 128 + row] = acc[sl][v];
      }
    }
  }
}

// Shared by both subspace kernels: the fixed +-1 start, the storage of S and L, and the
// Cholesky factorisation.

__device__ __forceinline__ float seed_value(int i, int j, int round) {
  uint32_t h = (uint32_t)i * 0x9E3779B1u ^ ((uint32_t)j + 0x7F4A7C15u) * 0x85EBCA77u ^
               (uint32_t)round * 0xC2B2AE3Du;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  return (h & 1u) ? 1.f : -1.f;
}

// Storage of S and L (lower triangle, fp64) for one unit of rank class MP, packed by columns
// (lcol).
template <int MP>
__host__ __device__ constexpr int lm_size() { return MP * (MP + 1) / 2; }

// ---------------------------------------------------------------------------------------
// subspace (wide heads, 256 .. 512 features: the MLA latent): one block of 4 waves per unit.
// LDS: xs [D][MMAX+1] fp32, holding X, then Y = G X, then X = orth(Y) (odd row stride), ss
// fp64 S and then L (packed lower): 76 KB for the 512-wide latent at rank 32, so two blocks
// share a CU.
//   Y = G X    fp32 MFMA 16x16x4, wave w takes row blocks w, w + 4, ... (G read from the
//              workspace, 16 bytes of a row per lane per K block, next block in flight); Y
//              stays in the accumulators until every wave has read X, then replaces it;
//   X = orth(Y) orth_wide: S = Y^T Y, the blocked Cholesky and the blocked substitution, all
//              on fp64 MFMA.
// ---------------------------------------------------------------------------------------

template <int DMAX, int MMAX>
__device__ void gx_mfma_block(const float* G, float* xs_generic, int D, int mp) {
  // X lives in LDS: said explicitly, since the compiler may keep this function out of line
  // (inlining it costs the 512-wide rank-16 kernel its registers), where a generic pointer
  // would make every access a FLAT one
  __attribute__((address_space(3))) float* xs = (__attribute__((address_space(3))) float*)xs_generic;
  constexpr int NCB = MMAX / 16;
  constexpr int NS = DMAX / 64;   // row blocks per wave (D / 16 of them over 4 waves)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, kk = lane >> 4;
  const int nrb = D / 16;
  const int nt = D / 16;
  const int XS = mp + 1;
  f32x4 acc[NS][NCB];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[s][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A = G[16 rb + i][kappa], kappa = 16 t + 4 kk + u; B = X[kappa][16 cb + i]
  const float* grow = G + (int64_t)li * D + 4 * kk;
  f32x4 ga[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rb = wave + 4 * s;
    ga[s] = rb < nrb ? ((const CGLOBAL f32x4*)(grow + (int64_t)16 * rb * D))[0]
                     : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int t = 0; t < nt; ++t) {
    const int tn = t + 1 < nt ? t + 1 : t;   // past the end: reload (unused)
    float bv[4][NCB];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        bv[u][cb] = 16 * cb < mp ? xs[(16 * t + 4 * kk + u) * XS + 16 * cb + li] : 0.f;
    // consecutive MFMAs go to different accumulators (row blocks), so none waits on the last
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (wave + 4 * s < nrb)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[s][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[s][u], bv[u][cb], acc[s][cb], 0, 0, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int rb = wave + 4 * s;
      if (rb < nrb) ga[s] = ((const CGLOBAL f32x4*)(grow + (int64_t)16 * rb * D + 16 * tn))[0];
    }
  }
  __syncthreads();   // every wave has read X: Y replaces it
  // lane 16 kk + i holds rows 16 rb + 4 kk + v, columns 16 cb + i
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rb = wave + 4 * s;
    if (rb < nrb) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        if (16 * cb < mp)
#pragma unroll
          for (int v = 0; v < 4; ++v) xs[(16 * rb + 4 * kk + v) * XS + 16 * cb + li] = acc[s][cb][v];
    }
  }
}

template <int MP>
__device__ __forceinline__ int lcol(int r, int c) { return c * MP - c * (c - 1) / 2 + (r - c); }

__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// L L^T = S by 16 x 16 block columns, by one whole wave: lm holds S (lower, lcol layout) on
// entry and L on exit, with each diagonal block holding T_KK = L_KK^-1 instead of L_KK; inv
// and dead as in the unblocked form (a collapsed column gets 1 / l_jj = 0).
template <int MP>
__device__ __forceinline__ void chol_blocked(double* lm, double* inv, int* dead, int m) {
  static_assert(MP % 16 == 0 && MP <= 64, "16-column blocks, rank classes up to 64");
  constexpr int NB = MP / 16;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, kk = lane >> 4;
  if (lane < MP) inv[lane] = lm[lcol<MP>(lane, lane)];   // starting diagonal (dead-column test)
  wave_lds_sync();

  // L L^T = S by block columns; diagonal blocks end up holding T_KK = L_KK^-1
#pragma unroll
  for (int K = 0; K < NB; ++K) {
    const int g0 = 16 * K;
    double sv[16], s0[16], tv[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      sv[c] = li >= c ? lm[lcol<MP>(g0 + li, g0 + c)] : lm[lcol<MP>(g0 + c, g0 + li)];
      s0[c] = inv[g0 + c];
      tv[c] = c == li ? 1.0 : 0.0;   // column li of T, solved right-looking
    }
    // step j: lane i's sv[0] is entry (i, j) of what is left of the block (its row shifts by
    // one column per step, so every index is static); the steps have no branch, so one step's
    // updates can overlap the next pivot's square root and reciprocal
    uint32_t dbits = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double d = readlane_f64(sv[0], j);
      const bool real = g0 + j < m;
      const bool dk = real && d <= kDeadTol * s0[j];
      const bool live = real && !dk;
      // 1 / sqrt(d): the hardware estimate and two Newton steps (a shorter dependent chain
      // than a correctly rounded square root followed by a division)
      double rq = __builtin_amdgcn_rsq(d);
      rq = __builtin_fma(0.5 * rq, __builtin_fma(-d * rq, rq, 1.0), rq);
      rq = __builtin_fma(0.5 * rq, __builtin_fma(-d * rq, rq, 1.0), rq);
      const double iv = live ? rq : 0.0;
      dbits |= dk ? 1u << j : 0u;
      const double lij = li > j ? sv[0] * iv : 0.0;
      const double tj = tv[j] * iv;
      tv[j] = tj;
#pragma unroll
      for (int c = 1; c < 16 - j; ++c) {
        const double lc = readlane_f64(lij, j + c);   // L[j + c][j]
        sv[c - 1] = __builtin_fma(-lij, lc, sv[c]);
        tv[j + c] = __builtin_fma(-lc, tj, tv[j + c]);
      }
    }
    if (lane < 16) dead[g0 + lane] = (dbits >> lane) & 1u;
    wave_lds_sync();   // every lane has read the diagonal block
    if (kk == 0) {
#pragma unroll
      for (int n = 0; n < 16; ++n)
        if (n >= li) lm[lcol<MP>(g0 + n, g0 + li)] = tv[n];
    }
    wave_lds_sync();
    if (K + 1 < NB) {
      // panel: L_IK = S_IK T_KK^T (B operand: T[li][4 s + kk])
      double bt[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int cc = 4 * s2 + kk;
        bt[s2] = li >= cc ? lm[lcol<MP>(g0 + li, g0 + cc)] : 0.0;
      }
#pragma unroll
      for (int I = K + 1; I < NB; ++I) {
        double a[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) a[s2] = lm[lcol<MP>(16 * I + li, g0 + 4 * s2 + kk)];
        f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) acc = mfma_f64(a[s2], bt[s2], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) lm[lcol<MP>(16 * I + kk + 4 * v, g0 + li)] = acc[v];
      }
      wave_lds_sync();
      // trailing update: S_IJ -= L_IK L_JK^T for K < J <= I
#pragma unroll
      for (int J = K + 1; J < NB; ++J) {
        double b[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) b[s2] = lm[lcol<MP>(16 * J + li, g0 + 4 * s2 + kk)];
#pragma unroll
        for (int I = J; I < NB; ++I) {
          f64x4 acc;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * I + kk + 4 * v, col = 16 * J + li;
            acc[v] = row >= col ? lm[lcol<MP>(row, col)] : 0.0;
          }
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            acc = mfma_f64(-lm[lcol<MP>(16 * I + li, g0 + 4 * s2 + kk)], b[s2], acc);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = 16 * I + kk + 4 * v, col = 16 * J + li;
            if (row >= col) lm[lcol<MP>(row, col)] = acc[v];
          }
        }
      }
      wave_lds_sync();
    }
  }

}

// X = Y L^-T in place for the 16-row tiles rt_first, rt_first + 1, rt_first + rt_step, ... below
// rt_end (rows of bs floats in buf), by one whole wave, from chol_blocked's factor: per block
// column J, Z^T = Y_J^T - L_J,<J X_<J^T, then X_J = Z T_JJ^T, two row tiles at a time.
template <int MP>
__device__ __forceinline__ void subst_blocked(float* buf, int bs, const double* lm, const int* dead,
                                              int m, int rt_first, int rt_end, int rt_step,
                                              int reseed_round) {
  constexpr int NB = MP / 16;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, kk = lane >> 4;
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    double la[NB > 1 ? 4 * (NB - 1) : 1];   // -L[16 J + li][4 q + kk], q < 4 J
#pragma unroll
    for (int q = 0; q < 4 * J; ++q) la[q] = -lm[lcol<MP>(16 * J + li, 4 * q + kk)];
    double bt[4];               // T_JJ[li][4 s + kk]
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int cc = 4 * s2 + kk;
      bt[s2] = li >= cc ? lm[lcol<MP>(16 * J + li, 16 * J + cc)] : 0.0;
    }
    const int col = 16 * J + li;   // the output column of this lane
    const bool reseed = reseed_round >= 0 && col < m && dead[col] != 0;
    for (int rt = rt_first; rt < rt_end; rt += rt_step) {
      f64x4 z[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* yrow = buf + (16 * (rt + h) + li) * bs;
#pragma unroll
        for (int v = 0; v < 4; ++v) z[h][v] = (double)yrow[16 * J + kk + 4 * v];
      }
#pragma unroll
      for (int q = 0; q < 4 * J; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          z[h] = mfma_f64(la[q], (double)buf[(16 * (rt + h) + li) * bs + 4 * q + kk], z[h]);
      // lane 16 kk + li holds Z[16 rt + li][16 J + kk + 4 v] in register v: A[li][4 v + kk]
      f64x4 x[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int h = 0; h < 2; ++h) x[h] = mfma_f64(z[h][s2], bt[s2], x[h]);
      // lane 16 kk + li holds X[16 rt + kk + 4 v][16 J + li]
      if (col < m) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = 16 * (rt + h) + kk + 4 * v;
            buf[r * bs + col] = reseed ? seed_value(r, col, reseed_round + 1) : (float)x[h][v];
          }
      }
    }
    wave_lds_sync();
  }
}

// X = orth(Y) for the wide heads (Cholesky QR, fp64) in 16 x 16 blocks, X in LDS in rows of
// MP + 1 floats: S = Y^T Y on fp64 MFMA over all D rows (fp32 products exact in fp64, fp64
// sums; the lower tiles dealt to the waves) into the packed layout, the blocked Cholesky by
// wave 0 (chol_blocked), and X = Y L^-T on fp64 MFMA by all four waves (subst_blocked), wave w
// taking the row-tile pairs 2 w, 2 w + 8, ... . Collapsed columns give x_j = 0, or a fresh
// +-1 column when reseed_round >= 0 (the next round's G X spreads it). Replaces a form with
// the factorisation on one wave's scalar registers and the substitution one row per thread:
// MLA latent compile 18.3 -> 16.2 ms.
template <int MP>
__device__ __forceinline__ void orth_wide(float* xs, double* lm, double* inv, int* dead, int D,
                                          int m, int reseed_round) {
  static_assert(MP == 16 || MP == 32, "wide heads take ranks up to 32");
  constexpr int XS = MP + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    const int li = lane & 15, kk = lane >> 4;
    constexpr int nt = MP / 16;
    constexpr int ntiles = nt * (nt + 1) / 2;
    for (int q = wave; q < ntiles; q += kThreads / 64) {
      int ta = 0;
      while ((ta + 1) * (ta + 2) / 2 <= q) ++ta;
      const int tb = q - ta * (ta + 1) / 2;
      const float* ya = xs + kk * XS + 16 * ta + li;
      const float* yb = xs + kk * XS + 16 * tb + li;
      f64x4 sa[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) sa[c] = f64x4{0.0, 0.0, 0.0, 0.0};
      for (int r = 0; r < D; r += 16) {   // D is a multiple of 128
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sa[c] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)ya[(r + 4 * c) * XS],
                                                       (double)yb[(r + 4 * c) * XS], sa[c], 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * ta + kk + 4 * v, col = 16 * tb + li;
        if (col <= row) lm[lcol<MP>(row, col)] = (sa[0][v] + sa[1][v]) + (sa[2][v] + sa[3][v]);
      }
    }
  }
  __syncthreads();
  if (wave == 0) chol_blocked<MP>(lm, inv, dead, m);
  __syncthreads();
  subst_blocked<MP>(xs, XS, lm, dead, m, 2 * wave, D / 16, 8, reseed_round);
  __syncthreads();
}

template <typename T, int DMAX, int MMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void subspace_kernel(CParams P) {
  __shared__ __align__(16) float xs[DMAX * (MMAX + 1)];
  __shared__ double ss[MMAX * (MMAX + 1)];
  __shared__ double inv[MMAX];
  __shared__ int dead[MMAX];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  const int unit = blockIdx.x - P.starts[e];
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int D = J.width, m = J.m, mp = J.mp, tid = threadIdx.x;
  // X rows in LDS are MMAX + 1 floats whatever mp is (columns from m on stay zero)
  constexpr int XS = MMAX + 1;

  // G: the single partial, or the sum of the partial tiles assembled in the workspace
  const float* G;
  if (J.gfull < 0) {
    G = P.ws + J.gpart + (int64_t)unit * D * D;
  } else {
    float* gf = P.ws + J.gfull + (int64_t)unit * D * D;
    const int te = J.te, te2 = te * te;
    for (int pair = 0; pair < J.n_pairs; ++pair) {
      int bi, bj;
      pair_tiles(pair, J.nb, &bi, &bj);
      const float* part = P.ws + J.gpart + (int64_t)(unit * J.n_pairs + pair) * J.splits * te2;
      const float4* part4 = reinterpret_cast<const float4*>(part);
#pragma unroll 4
      for (int i4 = tid; i4 < te2 / 4; i4 += kThreads) {
        float4 v = part4[i4];
#pragma unroll 4
        for (int s = 1; s < J.splits; ++s) {
          const float4 w = part4[(int64_t)s * (te2 / 4) + i4];
          v.x += w.x;
          v.y += w.y;
          v.z += w.z;
          v.w += w.w;
        }
        const int ii = (4 * i4) / te, jj = 4 * i4 - ii * te;
        *reinterpret_cast<float4*>(gf + (bi * te + ii) * D + bj * te + jj) = v;
        if (bi != bj) {
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) gf[(bj * te + jj + c) * D + bi * te + ii] = vv[c];
        }
      }
    }
    __syncthreads();
    G = gf;
  }

  for (int idx = tid; idx < D * MMAX; idx += kThreads) {
    const int i = idx / MMAX, j = idx - i * MMAX;
    xs[i * XS + j] = j < m ? seed_value(i, j, 0) : 0.f;
  }
  __syncthreads();

  for (int round = 0; round < P.n_iter; ++round) {
    gx_mfma_block<DMAX, MMAX>(G, xs, D, MMAX);
    __syncthreads();
    orth_wide<MMAX>(xs, ss, inv, dead, D, m, round);
  }
  // last pass on X alone: orthonormal to fp32 rounding, collapsed columns zero
  orth_wide<MMAX>(xs, ss, inv, dead, D, m, -1);

  T* V = static_cast<T*>(J.V) + layer * J.v_ls + head * J.v_hs;
  float* xg = P.ws + J.xbase + (int64_t)unit * D * mp;
  for (int idx = tid; idx < D * mp; idx += kThreads) {
    const int i = idx / mp, j = idx - i * mp;
    const float v = xs[i * XS + j];
    xg[idx] = v;
    if (j < m) store_elem(V + i * m + j, v);
  }
}

// ---------------------------------------------------------------------------------------
// subspace_wave: widths up to 128, one wave per unit and WPB units per block; every step is
// wave-synchronous. MP = mp exactly. Per wave in LDS:
//   buf [128][MP+4] fp32: X, overwritten by Y = G X, overwritten again by X = orth(Y);
//   lm  (layout lcol) fp64: S = Y^T Y (lower), overwritten by its blocked Cholesky factor;
//       inv holds the starting diagonal, dead the collapsed columns.
// Lane l owns rows l and l + 64.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ void wave_global_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Every rank class (16 .. 64): orth() in 16 x 16 blocks, the products on fp64 MFMA
// 16x16x4 (lane 16 k + i supplies A[i][k] and B[k][i] and receives rows k + 4 v, column i of
// the product in register v). S and then L live in one packed lower triangle stored by columns
// (lcol), and after the factorisation each diagonal block holds T_KK = L_KK^-1 in place of
// L_KK, which is what the substitution needs.
//   S = Y^T Y        all lower tiles at once, four rows of Y per step (fp32 products exact in
//                    fp64, fp64 sums);
//   L L^T = S        right-looking by block column K: the 16 x 16 diagonal block is factored by
//                    lanes 0..15 in registers (lane i holds row i; the pivot and the published
//                    column come by readlane), T_KK is formed alongside (column a by lane a,
//                    right-looking on the same published entries), then the panel
//                    L_IK = S_IK T_KK^T and the trailing update S_IJ -= L_IK L_JK^T run on MFMA;
//   X = Y L^-T       by block column J and 16-row tile: Z^T = Y_J^T - L_J,<J X_<J^T (the
//                    transposed product leaves Z in exactly the A-operand layout), then
//                    X_J = Z T_JJ^T.
// A collapsed column (what is left of its pivot at most kDeadTol times its starting value) gets
// 1 / l_jj = 0: its row of T and its column of L below the pivot are zero, so its x (re-seeded
// between rounds, zero after the last) feeds no later column. The blocked form computes the
// same quantities as a column-by-column Cholesky QR in another order of fp64 additions; it
// replaced that form (the factorisation in one wave's registers and the substitution one row
// per lane, column after column) at every rank: compile of the Qwen2.5-VL-like batch (rank 16)
// 3.34 -> 3.11 ms, of the MLA batch (its 64-wide k_rope heads at rank 32) 16.4 -> 15.4 ms.

template <int MP>
__device__ __forceinline__ void orth_blocked(float* buf, double* lm, double* inv, int* dead, int D,
                                             int m, int reseed_round) {
  static_assert(MP % 16 == 0 && MP <= 64, "rank classes 16 .. 64");
  constexpr int BS = MP + 4, NB = MP / 16, NT = NB * (NB + 1) / 2;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, kk = lane >> 4;
  const int nrt = D / 16;   // D is a multiple of 32

  // S = Y^T Y, lower tiles (a, b <= a)
  {
    f64x4 st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) st[t] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int r = 0; r < D; r += 4) {
      const float* yr = buf + (r + kk) * BS + li;
      double y[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) y[b] = (double)yr[16 * b];
      int t = 0;
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b <= a; ++b, ++t) st[t] = mfma_f64(y[a], y[b], st[t]);
    }
    int t = 0;
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
      for (int b = 0; b <= a; ++b, ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * a + kk + 4 * v, col = 16 * b + li;
          if (row >= col) lm[lcol<MP>(row, col)] = st[t][v];
        }
  }
  wave_lds_sync();
  chol_blocked<MP>(lm, inv, dead, m);
  subst_blocked<MP>(buf, BS, lm, dead, m, 0, nrt, 2, reseed_round);
}

template <int MP>
__device__ __forceinline__ void orth_wave(float* buf, double* lm, double* inv, int* dead, int D, int m,
                                          int reseed_round) {
  orth_blocked<MP>(buf, lm, inv, dead, D, m, reseed_round);
}

#if KAMERA_SUBSPACE_MFMA
// Y = G X for one head, in place in buf (rows of X become rows of Y), on
// v_mfma_f32_16x16x4f32 in G's stored order: K runs over the stored columns kappa, and row
// block rb of the output holds the stored rows 16 rb .. 16 rb + 15 of Y (feature q(rho) for
// stored row rho; GP: G is stored in the symmetric permutation, q(rho) = 8 (rho % 16) +
// rho / 16, else q is the identity). At step (t, u) lane 16 kk + i gives
// A = G_stored[16 rb + i][kappa] and B = X[q(kappa)][16 cb + i], kappa = 16 t + 4 kk + u:
// the round's B operands are read from LDS into registers once (X may then be overwritten by
// Y), and one 16-byte load of a stored row feeds four steps; each piece of G is replaced by
// the next row block's as soon as it is used, so those loads are in flight while the rest of
// the block is multiplied. Even and odd t accumulate apart. D is a multiple of 32, at most 128.
template <int MP, bool GP>
__device__ __forceinline__ void gx_mfma(const float* G, float* buf, int D) {
  constexpr int BS = MP + 4, NCB = MP / 16;
  const int lane = threadIdx.x & 63;
  const int nrb = D / 16;
  const int li = lane & 15, kk = lane >> 4;
  // q(16 t + 4 kk + u) = kbase + kstep(t, u)
  const float* xb = buf + (GP ? 32 * kk : 4 * kk) * BS + li;
  float bx[8][4][NCB];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ks = GP ? 8 * u + t : 16 * t + u;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) bx[t][u][cb] = t < nrb ? xb[ks * BS + 16 * cb] : 0.f;
    }
  wave_lds_sync();   // every lane has read X
  const float* grow = G + (int64_t)li * D + 4 * kk;
  f32x4 ga[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    ga[t] = t < nrb ? ((const CGLOBAL f32x4*)(grow + 16 * t))[0] : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int rb = 0; rb < nrb; ++rb) {
    const int rn = rb + 1 < nrb ? rb + 1 : rb;   // past the end: reload (unused)
    const float* gnext = grow + (int64_t)16 * rn * D;
    f32x4 acc[2][NCB];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[e][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < nrb) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[t & 1][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[t][u], bx[t][u][cb],
                                                                  acc[t & 1][cb], 0, 0, 0);
        ga[t] = ((const CGLOBAL f32x4*)(gnext + 16 * t))[0];   // next row block's piece
      }
    }
    // lane 16 kk + i holds stored rows 16 rb + 4 kk + v, columns 16 cb + i
    float* yb = buf + (GP ? 8 * (4 * kk) * BS + rb * BS : (16 * rb + 4 * kk) * BS) + li;
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        yb[(GP ? 8 * v : v) * BS + 16 * cb] = acc[0][cb][v] + acc[1][cb][v];
  }
  wave_lds_sync();
}
#endif

// Waves per SIMD the subspace kernel is compiled for (MFMA form): a round's X operands, a row
// block of G and the accumulators are live together.
#if KAMERA_SUBSPACE_MFMA
#define KAMERA_SUBSPACE_OCCUPANCY(MP) \
  __attribute__((amdgpu_waves_per_eu((MP) <= 16 ? 3 : ((MP) <= 32 ? 2 : 1), 8)))
#else
#define KAMERA_SUBSPACE_OCCUPANCY(MP)
#endif

template <typename T, int MP, int WPB>
__global__ __launch_bounds__(64 * WPB) KAMERA_SUBSPACE_OCCUPANCY(MP) void subspace_wave_kernel(CParams P) {
  constexpr int BS = MP + 4;
  __shared__ __align__(16) float buf_s[WPB][128 * BS];
  __shared__ __align__(16) double lm_s[WPB][lm_size<MP>()];
  __shared__ double inv_s[WPB][MP];
  __shared__ int dead_s[WPB][MP];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int u = blockIdx.x * WPB + w;
  if (u >= P.n_total) return;   // whole wave; no block-wide barrier follows
  float* buf = buf_s[w];
  double* lm = lm_s[w];
  double* inv = inv_s[w];
  int* dead = dead_s[w];

  const int e = find_entry(P, u);
  const CJob& J = P.jobs[P.job_of[e]];
  const int unit = u - P.starts[e];
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int D = J.width, m = J.m;

  const float* G;
  if (J.gfull < 0) {
    G = P.ws + J.gpart + (int64_t)unit * D * D;
  } else {
    // width <= 128 is a single tile pair: sum the token splits
    float* gf = P.ws + J.gfull + (int64_t)unit * D * D;
    const float4* part4 = reinterpret_cast<const float4*>(P.ws + J.gpart +
                                                          (int64_t)unit * J.splits * D * D);
    const int n4 = D * D / 4;
#pragma unroll 4
    for (int i4 = lane; i4 < n4; i4 += 64) {
      float4 v = part4[i4];
      for (int s = 1; s < J.splits; ++s) {
        const float4 x = part4[(int64_t)s * n4 + i4];
        v.x += x.x;
        v.y += x.y;
        v.z += x.z;
        v.w += x.w;
      }
      reinterpret_cast<float4*>(gf)[i4] = v;
    }
    wave_global_sync();
    G = gf;
  }

#if !KAMERA_SUBSPACE_MFMA
  const int r0 = lane, r1 = lane + 64;
  const int c0 = r0 < D ? r0 : 0, c1 = r1 < D ? r1 : 0;
  // G stored permuted (gram_stream_kernel): element (k, c) at (p(k), p(c))
  const int gp0 = J.gperm ? gperm_row(c0) : c0, gp1 = J.gperm ? gperm_row(c1) : c1;
#endif
  for (int h = 0; h < 2; ++h) {
    const int r = lane + 64 * h;
    if (r >= D) continue;
#pragma unroll
    for (int j = 0; j < MP; ++j) buf[r * BS + j] = j < m ? seed_value(r, j, 0) : 0.f;
  }
  wave_lds_sync();

  for (int round = 0; round < P.n_iter; ++round) {
#if KAMERA_SUBSPACE_MFMA
    if (J.gperm) gx_mfma<MP, true>(G, buf, D);
    else gx_mfma<MP, false>(G, buf, D);
#else
    // Y = G X for rows r0, r1. G is symmetric, so each lane reads its own rows of G along
    // their stored order with 16-byte loads (stored column kappa is feature k = q(kappa)),
    // keeping the next 16 columns in flight while it uses the current ones.
    float y0[MP], y1[MP];
#pragma unroll
    for (int c = 0; c < MP; ++c) y0[c] = y1[c] = 0.f;
    const float* g0row = G + (int64_t)gp0 * D;
    const float* g1row = G + (int64_t)gp1 * D;
    f32x4 ra[4], rb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ra[c] = ((const CGLOBAL f32x4*)g0row)[c];
      rb[c] = ((const CGLOBAL f32x4*)g1row)[c];
    }
    for (int kc0 = 0; kc0 < D; kc0 += 16) {   // D is a multiple of 32
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int kc = kc0 + 4 * c;
        const f32x4 ga = ra[c], gb = rb[c];
        const int kn = kc + 16 < D ? kc + 16 : kc;   // past the end: reload (unused)
        ra[c] = ((const CGLOBAL f32x4*)(g0row + kn))[0];
        rb[c] = ((const CGLOBAL f32x4*)(g1row + kn))[0];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kap = kc + t;
          const int k = J.gperm ? 8 * (kap & 15) + (kap >> 4) : kap;
          const float g0 = ga[t], g1 = gb[t];
          const float4* xr = reinterpret_cast<const float4*>(buf + k * BS);
#pragma unroll
          for (int q = 0; q < MP / 4; ++q) {
            const float4 x = xr[q];
            y0[4 * q] += g0 * x.x;
            y0[4 * q + 1] += g0 * x.y;
            y0[4 * q + 2] += g0 * x.z;
            y0[4 * q + 3] += g0 * x.w;
            y1[4 * q] += g1 * x.x;
            y1[4 * q + 1] += g1 * x.y;
            y1[4 * q + 2] += g1 * x.z;
            y1[4 * q + 3] += g1 * x.w;
          }
        }
      }
    }
    wave_lds_sync();   // every lane has read X
    if (r0 < D) {
      float4* row = reinterpret_cast<float4*>(buf + r0 * BS);
#pragma unroll
      for (int q = 0; q < MP / 4; ++q)
        row[q] = make_float4(y0[4 * q], y0[4 * q + 1], y0[4 * q + 2], y0[4 * q + 3]);
    }
    if (r1 < D) {
      float4* row = reinterpret_cast<float4*>(buf + r1 * BS);
#pragma unroll
      for (int q = 0; q < MP / 4; ++q)
        row[q] = make_float4(y1[4 * q], y1[4 * q + 1], y1[4 * q + 2], y1[4 * q + 3]);
    }
    wave_lds_sync();
#endif
    orth_wave<MP>(buf, lm, inv, dead, D, m, round);
  }
  // last pass on X alone: orthonormal to fp32 rounding, collapsed columns zero
  orth_wave<MP>(buf, lm, inv, dead, D, m, -1);

  T* V = static_cast<T*>(J.V) + layer * J.v_ls + head * J.v_hs;
  float* xg = P.ws + J.xbase + (int64_t)unit * D * MP;
  for (int h = 0; h < 2; ++h) {
    const int r = lane + 64 * h;
    if (r >= D) continue;
#pragma unroll
    for (int j = 0; j < MP; ++j) {
      const float v = buf[r * BS + j];
      xg[r * MP + j] = v;
      if (j < m) store_elem(V + r * m + j, v);
    }
  }
}

// ---------------------------------------------------------------------------------------
// project: U = Delta X for kProjTokens tokens of one unit per block, fp32 MFMA 16x16x4.
// Each step stages 16*TG tokens of Delta (row stride width+4: the 16 rows an MFMA operand
// reads fall in distinct LDS banks); wave w takes token group w % TG and every (4/TG)-th
// 16-column block of X. X sits in LDS with row stride SV (16, or 80 for wider mp at widths
// up to 128, or mp for wider heads).
// ---------------------------------------------------------------------------------------

template <typename T, int DMAX, int TG>
__global__ __launch_bounds__(kThreads) void project_kernel(CParams P) {
  constexpr int RG = 4 / TG;
  constexpr int STEP = 16 * TG;
  constexpr int SVMAX = DMAX <= 128 ? 80 : 32;
  __shared__ __align__(16) float vs[DMAX * SVMAX];
  __shared__ __align__(16) float dl[STEP * (DMAX + 4)];
  __shared__ float2 cs[64];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  const int local = blockIdx.x - P.starts[e];
  const int tblocks = (J.n_tokens + kProjTokens - 1) / kProjTokens;
  const int unit = local / tblocks, tb = local - unit * tblocks;
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int D = J.width, m = J.m, mp = J.mp, tid = threadIdx.x;
  const int DS = D + 4;
  const int SV = mp == 16 ? 16 : (DMAX <= 128 ? 80 : mp);
  if (J.rotate) fill_phases(cs, J, P);
  const float* xg = P.ws + J.xbase + (int64_t)unit * D * mp;
  for (int idx = tid; idx < D * mp; idx += kThreads) {
    const int f = idx / mp, r = idx - f * mp;
    vs[f * SV + r] = xg[idx];
  }

  T* U = static_cast<T*>(J.U) + layer * J.u_ls + head * J.u_hs;
  const int t_lo = tb * kProjTokens, t_hi = min(J.n_tokens, t_lo + kProjTokens);
  const int wave = tid >> 6, lane = tid & 63;
  const int tg = wave % TG, rg = wave / TG;
  const int nrb = mp / 16;
  const int arow = (16 * tg + (lane & 15)) * DS + (lane >> 4);
  const int brow = (lane >> 4) * SV + (lane & 15);
  for (int tok0 = t_lo; tok0 < t_hi; tok0 += STEP) {
    __syncthreads();
    stage_delta<T, STEP>(J, P, cs, layer, head, tok0, t_hi, 0, D, dl, DS);
    __syncthreads();
    f32x4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < D; k0 += 4) {
      const float a = dl[arow + k0];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rb = rg + q * RG;
        if (rb < nrb) {
          const float b = vs[brow + k0 * SV + 16 * rb];
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[q], 0, 0, 0);
        }
      }
    }
    // lane holds U rows tok0 + 16 tg + 4 (lane / 16) + i, column 16 rb + lane % 16
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rb = rg + q * RG;
      const int col = 16 * rb + (lane & 15);
      if (rb < nrb && col < m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tok0 + 16 * tg + 4 * (lane >> 4) + i;
          if (tok < t_hi) store_elem(U + (int64_t)tok * m + col, acc[q][i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// project_stream: U = Delta X with Delta formed in registers (no LDS staging of Delta).
// The sum over a head's features may be taken in any order, so each lane contracts the
// features it loaded itself: lane 16g + n holds token t0 + n and S slots (pieces of 8
// features) per 128-feature slab; MFMA step s takes element s%8 of slot s/8 as A[n][g], and X
// sits in LDS with its rows permuted to match (row 4s + g holds the feature that lane group g
// contracts at step s). Both members of every RoPE pair sit in one lane:
//   contiguous layout: slot p of lane group g is piece 16c + 4p + g of slab c, so one load
//     instruction covers 64 contiguous bytes of each of 16 token rows; half-split partners
//     (pieces i and i + R/16) share a lane when R is a multiple of 64, interleaved pairs
//     always do;
//   pair-unit layout (half-split, R not a multiple of 64, S even): the pieces are listed as
//     pairs (i, i + R/16) followed by the pass-through pieces, and lane group g takes list
//     positions gS .. gS + S - 1.
// Each wave keeps the loads of its next (tile, slab) in flight while it computes the current
// one. Other shapes use project_kernel.
// ---------------------------------------------------------------------------------------

// Dynamic LDS of the streamed projection: bf16 data keeps X^T as bf16 high and low parts
// (rows of width + 8), fp32 data X in fp32 with stream_sv columns.
__host__ __device__ inline size_t stream_lds_bytes(int width, int mp, bool bf16) {
  return bf16 ? (size_t)2 * mp * (width + 8) * sizeof(uint16_t)
              : (size_t)width * stream_sv(width, mp) * sizeof(float);
}

// Tokens per block of the streamed projection: the longest of 2048, 1024 and 512 that still
// gives the launch kProjMinBlocks blocks, each job's tokens cut into equal 16-token multiples
// (long blocks stage X in LDS fewer times; measured on 2 chunks of the rank-64 MHA batch:
// 512 tokens 9.73 ms, 1024 9.48, 2048 9.40; the Qwen2.5-VL-like batch, 7168 heads of 1296
// tokens, kept 512: one 1296-token block per head was 1.7 % slower).
constexpr int kStreamTokenCaps[3] = {2048, 1024, 512};
constexpr int64_t kProjMinBlocks = 16384;

// A finished 16-token tile of U held by one lane (its 4 column blocks x 4 rows) until it is
// stored, in the output element type.
template <typename T> struct UTile;
template <> struct UTile<uint16_t> {
  uint32_t w[8];
  __device__ __forceinline__ void put(int k, float v) {
    const uint32_t h = __builtin_bit_cast(uint16_t, (__bf16)v);   // RNE
    w[k >> 1] = (k & 1) ? (w[k >> 1] | (h << 16)) : h;
  }
  __device__ __forceinline__ void store(uint16_t* p, int k) const {
    *p = (uint16_t)((k & 1) ? (w[k >> 1] >> 16) : (w[k >> 1] & 0xffffu));
  }
};
template <> struct UTile<float> {
  float w[16];
  __device__ __forceinline__ void put(int k, float v) { w[k] = v; }
  __device__ __forceinline__ void store(float* p, int k) const { *p = w[k]; }
};

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 2, 8))) void project_stream_kernel(CParams P) {
  extern __shared__ __align__(16) float vs[];   // permuted X [width][SV]
  __shared__ float2 cs[64];

  const int e = find_entry(P, blockIdx.x);
  const CJob& J = P.jobs[P.job_of[e]];
  const int local = blockIdx.x - P.starts[e];
  const int tblocks = (J.n_tokens + J.ptok - 1) / J.ptok;
  const int unit = local / tblocks, tb = local - unit * tblocks;
  const int layer = unit / J.heads, head = unit - layer * J.heads;
  const int W = J.width, m = J.m, mp = J.mp, tid = threadIdx.x;
  const int S = min(W, 128) / 32;            // slots per lane per slab
  const int nslab = (W + 127) / 128;
  const int R = J.rotate ? J.rot_dim : 0;
  const int hp = R / 16;
  const bool inter = P.layout != KAMERA_ROPE_HALF_SPLIT;
  const int unit_layout = (J.rotate && !inter && R % 64 != 0) ? 1 : 0;
  const int SV = stream_sv(W, mp);
  const int nrb = mp / 16;

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  // this lane's slots: feature offset, and for a rotated head the role (0 pass-through,
  // 1 first member of a half-split pair, 2 second member, 3 interleaved pairs), the first
  // pair index and the partner slot
  int off[4], kind[4], pair0[4], part[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = p < S ? stream_piece(g, p, 0, S, unit_layout, hp) : 0;
    off[p] = 8 * i;
    kind[p] = 0;
    pair0[p] = 0;
    part[p] = p;
    if (p < S && J.rotate) {
      int pi = -1;
      if (inter) {
        if (i < R / 8) { kind[p] = 3; pair0[p] = 4 * i; }
      } else if (i < hp) {
        kind[p] = 1; pair0[p] = 8 * i; pi = i + hp;
      } else if (i < 2 * hp) {
        kind[p] = 2; pair0[p] = 8 * (i - hp); pi = i - hp;
      }
      if (pi >= 0)
        for (int q = 0; q < S; ++q)
          if (stream_piece(g, q, 0, S, unit_layout, hp) == pi) part[p] = q;
    }
  }

  const CMember* mem = P.members + J.member_off;
  const int K = J.n_members;
  const int64_t head_off = (int64_t)head * W;
  const T* canon = static_cast<const T*>(J.canon) + layer * J.canon_ls + head_off;
  const T* cond0 = static_cast<const T*>(mem[0].cond) + layer * mem[0].cond_ls + head_off;
  T* U = static_cast<T*>(J.U) + layer * J.u_ls + head * J.u_hs;
  const int t_lo = tb * J.ptok, t_hi = min(J.n_tokens, t_lo + J.ptok);
  const int ntile = (t_hi - t_lo + 15) / 16;
  const int mine = wave < ntile ? (ntile - wave + 3) / 4 : 0;
  const int total = mine * nslab;

  struct Buf {
    Piece<T> x[4], c[4];
  };
  auto load_unit = [&](int u, Buf& b) {
    const int it = u / nslab, c = u - it * nslab;
    const int tok = t_lo + 16 * (wave + 4 * it) + n;
    const bool ok = tok < t_hi;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < S && ok) {
        load_piece(canon + (int64_t)tok * J.canon_ts + 128 * c + off[p], b.x[p]);
        load_piece(cond0 + (int64_t)tok * mem[0].cond_ts + 128 * c + off[p], b.c[p]);
      } else {
#pragma unroll
        for (int k = 0; k < (int)(sizeof(T) / 2); ++k) {
          b.x[p].w[k] = u32x4{0u, 0u, 0u, 0u};
          b.c[p].w[k] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  // the first unit's loads go out before the block's set-up (phase table, X in LDS), so
  // their latency overlaps it
  Buf cur, nxt;
  f32x4 acc[4];
  if (total > 0) load_unit(0, cur);

  if (J.rotate) fill_phases(cs, J, P);
  const float* xg = P.ws + J.xbase + (int64_t)unit * W * mp;
  // bf16 data: X^T as bf16 high and low parts, row r (rank column) holding the features in
  // order (row stride W + 8: the 16 rows an MFMA operand reads start in distinct banks);
  // fp32 data: X with its rows permuted to the lanes' contraction order
  constexpr bool kBf16 = sizeof(T) == 2;
  const int XW = W + 8;
  uint16_t* xth = reinterpret_cast<uint16_t*>(vs);
  uint16_t* xtl = xth + mp * XW;
  if constexpr (kBf16) {
    for (int idx = tid; idx < W * mp; idx += kThreads) {
      const int f = idx / mp, r = idx - f * mp;
      const float x = xg[idx];
      const uint16_t h = bf16_rne(x);
      xth[r * XW + f] = h;
      xtl[r * XW + f] = bf16_rne(x - __uint_as_float((uint32_t)h << 16));
    }
  } else {
    for (int idx = tid; idx < W * mp; idx += kThreads) {
      const int k = idx / mp, r = idx - k * mp;
      const int sg = k >> 2, gg = k & 3;
      const int c = sg / (8 * S), within = sg - c * 8 * S;
      const int f = 8 * stream_piece(gg, within >> 3, c, S, unit_layout, hp) + (within & 7);
      vs[k * SV + r] = xg[(int64_t)f * mp + r];
    }
  }
  __syncthreads();

  // A tile's U is stored during the next tile, just after that tile's loads are issued. The
  // wait for the next rows (before they become the current ones) covers every earlier memory
  // operation, since loads and stores share one counter; stored this way, the stores have had
  // a tile's compute to complete by then, instead of being issued just before the wait.
  UTile<T> prev;
  int prev_tok = -1;   // first token of the tile in prev, or -1
  auto flush = [&]() {
    if (prev_tok < 0) return;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = 16 * q + n;
      if (q < nrb && col < m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = prev_tok + 4 * g + i;
          if (t < t_hi) prev.store(U + (int64_t)t * m + col, 4 * q + i);
        }
      }
    }
    prev_tok = -1;
  };
  for (int u = 0; u < total; ++u) {
    if (u + 1 < total) load_unit(u + 1, nxt);
    flush();
    const int it = u / nslab, c = u - it * nslab;
    const int tile_tok = t_lo + 16 * (wave + 4 * it);
    const int tok = tile_tok + n;
    if (c == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // per slot: Delta = conditioned - R(delta) canonical, then its 8 MFMA steps
    // (U tile += Delta X, v_mfma_f32_16x16x4f32 per 16-column block)
    const int row0 = 4 * (c * 8 * S) + g;
    const float inv_k = 1.0f / (float)K;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p >= S) continue;
      float d[8], x[8];
      piece_floats(cur.c[p], d);
      if (K > 1) {
        // several orderings: the mean of their conditioned rows
        if (tok < t_hi) {
          for (int k = 1; k < K; ++k) {
            const T* ck = static_cast<const T*>(mem[k].cond) + layer * mem[k].cond_ls +
                          head_off + (int64_t)tok * mem[k].cond_ts + 128 * c + off[p];
            Piece<T> pc;
            load_piece(ck, pc);
            float y[8];
            piece_floats(pc, y);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += y[q];
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] *= inv_k;
      }
      piece_floats(cur.x[p], x);
      const int kd = kind[p];
      if (kd == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = d[q] - x[q];
      } else if (kd == 3) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 r = cs[pair0[p] + j];
          const float a = x[2 * j], b = x[2 * j + 1];
          d[2 * j] = d[2 * j] - (a * r.x - b * r.y);
          d[2 * j + 1] = d[2 * j + 1] - (b * r.x + a * r.y);
        }
      } else {
        const int q0 = part[p];
        Piece<T> praw;
#pragma unroll
        for (int k = 0; k < (int)(sizeof(T) / 2); ++k)
          praw.w[k] = q0 == 0 ? cur.x[0].w[k]
                    : q0 == 1 ? cur.x[1].w[k] : q0 == 2 ? cur.x[2].w[k] : cur.x[3].w[k];
        float y[8];
        piece_floats(praw, y);
        const float sg = kd == 1 ? -1.f : 1.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float2 r = cs[pair0[p] + q];
          d[q] = d[q] - (x[q] * r.x + (sg * y[q]) * r.y);
        }
      }
      if constexpr (kBf16) {
        // U tile += Delta X on v_mfma_f32_16x16x32_bf16: the lane's 8 features are one k-step's
        // A operand (token n), the same 8 features of X^T row 16 b + n its B operand; Delta and
        // X are cut into bf16 high and low parts (round to nearest) and the three products
        // other than low x low are summed small first (dropped: at most ~2^-16 of |Delta X|
        // per term, far below the bf16 rounding of U)
        bf16x8 dh, dl;
        split8_bf16(d, &dh, &dl);
        const int f0 = 128 * c + off[p];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < nrb) {
            const int r = 16 * b + n;
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(xth + r * XW + f0);
            const bf16x8 xl = *reinterpret_cast<const bf16x8*>(xtl + r * XW + f0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dl, xh, acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dh, xl, acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dh, xh, acc[b], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float* br = vs + (row0 + 4 * (8 * p + q)) * SV + n;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (b < nrb) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(d[q], br[16 * b], acc[b], 0, 0, 0);
        }
      }
    }
    if (c == nslab - 1) {
      // lane holds U rows tile_tok + 4g + i, column 16q + n
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) prev.put(4 * q + i, acc[q][i]);
      prev_tok = tile_tok;
    }
    cur = nxt;
  }
  flush();
}

// ---------------------------------------------------------------------------------------
// host: validation, plan, launches
// ---------------------------------------------------------------------------------------

enum Kind { kGram = 0, kSubspace = 1, kProject = 2 };

struct Launch {
  int kind;
  int cls;                          // gram: NB, 0 = streamed; subspace: 0..4; project: 0..1, 2 = streamed
  std::vector<int32_t> starts, job_of;
  int64_t blocks = 0;
  size_t off = 0;                   // byte offset of starts (job_of follows)
  size_t lds = 0;                   // dynamic LDS bytes (streamed projection)
};

// Can project_stream_kernel take this job? Both members of every pair must fit one lane.
bool stream_eligible(const CJob& J, int layout) {
  if (!J.rotate || layout != KAMERA_ROPE_HALF_SPLIT || J.rot_dim % 64 == 0) return true;
  return (std::min(J.width, 128) / 32) % 2 == 0;
}

// A chunk to compile, whichever entry point described it: its orderings (one for a plain
// compile), canonical rows and output factors.
struct MemberIn {
  int64_t delta, delta_s[2];
  kamera_src cond[2];
};
struct ChunkIn {
  int32_t n_tokens = 0, m = 0;
  std::vector<MemberIn> members;
  kamera_src canonical[2];
  kamera_factors_out out[2];
};

struct CPlan {
  std::vector<CJob> jobs;
  std::vector<CMember> members;
  size_t members_off = 0;
  std::vector<Launch> launches;
  size_t freq_off = 0;   // frequency table (kMaxPairs doubles) and pair sections (kMaxPairs bytes)
  size_t sec_off = 0;
  size_t table_bytes = 0;
  size_t data_off = 0;
  size_t total_bytes = 0;
};

// subspace classes: 0..3 one wave per unit (width <= 128, mp = 16, 32, 48, 64); 4, 5 one block
// per unit (width up to 512, mp <= 16, <= 32)
constexpr int kWaveClasses = 4;
constexpr int kWavesPerBlock[kWaveClasses] = {4, 2, 1, 1};   // LDS per block <= 54 KB, 69 KB

int subspace_class(int D, int mp) {
  if (D <= 128) return mp / 16 - 1;
  return mp <= 16 ? 4 : 5;
}

bool width_supported(const Channel& g) {
  if (g.width % 32) return false;
  if (g.rotate) return g.width <= 128;
  return g.width <= 128 || (g.width % 128 == 0 && g.width <= 512);
}

// Views whose elements are base + a*sa + b*sb + [0, size) for a < na, b < nb must not
// overlap themselves (they are written).
bool strided_disjoint(int64_t sa, int64_t na, int64_t sb, int64_t nb, int64_t size) {
  if (na <= 1) { sa = 0; na = 1; }
  if (nb <= 1) { sb = 0; nb = 1; }
  if (na > 1 && nb > 1 && sa > sb) { std::swap(sa, sb); std::swap(na, nb); }
  if (na > 1 && sa < size) return false;
  if (nb > 1) {
    const int64_t inner = na > 1 ? (na - 1) * sa + size : size;
    if (sb < inner) return false;
  }
  return true;
}

kamera_status plan_compile(const kamera_model& M, const std::vector<ChunkIn>& chunks,
                           CPlan* plan) {
  int64_t floats = 0;
  for (int32_t i = 0; i < (int32_t)chunks.size(); ++i) {
    const ChunkIn& k = chunks[i];
    if (k.n_tokens < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: n_tokens < 0", i);
    if (k.n_tokens == 0) continue;
    if (k.m < 1) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: m must be >= 1", i);
    if (k.m > KAMERA_COMPILE_MAX_RANK)
      return fail(KAMERA_ERR_UNSUPPORTED, "chunk %d: m = %d exceeds %d", i, k.m,
                  KAMERA_COMPILE_MAX_RANK);
    auto big = [](int64_t d) { return d >= (int64_t(1) << 31) || d <= -(int64_t(1) << 31); };
    for (size_t q = 0; q < k.members.size(); ++q) {
      const MemberIn& mb = k.members[q];
      if (big(mb.delta))
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d member %d: |delta| must be < 2^31",
                    i, (int)q);
      for (int sct = 1; sct < M.n_sections; ++sct)
        if (big(mb.delta_s[sct - 1]))
          return fail(KAMERA_ERR_INVALID_ARGUMENT,
                      "chunk %d member %d: |delta_sections[%d]| must be < 2^31", i, (int)q,
                      sct - 1);
    }
    for (int ch = 0; ch < 2; ++ch) {
      const Channel g = channel_of(M, ch);
      if (g.rotate && M.rope_dim < g.width && (M.rope_dim % 16 || (g.width - M.rope_dim) % 8))
        return fail(KAMERA_ERR_UNSUPPORTED,
                    "chunk %d channel %d: partial rotary needs rope_dim a multiple of 16 and "
                    "the pass-through width a multiple of 8", i, ch);
      if (!width_supported(g))
        return fail(KAMERA_ERR_UNSUPPORTED,
                    "chunk %d channel %d: width %d not supported by the compile (rotated: a "
                    "multiple of 32 up to 128; unrotated: that or a multiple of 128 up to 512)",
                    i, ch, g.width);
      if (k.m > g.width)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: m = %d exceeds width %d",
                    i, ch, k.m, g.width);
      if (g.width > 128 && k.m > 32)
        return fail(KAMERA_ERR_UNSUPPORTED,
                    "chunk %d channel %d: m = %d above 32 needs width <= 128", i, ch, k.m);
      CJob J{};
      J.canon = k.canonical[ch].ptr;
      J.U = k.out[ch].U;
      J.V = k.out[ch].V;
      J.canon_ls = k.canonical[ch].layer_stride;
      J.canon_ts = k.canonical[ch].token_stride;
      J.u_ls = k.out[ch].u_layer_stride;
      J.u_hs = k.out[ch].u_head_stride;
      J.v_ls = k.out[ch].v_layer_stride;
      J.v_hs = k.out[ch].v_head_stride;
      J.member_off = (int32_t)plan->members.size();
      J.n_members = (int32_t)k.members.size();
      for (const MemberIn& mb : k.members) {
        CMember c{};
        c.cond = mb.cond[ch].ptr;
        c.cond_ls = mb.cond[ch].layer_stride;
        c.cond_ts = mb.cond[ch].token_stride;
        c.delta = mb.delta;
        c.delta_s1 = M.n_sections > 1 ? mb.delta_s[0] : mb.delta;
        c.delta_s2 = M.n_sections > 2 ? mb.delta_s[1] : mb.delta;
        plan->members.push_back(c);
      }
      J.rot_dim = g.rotate ? M.rope_dim : 0;
      // 128-wide heads: gram_split_kernel for bf16 rows whose turning features come in whole
      // 16-feature groups (G in natural order), else gram_stream_kernel (G permuted)
      J.gsplit = M.dtype == KAMERA_DTYPE_BF16 && g.width == 128 &&
                 (!g.rotate || M.rope_dim % 16 == 0) ? 1 : 0;
      J.gperm = g.width == 128 && !J.gsplit ? 1 : 0;
      J.n_tokens = k.n_tokens;
      J.m = k.m;
      J.mp = (k.m + 15) / 16 * 16;
      J.width = g.width;
      J.heads = g.heads;
      J.rotate = g.rotate ? 1 : 0;
      J.te = std::min(g.width, 128);
      J.nb = g.width / J.te;
      J.n_pairs = J.nb * (J.nb + 1) / 2;
      J.n_units = M.n_layers * g.heads;
      // token splits depend on this job alone, so a chunk compiles to the same bits in any
      // batch; only jobs with few Gram tiles split (a split costs a partial G in HBM)
      const int64_t tiles = (int64_t)J.n_units * J.n_pairs;
      int splits = (int)std::max<int64_t>(1, (kGramTilesPerJob + tiles - 1) / tiles);
      splits = std::min(splits, std::max(1, (k.n_tokens + kMinSplitTokens - 1) / kMinSplitTokens));
      int st = (k.n_tokens + splits - 1) / splits;
      st = (st + kStepTokens - 1) / kStepTokens * kStepTokens;
      J.split_tokens = st;
      J.splits = (k.n_tokens + st - 1) / st;
      const int64_t te2 = (int64_t)J.te * J.te;
      J.gpart = floats;
      floats += (int64_t)J.n_units * J.n_pairs * J.splits * te2;
      if (J.n_pairs > 1 || J.splits > 1) {
        J.gfull = floats;
        floats += (int64_t)J.n_units * J.width * J.width;
      } else {
        J.gfull = -1;
      }
      J.xbase = floats;
      floats += (int64_t)J.n_units * J.width * J.mp;
      floats = (floats + 63) / 64 * 64;
      plan->jobs.push_back(J);
    }
  }
  // launches: one per kernel class present
  auto add = [&](int kind, int cls, int job, int64_t blocks, size_t lds = 0) -> bool {
    Launch* L = nullptr;
    for (auto& l : plan->launches)
      if (l.kind == kind && l.cls == cls) L = &l;
    if (!L) {
      plan->launches.push_back(Launch{});
      L = &plan->launches.back();
      L->kind = kind;
      L->cls = cls;
    }
    if (L->blocks + blocks > INT32_MAX) return false;
    L->starts.push_back((int32_t)L->blocks);
    L->job_of.push_back(job);
    L->blocks += blocks;
    L->lds = std::max(L->lds, lds);
    return true;
  };
  {
    auto ptok_at = [](int n, int cap) {
      const int nb = std::max(1, (n + cap - 1) / cap);
      return std::max(16, ((n + nb - 1) / nb + 15) / 16 * 16);
    };
    int cap = kStreamTokenCaps[2];
    for (int c = 0; c < 3; ++c) {
      int64_t b = 0;
      for (const CJob& J : plan->jobs)
        if (stream_eligible(J, M.rope_layout)) {
          const int pt = ptok_at(J.n_tokens, kStreamTokenCaps[c]);
          b += (int64_t)J.n_units * ((J.n_tokens + pt - 1) / pt);
        }
      if (b >= env_int("KAMERA_PROJ_MIN_BLOCKS", (int)kProjMinBlocks)) {
        cap = kStreamTokenCaps[c];
        break;
      }
    }
    for (CJob& J : plan->jobs) J.ptok = ptok_at(J.n_tokens, cap);
  }
  for (size_t j = 0; j < plan->jobs.size(); ++j) {
    const CJob& J = plan->jobs[j];
    const bool stream = stream_eligible(J, M.rope_layout);
    const int tblocks = stream ? (J.n_tokens + J.ptok - 1) / J.ptok
                               : (J.n_tokens + kProjTokens - 1) / kProjTokens;
    const size_t lds = stream ? stream_lds_bytes(J.width, J.mp, M.dtype == KAMERA_DTYPE_BF16) : 0;
    bool ok = add(kGram, J.gsplit ? (J.n_members > 1 ? 6 : 5) : (J.gperm ? 0 : J.te / 32), (int)j,
                  (int64_t)J.n_units * J.n_pairs * J.splits) &&
              add(kSubspace, subspace_class(J.width, J.mp), (int)j, J.n_units) &&
              add(kProject, stream ? 2 : (J.width <= 128 ? 0 : 1), (int)j,
                  (int64_t)J.n_units * tblocks, lds);
    if (!ok) return fail(KAMERA_ERR_UNSUPPORTED, "batch needs more than 2^31-1 blocks");
  }
  size_t off = round_up(plan->jobs.size() * sizeof(CJob), 16);
  plan->members_off = off;
  off = round_up(off + plan->members.size() * sizeof(CMember), 16);
  plan->freq_off = off;
  off += kamera::kMaxPairs * sizeof(double);
  plan->sec_off = off;
  off = round_up(off + kamera::kMaxPairs, 16);
  for (auto& l : plan->launches) {
    l.off = off;
    off += 2 * l.starts.size() * sizeof(int32_t);
    off = round_up(off, 16);
  }
  plan->table_bytes = off;
  plan->data_off = round_up(off, 256);
  plan->total_bytes = plan->data_off + (size_t)floats * sizeof(float);
  return KAMERA_OK;
}

kamera_status validate_compile_pointers(const kamera_model& M, const std::vector<ChunkIn>& chunks) {
  const int64_t es = M.dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  struct Tagged {
    Range r;
    int chunk, ch;
    const char* what;
  };
  std::vector<Tagged> outs, ins;
  auto a16 = [&](int64_t stride) { return (stride * es) % 16 == 0; };
  for (int32_t i = 0; i < (int32_t)chunks.size(); ++i) {
    const ChunkIn& k = chunks[i];
    if (k.n_tokens == 0) continue;
    for (int ch = 0; ch < 2; ++ch) {
      const Channel g = channel_of(M, ch);
      const int64_t row = (int64_t)g.heads * g.width;
      std::vector<const kamera_src*> srcs{&k.canonical[ch]};
      std::vector<const char*> names{"canonical"};
      for (const MemberIn& mb : k.members) {
        srcs.push_back(&mb.cond[ch]);
        names.push_back("conditioned");
      }
      for (size_t s = 0; s < srcs.size(); ++s) {
        const kamera_src& x = *srcs[s];
        if (!x.ptr)
          return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: %s is NULL", i, ch,
                      names[s]);
        if (x.layer_stride < 0 || x.token_stride < row)
          return fail(KAMERA_ERR_INVALID_ARGUMENT,
                      "chunk %d channel %d: %s token_stride %lld shorter than the row (%lld)", i,
                      ch, names[s], (long long)x.token_stride, (long long)row);
        if (!aligned16(x.ptr) || !a16(x.layer_stride) || !a16(x.token_stride))
          return fail(KAMERA_ERR_UNSUPPORTED,
                      "chunk %d channel %d: %s rows must start on 16-byte boundaries", i, ch,
                      names[s]);
        ins.push_back({view_range(x.ptr, x.layer_stride, M.n_layers, x.token_stride, k.n_tokens,
                                  row, es),
                       i, ch, names[s]});
      }
      const kamera_factors_out& o = k.out[ch];
      if (!o.U || !o.V)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: U or V is NULL", i, ch);
      if (o.u_layer_stride < 0 || o.u_head_stride < 0 || o.v_layer_stride < 0 ||
          o.v_head_stride < 0)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: negative factor stride",
                    i, ch);
      const int64_t usz = (int64_t)k.n_tokens * k.m, vsz = (int64_t)g.width * k.m;
      if (!strided_disjoint(o.u_layer_stride, M.n_layers, o.u_head_stride, g.heads, usz))
        return fail(KAMERA_ERR_INVALID_ARGUMENT,
                    "chunk %d channel %d: U strides make layers or heads overlap", i, ch);
      if (!strided_disjoint(o.v_layer_stride, M.n_layers, o.v_head_stride, g.heads, vsz))
        return fail(KAMERA_ERR_INVALID_ARGUMENT,
                    "chunk %d channel %d: V strides make layers or heads overlap", i, ch);
      // extent of a (layers x heads) strided view
      auto extent = [&](const void* p, int64_t ls, int64_t hs, int64_t size) {
        const int64_t last = (M.n_layers - 1) * ls + (g.heads - 1) * hs + size;
        const uintptr_t b = reinterpret_cast<uintptr_t>(p);
        return Range{b, b + (uintptr_t)(last * es)};
      };
      outs.push_back({extent(o.U, o.u_layer_stride, o.u_head_stride, usz), i, ch, "U"});
      outs.push_back({extent(o.V, o.v_layer_stride, o.v_head_stride, vsz), i, ch, "V"});
    }
  }
  std::sort(outs.begin(), outs.end(),
            [](const Tagged& a, const Tagged& b) { return a.r.lo < b.r.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (outs[i].r.lo < outs[i - 1].r.hi)
      return fail(KAMERA_ERR_OVERLAP, "chunk %d channel %d %s overlaps chunk %d channel %d %s",
                  outs[i].chunk, outs[i].ch, outs[i].what, outs[i - 1].chunk, outs[i - 1].ch,
                  outs[i - 1].what);
  for (const Tagged& in : ins) {
    // first output whose end lies past the input's start (ends ascend with starts here,
    // since the outputs are disjoint)
    auto it = std::upper_bound(outs.begin(), outs.end(), in.r.lo,
                               [](uintptr_t v, const Tagged& o) { return v < o.r.hi; });
    if (it != outs.end() && it->r.lo < in.r.hi)
      return fail(KAMERA_ERR_OVERLAP, "chunk %d channel %d %s overlaps chunk %d channel %d %s",
                  it->chunk, it->ch, it->what, in.chunk, in.ch, in.what);
  }
  return KAMERA_OK;
}

template <typename T>
hipError_t launch_one(const Launch& L, CParams P, hipStream_t stream) {
  const dim3 grid((unsigned)L.blocks), block(kThreads);
  switch (L.kind) {
    case kGram:
      switch (L.cls) {
        case 0: gram_stream_kernel<T><<<grid, block, 0, stream>>>(P); break;
        case 1: gram_kernel<T, 1><<<grid, block, 0, stream>>>(P); break;
        case 2: gram_kernel<T, 2><<<grid, block, 0, stream>>>(P); break;
        case 3: gram_kernel<T, 3><<<grid, block, 0, stream>>>(P); break;
        case 4: gram_kernel<T, 4><<<grid, block, 0, stream>>>(P); break;
        case 5:
        case 6:
          if constexpr (sizeof(T) == 2) {
            if (L.cls == 5) gram_split_kernel<T, false><<<grid, block, 0, stream>>>(P);
            else gram_split_kernel<T, true><<<grid, block, 0, stream>>>(P);
            break;
          }
          return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
      }
      break;
    case kSubspace: {
      if (L.cls < kWaveClasses) {
        const int wpb = kWavesPerBlock[L.cls];
        const dim3 wgrid((unsigned)((L.blocks + wpb - 1) / wpb)), wblock(64 * wpb);
        P.n_total = (int32_t)L.blocks;
        switch (L.cls) {
          case 0: subspace_wave_kernel<T, 16, 4><<<wgrid, wblock, 0, stream>>>(P); break;
          case 1: subspace_wave_kernel<T, 32, 2><<<wgrid, wblock, 0, stream>>>(P); break;
          case 2: subspace_wave_kernel<T, 48, 1><<<wgrid, wblock, 0, stream>>>(P); break;
          case 3: subspace_wave_kernel<T, 64, 1><<<wgrid, wblock, 0, stream>>>(P); break;
        }
      } else if (L.cls == 4) {
        subspace_kernel<T, 512, 16><<<grid, block, 0, stream>>>(P);
      } else {
        subspace_kernel<T, 512, 32><<<grid, block, 0, stream>>>(P);
      }
      break;
    }
    case kProject:
      if (L.cls == 2) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&project_stream_kernel<T>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds);
        if (e != hipSuccess) return e;
        project_stream_kernel<T><<<grid, block, L.lds, stream>>>(P);
      } else if (L.cls == 0) {
        project_kernel<T, 128, 4><<<grid, block, 0, stream>>>(P);
      } else {
        project_kernel<T, 512, 2><<<grid, block, 0, stream>>>(P);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}



// The plain compile: one ordering per chunk.
kamera_status lower_plain(const kamera_compile_chunk* chunks, int32_t n_chunks,
                          std::vector<ChunkIn>* out) {
  if (n_chunks < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_chunks must be >= 0");
  if (n_chunks > 0 && !chunks) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunks is NULL");
  out->resize(n_chunks);
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_compile_chunk& k = chunks[i];
    ChunkIn& c = (*out)[i];
    c.n_tokens = k.n_tokens;
    c.m = k.m;
    MemberIn mb{};
    mb.delta = k.delta;
    mb.delta_s[0] = k.delta_sections[0];
    mb.delta_s[1] = k.delta_sections[1];
    for (int ch = 0; ch < 2; ++ch) {
      mb.cond[ch] = k.conditioned[ch];
      c.canonical[ch] = k.canonical[ch];
      c.out[ch] = k.out[ch];
    }
    c.members.push_back(mb);
  }
  return KAMERA_OK;
}

// The orbit compile: the orderings each chunk lists.
kamera_status lower_orbit(const kamera_orbit_chunk* chunks, int32_t n_chunks,
                          std::vector<ChunkIn>* out) {
  if (n_chunks < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_chunks must be >= 0");
  if (n_chunks > 0 && !chunks) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunks is NULL");
  out->resize(n_chunks);
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_orbit_chunk& k = chunks[i];
    ChunkIn& c = (*out)[i];
    c.n_tokens = k.n_tokens;
    c.m = k.m;
    for (int ch = 0; ch < 2; ++ch) {
      c.canonical[ch] = k.canonical[ch];
      c.out[ch] = k.out[ch];
    }
    if (k.n_tokens == 0) continue;
    if (k.n_members < 1 || k.n_members > KAMERA_ORBIT_MAX_MEMBERS)
      return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: n_members must be in [1, %d] (got %d)",
                  i, KAMERA_ORBIT_MAX_MEMBERS, k.n_members);
    if (!k.members) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: members is NULL", i);
    for (int32_t q = 0; q < k.n_members; ++q) {
      const kamera_orbit_member& om = k.members[q];
      MemberIn mb{};
      mb.delta = om.delta;
      mb.delta_s[0] = om.delta_sections[0];
      mb.delta_s[1] = om.delta_sections[1];
      for (int ch = 0; ch < 2; ++ch) mb.cond[ch] = om.conditioned[ch];
      c.members.push_back(mb);
    }
  }
  return KAMERA_OK;
}

size_t workspace_for(const kamera_model* model, const std::vector<ChunkIn>& chunks) {
  CPlan plan;
  if (plan_compile(*model, chunks, &plan) != KAMERA_OK) return 0;
  return round_up(std::max<size_t>(plan.total_bytes, 256), 256);
}

kamera_status compile(const kamera_model* model, const std::vector<ChunkIn>& chunks,
                      int32_t n_iter, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  if (n_iter < 1 || n_iter > 100)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_iter must be in [1, 100] (got %d)", n_iter);
  CPlan plan;
  kamera_status st = plan_compile(*model, chunks, &plan);
  if (st != KAMERA_OK) return st;
  st = validate_compile_pointers(*model, chunks);
  if (st != KAMERA_OK) return st;
  if (!workspace) return fail(KAMERA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(KAMERA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = round_up(std::max<size_t>(plan.total_bytes, 256), 256);
  if (workspace_bytes < need)
    return fail(KAMERA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if (plan.jobs.empty()) return KAMERA_OK;

  std::vector<uint8_t> table(plan.table_bytes, 0);
  std::memcpy(table.data(), plan.jobs.data(), plan.jobs.size() * sizeof(CJob));
  std::memcpy(table.data() + plan.members_off, plan.members.data(),
              plan.members.size() * sizeof(CMember));
  const int pairs = model->rope_dim / 2;
  if (model->inv_freq)
    std::memcpy(table.data() + plan.freq_off, model->inv_freq, pairs * sizeof(double));
  if (model->pair_section)
    std::memcpy(table.data() + plan.sec_off, model->pair_section, pairs);
  for (const Launch& l : plan.launches) {
    std::memcpy(table.data() + l.off, l.starts.data(), l.starts.size() * sizeof(int32_t));
    std::memcpy(table.data() + l.off + l.starts.size() * sizeof(int32_t), l.job_of.data(),
                l.job_of.size() * sizeof(int32_t));
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  st = upload(table, workspace, stream);
  if (st != KAMERA_OK) return st;

  uint8_t* base = static_cast<uint8_t*>(workspace);
  CParams P{};
  P.jobs = reinterpret_cast<const CJob*>(base);
  P.members = reinterpret_cast<const CMember*>(base + plan.members_off);
  P.ws = reinterpret_cast<float*>(base + plan.data_off);
  P.theta = model->rope_theta;
  P.inv_freq = model->inv_freq ? reinterpret_cast<const double*>(base + plan.freq_off) : nullptr;
  P.pair_section = model->pair_section ? base + plan.sec_off : nullptr;
  P.layout = model->rope_layout;
  P.n_iter = n_iter;
  // kernels in dependency order: every Gram tile, then every subspace, then every projection
  for (int kind = kGram; kind <= kProject; ++kind) {
    for (const Launch& l : plan.launches) {
      if (l.kind != kind || l.blocks == 0) continue;
      P.starts = reinterpret_cast<const int32_t*>(base + l.off);
      P.job_of = P.starts + l.starts.size();
      P.n_entries = (int32_t)l.starts.size();
      const hipError_t e = model->dtype == KAMERA_DTYPE_BF16 ? launch_one<uint16_t>(l, P, stream)
                                                             : launch_one<float>(l, P, stream);
      if (e != hipSuccess)
        return fail(KAMERA_ERR_HIP, "compile kernel launch: %s", hipGetErrorString(e));
    }
  }
  return KAMERA_OK;
}

}  // namespace

extern "C" {

size_t kamera_compile_workspace_bytes(const kamera_model* model,
                                      const kamera_compile_chunk* chunks, int32_t n_chunks) {
  if (validate_model(model) != KAMERA_OK) return 0;
  std::vector<ChunkIn> in;
  if (lower_plain(chunks, n_chunks, &in) != KAMERA_OK) return 0;
  return workspace_for(model, in);
}

kamera_status kamera_patch_compile(const kamera_model* model, const kamera_compile_chunk* chunks,
                                   int32_t n_chunks, int32_t n_iter, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  clear_error();
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  std::vector<ChunkIn> in;
  st = lower_plain(chunks, n_chunks, &in);
  if (st != KAMERA_OK) return st;
  return compile(model, in, n_iter, workspace, workspace_bytes, stream);
}

size_t kamera_orbit_compile_workspace_bytes(const kamera_model* model,
                                            const kamera_orbit_chunk* chunks, int32_t n_chunks) {
  if (validate_model(model) != KAMERA_OK) return 0;
  std::vector<ChunkIn> in;
  if (lower_orbit(chunks, n_chunks, &in) != KAMERA_OK) return 0;
  return workspace_for(model, in);
}

kamera_status kamera_patch_compile_orbit(const kamera_model* model,
                                         const kamera_orbit_chunk* chunks, int32_t n_chunks,
                                         int32_t n_iter, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  clear_error();
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  std::vector<ChunkIn> in;
  st = lower_orbit(chunks, n_chunks, &in);
  if (st != KAMERA_OK) return st;
  return compile(model, in, n_iter, workspace, workspace_bytes, stream);
}

}  // extern "C"
