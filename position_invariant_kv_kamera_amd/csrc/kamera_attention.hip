// kamera_attention.hip — the consumer side on gfx950: decode attention over the relocated,
// paged KV cache, and the standard state merge.
//
// The Kamera abstract states that the direct readout of a cached chunk is recovered exactly
// by the standard state merge: attention over several key sets equals the log-sum-exp
// weighted combination of the attention over each. Decode attention is built on it: each
// segment (4096, 2048, 1024 or 512 tokens, per call) of a query's key range is attended on its
// own, and the segments are merged.
//
// attn_rows_kernel<D>: GQA/MHA with n_kv_heads a multiple of 4: block = (segment, quad of KV
//   heads), wave w takes KV head 4 q + w over every 16-token tile of the segment, so each
//   tile's rows are read across four heads at once; each wave writes its head's part.
// attn_segment_kernel<D>: other head counts: block = (segment, KV head), 4 waves; wave w takes
//   the 16-token tiles w, w+4, ... of the segment. Per tile: S = Q K^T with v_mfma_f32_16x16x32_bf16 (the
//   query heads of the KV head are the 16 MFMA rows, padded; q and k are bf16 already, so
//   the products are exact), online softmax per query row in base 2 (max and sum across the
//   16 lanes that hold a row, by DPP row operations), then O += P V on
//   v_mfma_f32_16x16x16_bf16: each fp32 weight is cut exactly into three bf16 terms (hi by
//   truncation, mid = trunc(p - hi), lo = p - hi - mid), so every product is exact and the sum
//   keeps fp32 weights; the V tile passes through LDS as bf16 (the MLA and chunk kernels read
//   its MFMA operands with the LDS transpose read). The four waves' states are merged in LDS
//   and the segment's normalised output and lse are written to the workspace.
// mla_segment_kernel: the same over an MLA cache in the absorbed form; the four waves split
//   the 512 latent features, wave 0 also takes k_rope. The k_rope score MFMA is issued by the
//   compiler for every wave under wave 0's condition (an empty exec mask elsewhere), and an MFMA
//   still reads its operands then, so the other waves keep their k_rope operand registers at
//   zero (stale -inf there once turned 0 x -inf into NaN scores).
// chunk_rows_kernel / chunk_attn_kernel: attention over chunks read in place (relocation
//   folded into the query, the patch into the scores and values), blocks as the two decode
//   kernels above.
// attn_merge_kernel: one block per (query, query head) merges its segments.
// state_merge_kernel: the same merge over caller-given parts.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "kamera_host.h"
#include "kamera_internal.h"

using namespace kamera::host;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Segment length: the longest of the choices that still gives the call at least
// kTargetSegBlocks blocks, or kTargetRowBlocks for attn_rows_kernel (long segments amortise a
// block's set-up and merge; short ones keep a single long context spread over the chip). On
// 64 x 16K tokens of 4 KV heads the rows kernel took 0.389 ms per call at 512 blocks (2048-token
// segments), 0.410 at 1024, 0.428 at 2048 and 0.42 at 256 (4096-token segments); the MLA
// kernel is fastest at 2048 blocks.
constexpr int kSegChoices[4] = {4096, 2048, 1024, KAMERA_ATTN_SEGMENT};
constexpr int64_t kTargetSegBlocks = 2048;
constexpr int64_t kTargetRowBlocks = 512;   // attn_rows_kernel
constexpr int kThreads = 256;
constexpr int kTile = 16;
constexpr int kMaxGroup = 16;

// Max and sum over the 16 lanes of one DPP row (lanes 16 r .. 16 r + 15), every lane taking the
// result: combine with the partner lane in the pair, then in the quad (quad_perm), then with the
// mirrored lane of the half row and of the row. At each step both lanes of a partner pair combine
// the same two values, so all 16 lanes end with the same bits.
template <int CTRL>
__device__ inline float dpp_row(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E;            // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;    // row_half_mirror, row_mirror
__device__ inline float row16_sum(float v) {
  v += dpp_row<kDppSwap1>(v);
  v += dpp_row<kDppSwap2>(v);
  v += dpp_row<kDppHalfMirror>(v);
  return v + dpp_row<kDppMirror>(v);
}
// The max runs on integer keys that order like the floats (non-NaN), so each step is one fused
// DPP integer max.
__device__ inline int order_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ inline float order_key_inv(int k) {
  return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7fffffff));
}
template <int CTRL>
__device__ inline int dpp_row_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ inline float row16_max(float v) {
  int k = order_key(v);
  k = max(k, dpp_row_i<kDppSwap1>(k));
  k = max(k, dpp_row_i<kDppSwap2>(k));
  k = max(k, dpp_row_i<kDppHalfMirror>(k));
  return order_key_inv(max(k, dpp_row_i<kDppMirror>(k)));
}

// Scores run in base-2 units: the host folds log2(e) into the scale (one fp32 rounding), the
// weights are 2^(s - m) from the hardware exp2, and a state's lse is converted back to the
// natural log when it is written: lse = m ln 2 + ln l.
constexpr float kLn2 = 0.693147180559945309f;
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax step of the 4 query rows a lane holds (rows 4 grp + r, token col of the tile):
// s2 are this tile's scores (base 2, -inf for masked tokens). Updates m and l, writes the
// weights p to prow[r * pstride] and returns each row's correction 2^(m_old - m_new) in corr.
__device__ inline void softmax_step(const float (&s2)[4], float (&m)[4], float (&l)[4],
                                    float (&corr)[4], float* prow, int pstride) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float mn = fmaxf(m[r], row16_max(s2[r]));
    float p = 0.f;
    corr[r] = 1.f;
    if (mn != -INFINITY) {
      corr[r] = exp2_hw(m[r] - mn);
      p = exp2_hw(s2[r] - mn);
    }
    l[r] = l[r] * corr[r] + row16_sum(p);
    m[r] = mn;
    prow[r * pstride] = p;
  }
}

// o[c][r] *= corr[r], skipped when no lane's running max moved (every corr is then exactly 1).
template <int NC>
__device__ inline void rescale_rows(f32x4 (&o)[NC], const float (&corr)[4]) {
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[c][r] *= corr[r];
}
__device__ inline bool any_moved(const float (&corr)[4]) {
  return __any(corr[0] != 1.f || corr[1] != 1.f || corr[2] != 1.f || corr[3] != 1.f);
}


struct alignas(16) AQuery {
  int32_t kv_start, kv_len, seg_start, n_segs;
};

struct AParams {
  const AQuery* queries;
  const int32_t* seg_query;   // owning query of each segment
  const uint16_t* q;          // [n_queries][n_q][D]
  const uint16_t* kpool;      // the layer's K pool
  const uint16_t* vpool;      // the layer's V pool
  const int32_t* page_table;  // or NULL (identity)
  float* part_o;              // [segments][n_q][D]
  float* part_lse;            // [segments][n_q]
  float* out;
  float* lse;
  int64_t pool_ts;
  float scale;                  // the call's scale times log2(e): scores in base-2 units
  int32_t n_queries, n_q, n_kv, group, page_size, page_shift, n_pages;
  int32_t seg;                // tokens per segment
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Logical token p -> (logical page, slot).
__device__ __forceinline__ void page_slot(const AParams& P, int64_t p, int64_t* page,
                                          int64_t* slot) {
  if (P.page_shift >= 0) {
    *page = p >> P.page_shift;
    *slot = p & ((int64_t(1) << P.page_shift) - 1);
  } else {
    *page = p / P.page_size;
    *slot = p - *page * P.page_size;
  }
}

// Physical page of token p (its table entry), or -1 for no token.
__device__ __forceinline__ int32_t page_entry(const AParams& P, int64_t p, bool on) {
  if (!on) return -1;
  int64_t page, slot;
  page_slot(P, p, &page, &slot);
  return P.page_table ? P.page_table[page] : (int32_t)page;
}

// Element offset of token p's row given its table entry, or -1 (no token, or a page outside
// the pool).
__device__ __forceinline__ int64_t row_at(const AParams& P, int64_t p, int32_t phys) {
  if (phys < 0 || phys >= P.n_pages) return -1;
  int64_t page, slot;
  page_slot(P, p, &page, &slot);
  return ((int64_t)phys * P.page_size + slot) * P.pool_ts;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }

// P V of one 16-token tile on bf16 MFMA (16x16x16) without rounding the fp32 weights: each
// weight p is cut by truncation into hi (p with its low 16 bits cleared), mid (the same of
// p - hi) and lo = p - hi - mid. Both subtractions are exact (Sterbenz) and lo keeps at most 8
// significant bits, so hi + mid + lo = p exactly and each product with a bf16 value is exact in
// fp32; the three terms are accumulated small first.
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct PSplit {
  s16x4 hi, mid, lo;
};
__device__ inline PSplit split_weights(const float* w4) {
  PSplit s;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t hb = __float_as_uint(w4[j]) & 0xffff0000u;
    const float r = w4[j] - __uint_as_float(hb);
    const uint32_t mb = __float_as_uint(r) & 0xffff0000u;
    const float r2 = r - __uint_as_float(mb);
    s.hi[j] = (short)(hb >> 16);
    s.mid[j] = (short)(mb >> 16);
    s.lo[j] = (short)(__float_as_uint(r2) >> 16);
  }
  return s;
}
// o[c] += P V[:, 16 c ..] for c < n_blocks: lane (col, grp) holds the weights of query row col
// for tokens 4 grp .. 4 grp + 3 (A operand) and takes V rows 4 grp + j, feature 16 c + col
// (bf16, row stride vs, vcol = &V[4 grp][col]; B operand). TR: with one LDS transpose read
// (ds_read_b64_tr_b16): lane s of a 16-lane group points at row s / 4 of its group's four rows,
// features 4 (s % 4) .. + 3 of the block, and lane i receives feature i of the four rows (the
// lane layout was checked on the device); else with four 2-byte reads. The transpose read
// took the MLA and chunk kernels 3 % faster and the GQA decode 0.5 % slower (interleaved A/B).
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
template <bool TR, int NC>
__device__ inline void pv_accumulate(f32x4 (&o)[NC], const PSplit& w, const uint16_t* vcol, int vs,
                                     int n_blocks = NC) {
  const int col = threadIdx.x & 15;
  const uint16_t* tr = vcol - col + (col >> 2) * vs + 4 * (col & 3);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c >= n_blocks) continue;
    s16x4 b;
    if constexpr (TR) {
      b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tr + 16 * c));
    } else {
      const uint16_t* v = vcol + 16 * c;
      b = s16x4{(short)v[0], (short)v[vs], (short)v[2 * vs], (short)v[3 * vs]};
    }
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(w.lo, b, o[c], 0, 0, 0);
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(w.mid, b, o[c], 0, 0, 0);
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(w.hi, b, o[c], 0, 0, 0);
  }
}

// One wave's pass over KV head h for query j: the 16-token tiles starting at t0, t0 + step, ...
// below t_hi, into the online-softmax state of the head's query rows (lane: rows 4 grp + r, m
// and l in base 2, o unnormalised; all 16 lanes of a row group hold the same m and l). vt and
// pt are the wave's own LDS tiles.
template <int D>
__device__ __forceinline__ void attend_tiles(const AParams& P, int j, int h, int t0, int t_hi,
                                             int step, uint16_t* vt, float* pt, float (&m)[4],
                                             float (&l)[4], f32x4 (&o)[D / 16]) {
  constexpr int KS = D / 32;   // bf16 MFMA k-steps of Q K^T
  constexpr int NC = D / 16;   // 16-feature column blocks of O
  constexpr int VS = D + 8;    // LDS row stride of a V tile (bf16): rows start in distinct banks
  constexpr int PS = 17;       // LDS row stride of a P tile (fp32)
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;

  // Q rows: query heads h*group + col (rows past the group are zero)
  bf16x8 qa[KS];
  {
    const bool on = col < P.group;
    const uint16_t* qp = P.q + ((int64_t)j * P.n_q + h * P.group + (on ? col : 0)) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const u32x4 w = on ? *reinterpret_cast<const u32x4*>(qp + 32 * k + 8 * grp)
                         : u32x4{0u, 0u, 0u, 0u};
      qa[k] = __builtin_bit_cast(bf16x8, w);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int koff = h * D;
  auto load_tile = [&](int64_t row, bf16x8* kb, u32x4* vr) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      if (row >= 0) {
        kb[k] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(P.kpool + row + koff + 32 * k + 8 * grp));
        vr[k] = *reinterpret_cast<const u32x4*>(P.vpool + row + koff + 32 * k + 8 * grp);
      } else {
        kb[k] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        vr[k] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto row_of = [&](int t, int32_t pe) { return t + col < t_hi ? row_at(P, t + col, pe) : -1; };
  auto entry_of = [&](int t) { return page_entry(P, t + col, t + col < t_hi); };
  auto tile_step = [&](int64_t row, const bf16x8* kb, const u32x4* vraw) {
    // S: lane holds query rows 4 grp + r of token col
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], kb[k], sacc, 0, 0, 0);
    // the V tile goes to LDS (token col, features 32k + 8 grp ..)
#pragma unroll
    for (int k = 0; k < KS; ++k)
      *reinterpret_cast<u32x4*>(&vt[col * VS + 32 * k + 8 * grp]) = vraw[k];
    float s2[4], corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[r] = row >= 0 ? sacc[r] * P.scale : -INFINITY;
    softmax_step(s2, m, l, corr, &pt[4 * grp * PS + col], PS);
    if (any_moved(corr)) rescale_rows(o, corr);
    wave_lds_sync();
    // O += P V
    pv_accumulate<false>(o, split_weights(&pt[col * PS + 4 * grp]), &vt[4 * grp * VS + col], VS);
    wave_lds_sync();   // the next tile rewrites this wave's P and V tiles
  };
  // software pipeline: the K and V rows of the next tile are in flight while this tile is
  // computed (two tiles ahead, at two waves per SIMD, was 5 % slower in attn_rows_kernel);
  // page-table entries are fetched one tile before the rows they locate
  bf16x8 kb[KS], kb_n[KS];
  u32x4 vraw[KS], vraw_n[KS];
  int64_t row = row_of(t0, entry_of(t0));
  int32_t pe_n = entry_of(t0 + step);
  load_tile(row, kb, vraw);
  for (; t0 < t_hi; t0 += step) {
    const int64_t row_n = row_of(t0 + step, pe_n);
    load_tile(row_n, kb_n, vraw_n);
    pe_n = entry_of(t0 + 2 * step);
    tile_step(row, kb, vraw);
    row = row_n;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kb[k] = kb_n[k];
      vraw[k] = vraw_n[k];
    }
  }
}

// Compiled for 3 waves per SIMD: 160 VGPRs at D = 128, no spills (the unconstrained choice,
// 184 registers at 2 waves per SIMD, streamed ~12 % slower; 4 waves spill).
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void attn_segment_kernel(AParams P) {
  constexpr int NC = D / 16;
  constexpr int VS = D + 8;
  constexpr int PS = 17;
  __shared__ __align__(16) uint16_t vt[4][kTile * VS];
  __shared__ float pt[4][kTile * PS];
  __shared__ float mrg_m[4][kMaxGroup], mrg_l[4][kMaxGroup];
  __shared__ float mrg_o[kMaxGroup * D];   // the waves' weighted outputs, summed in order

  const int g = blockIdx.x / P.n_kv;
  const int h = blockIdx.x - g * P.n_kv;
  const int j = P.seg_query[g];
  const AQuery Q = P.queries[j];
  const int s = g - Q.seg_start;
  const int t_lo = Q.kv_start + s * P.seg;
  const int t_hi = min(Q.kv_start + Q.kv_len, t_lo + P.seg);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;

  float m[4], l[4];
  f32x4 o[NC];
  attend_tiles<D>(P, j, h, t_lo + kTile * wave, t_hi, 4 * kTile, vt[wave], pt[wave], m, l, o);

  // merge the four waves' states (rows 4 grp + r of this lane; all 16 lanes of a row group
  // hold the same m and l): weights exp(m_w - M), outputs summed wave by wave in a fixed order
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrg_m[wave][4 * grp + r] = m[r];
      mrg_l[wave][4 * grp + r] = l[r];
    }
  }
  __syncthreads();
  float wgt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rw = 4 * grp + r;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_m[w][rw]);
    wgt[r] = M == -INFINITY ? 0.f : exp2_hw(m[r] - M);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* dst = &mrg_o[(4 * grp + r) * D + 16 * c + col];
          const float v = o[c][r] * wgt[r];
          *dst = w == 0 ? v : *dst + v;
        }
    }
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < P.group * D; idx += kThreads) {
    const int rw = idx / D, f = idx - rw * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_m[w][rw]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) L += mrg_l[w][rw] * exp2_hw(mrg_m[w][rw] - M);
    }
    const int64_t orow = (int64_t)g * P.n_q + h * P.group + rw;
    P.part_o[orow * D + f] = M == -INFINITY ? 0.f : mrg_o[rw * D + f] / L;
    if (f == 0) P.part_lse[orow] = M == -INFINITY ? -INFINITY : M * kLn2 + logf(L);
  }
}

// attn_rows_kernel<D>: the same segment attention with a block reading whole cache rows:
// block = (segment, quad of KV heads), wave w takes KV head 4 q + w, and the four waves step
// through the same 16-token tiles, so every tile's rows are read across all four heads at once
// rather than as four separate head-wide pieces by four blocks. (A read-only probe over a
// shuffled paged cache of 1 KB rows streamed 0.76 of 8 TB/s in this order against 0.66 with
// one head per block.) Each wave holds its head's whole segment state, so the block writes its
// parts with no merge of the waves. Used when n_kv_heads is a multiple of 4.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void attn_rows_kernel(AParams P) {
  constexpr int NC = D / 16;
  constexpr int VS = D + 8;
  constexpr int PS = 17;
  __shared__ __align__(16) uint16_t vt[4][kTile * VS];
  __shared__ float pt[4][kTile * PS];

  const int quads = P.n_kv >> 2;
  const int g = blockIdx.x / quads;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = 4 * (blockIdx.x - g * quads) + wave;
  const int j = P.seg_query[g];
  const AQuery Q = P.queries[j];
  const int s = g - Q.seg_start;
  const int t_lo = Q.kv_start + s * P.seg;
  const int t_hi = min(Q.kv_start + Q.kv_len, t_lo + P.seg);
  const int col = lane & 15, grp = lane >> 4;

  float m[4], l[4];
  f32x4 o[NC];
  attend_tiles<D>(P, j, h, t_lo, t_hi, kTile, vt[wave], pt[wave], m, l, o);

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rw = 4 * grp + r;
    if (rw >= P.group) continue;
    const int64_t orow = (int64_t)g * P.n_q + h * P.group + rw;
    const bool none = m[r] == -INFINITY;
#pragma unroll
    for (int c = 0; c < NC; ++c) P.part_o[orow * D + 16 * c + col] = none ? 0.f : o[c][r] / l[r];
    if (col == 0) P.part_lse[orow] = none ? -INFINITY : m[r] * kLn2 + logf(l[r]);
  }
}

// ---------------------------------------------------------------------------------------
// mla_segment_kernel: decode attention over an MLA cache in the absorbed form. Every query
// head reads the same single latent row, so the block's 16 MFMA rows are the query heads and
// the block covers one segment. The four waves take the same 16-token tiles: wave w owns
// latent features [128 w, 128 w + 128), its slice of the score (the rows as keys) and of the
// output (the same rows as values), and wave 0 also the k_rope part of the score. The partial
// scores meet in LDS and are summed in wave order, every wave forms the same softmax, and each
// accumulates its own 128 output features: no wave merge is needed at the end.
// ---------------------------------------------------------------------------------------

constexpr int kMlaLatent = 512, kMlaRope = 64;
// Rows of masked tokens are read from here (zeros), so tile loads need no select.
__device__ __align__(16) uint16_t kZeroRow[kMlaLatent + kMlaRope];

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void mla_segment_kernel(AParams P) {
  constexpr int DL = kMlaLatent, DQ = kMlaLatent + kMlaRope;
  constexpr int WS = DL / 4;          // latent features per wave
  constexpr int KSW = WS / 32;        // bf16 k-steps of the wave's latent slice
  constexpr int KSR = kMlaRope / 32;  // bf16 k-steps of k_rope (wave 0)
  constexpr int NCW = WS / 16;        // output column blocks per wave
  constexpr int VS = WS + 8;
  constexpr int PSTR = 17;
  __shared__ __align__(16) uint16_t vt[4][kTile * VS];
  __shared__ float pt[4][kTile * PSTR];
  __shared__ float sc[2][4][kTile * PSTR];   // partial scores, double-buffered by tile

  const int g = blockIdx.x;
  const int j = P.seg_query[g];
  const AQuery Q = P.queries[j];
  const int s = g - Q.seg_start;
  const int t_lo = Q.kv_start + s * P.seg;
  const int t_hi = min(Q.kv_start + Q.kv_len, t_lo + P.seg);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int f0 = WS * wave;

  // query operands: head col (rows past n_q are zero)
  bf16x8 qa[KSW], qr[KSR];
  {
    const bool on = col < P.n_q;
    const uint16_t* qp = P.q + ((int64_t)j * P.n_q + (on ? col : 0)) * DQ;
#pragma unroll
    for (int k = 0; k < KSW; ++k)
      qa[k] = __builtin_bit_cast(bf16x8, on ? *reinterpret_cast<const u32x4*>(qp + f0 + 32 * k + 8 * grp)
                                            : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int k = 0; k < KSR; ++k)
      qr[k] = __builtin_bit_cast(bf16x8, on && wave == 0
                                             ? *reinterpret_cast<const u32x4*>(qp + DL + 32 * k + 8 * grp)
                                             : u32x4{0u, 0u, 0u, 0u});
  }
  float m[4], l[4];
  f32x4 o[NCW];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NCW; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // row of token t0 + col from its page entry pe (-1 past the segment or masked)
  auto row_of = [&](int t0, int32_t pe) -> int64_t {
    return t0 + col < t_hi ? row_at(P, t0 + col, pe) : -1;
  };
  auto entry_of = [&](int t0) { return page_entry(P, t0 + col, t0 + col < t_hi); };
  // this wave's latent slice of token col's row (wave 0 also its k_rope)
  auto load_tile = [&](int64_t row, u32x4 (&lat)[KSW], u32x4 (&rope)[KSR]) {
    const uint16_t* lp = (row >= 0 ? P.vpool + row : kZeroRow) + f0 + 8 * grp;
#pragma unroll
    for (int k = 0; k < KSW; ++k) lat[k] = *reinterpret_cast<const u32x4*>(lp + 32 * k);
    if (wave == 0) {
      const uint16_t* rp = (row >= 0 ? P.kpool + row : kZeroRow) + 8 * grp;
#pragma unroll
      for (int k = 0; k < KSR; ++k) rope[k] = *reinterpret_cast<const u32x4*>(rp + 32 * k);
    }
  };
  auto tile_step = [&](int64_t row, const u32x4 (&lat)[KSW], const u32x4 (&rope)[KSR], int it) {
    // this wave's part of S: lane holds query rows 4 grp + r of token col
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KSW; ++k)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], __builtin_bit_cast(bf16x8, lat[k]),
                                                     sacc, 0, 0, 0);
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < KSR; ++k)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qr[k], __builtin_bit_cast(bf16x8, rope[k]),
                                                       sacc, 0, 0, 0);
    }
    float* scw = sc[it & 1][wave];
#pragma unroll
    for (int r = 0; r < 4; ++r) scw[(4 * grp + r) * PSTR + col] = sacc[r];
    // the latent slice of the tile is also the V operand of this wave's output features
#pragma unroll
    for (int k = 0; k < KSW; ++k)
      *reinterpret_cast<u32x4*>(&vt[wave][col * VS + 32 * k + 8 * grp]) = lat[k];
    __syncthreads();
    float s2[4], corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int idx = (4 * grp + r) * PSTR + col;
      const float tot = ((sc[it & 1][0][idx] + sc[it & 1][1][idx]) + sc[it & 1][2][idx]) +
                        sc[it & 1][3][idx];
      s2[r] = row >= 0 ? tot * P.scale : -INFINITY;
    }
    softmax_step(s2, m, l, corr, &pt[wave][4 * grp * PSTR + col], PSTR);
    if (any_moved(corr)) rescale_rows(o, corr);
    wave_lds_sync();
    pv_accumulate<true>(o, split_weights(&pt[wave][col * PSTR + 4 * grp]), &vt[wave][4 * grp * VS + col],
                  VS);
    wave_lds_sync();   // the next tile rewrites this wave's P and V tiles
  };
  // the rows of the next two tiles are in flight while one is computed (one tile ahead: 6.7 %
  // slower; three: past three waves per SIMD). The k_rope registers of waves 1-3 are zero and
  // stay zero: their k_rope MFMA sits under a wave-uniform branch that the compiler may issue
  // with an empty exec mask, and the MFMA then still runs on its operands.
  u32x4 lat[KSW], rope[KSR], lat_n[KSW], rope_n[KSR], lat_nn[KSW], rope_nn[KSR];
#pragma unroll
  for (int k = 0; k < KSR; ++k) rope[k] = rope_n[k] = rope_nn[k] = u32x4{0u, 0u, 0u, 0u};
  // page-table entries are fetched one tile ahead of the rows they locate
  int64_t row = row_of(t_lo, entry_of(t_lo));
  int64_t row_n = row_of(t_lo + kTile, entry_of(t_lo + kTile));
  int32_t pe_nn = entry_of(t_lo + 2 * kTile);
  load_tile(row, lat, rope);
  load_tile(row_n, lat_n, rope_n);
  int it = 0;
  for (int t0 = t_lo; t0 < t_hi; t0 += kTile, ++it) {
    const int64_t row_nn = row_of(t0 + 2 * kTile, pe_nn);
    load_tile(row_nn, lat_nn, rope_nn);
    pe_nn = entry_of(t0 + 3 * kTile);
    tile_step(row, lat, rope, it);
    row = row_n;
    row_n = row_nn;
#pragma unroll
    for (int k = 0; k < KSW; ++k) {
      lat[k] = lat_n[k];
      lat_n[k] = lat_nn[k];
    }
#pragma unroll
    for (int k = 0; k < KSR; ++k) {
      rope[k] = rope_n[k];
      rope_n[k] = rope_nn[k];
    }
  }
  // every wave holds the same m and l: its own output features, normalised
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int hq = 4 * grp + r;
    if (hq >= P.n_q) continue;
    const int64_t orow = (int64_t)g * P.n_q + hq;
    const bool empty = m[r] == -INFINITY;
#pragma unroll
    for (int c = 0; c < NCW; ++c)
      P.part_o[orow * DL + f0 + 16 * c + col] = empty ? 0.f : o[c][r] / l[r];
    if (wave == 0 && col == 0) P.part_lse[orow] = empty ? -INFINITY : m[r] * kLn2 + logf(l[r]);
  }
}

// Merge n parts of one row: lse of part i at lse_p[i * lse_stride], its output at
// o_p + i * o_stride. Writes out[0 .. D) and *lse_out. The part weights exp(lse_i - M) are
// formed once per row (in chunks of kMergeChunk parts through LDS). The row's features are cut
// into columns of VW floats (VW = 4: 16-byte loads, D % 4 == 0 and o_p 16-byte aligned); when
// a row has fewer columns than the block has threads, G = kMergeThreads / columns groups of
// threads take every G-th part, so many parts are in flight at once, and the groups' sums are
// added in group order through LDS. A part of weight 0 (lse = -inf) is skipped, whatever its
// output holds.
constexpr int kMergeChunk = 256;
constexpr int kMergeThreads = 256;
template <int VW>
__device__ void merge_row(const float* lse_p, int64_t lse_stride, const float* o_p,
                          int64_t o_stride, int n, int D, float* out, float* lse_out) {
  typedef float fv __attribute__((ext_vector_type(VW)));
  constexpr int NCOL = VW == 4 ? 1 : 4;   // columns per thread (D <= 1024)
  __shared__ float red[kMergeThreads / 64];
  __shared__ float wts[kMergeChunk];
  __shared__ __align__(16) float part_sum[kMergeThreads * VW];
  const int tid = threadIdx.x;
  float M = -INFINITY;
  for (int i = tid; i < n; i += kMergeThreads) M = fmaxf(M, lse_p[i * lse_stride]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w, 64));
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int C = D / VW;                              // columns of the row
  const int T = min(C, kMergeThreads);               // threads per group
  const int G = kMergeThreads / T;                   // groups
  const int grp = tid / T, c0 = tid - grp * T;
  const bool active = grp < G;
  fv acc[NCOL];
#pragma unroll
  for (int k = 0; k < NCOL; ++k) acc[k] = fv(0.f);
  float Z = 0.f;
  for (int p0 = 0; p0 < n; p0 += kMergeChunk) {
    const int cn = min(kMergeChunk, n - p0);
    __syncthreads();   // the previous chunk's weights are no longer read
    for (int i = tid; i < cn; i += kMergeThreads)
      wts[i] = M == -INFINITY ? 0.f : expf(lse_p[(p0 + i) * lse_stride] - M);
    __syncthreads();
    for (int i = 0; i < cn; ++i) Z += wts[i];
    if (!active) continue;
#pragma unroll 4
    for (int i = grp; i < cn; i += G) {
      const float e = wts[i];
      if (e == 0.f) continue;
      const float* oi = o_p + (int64_t)(p0 + i) * o_stride;
#pragma unroll
      for (int k = 0; k < NCOL; ++k) {
        const int c = c0 + T * k;
        if (c < C) acc[k] += e * *reinterpret_cast<const fv*>(oi + VW * c);
      }
    }
  }
  if (G > 1) {   // one column per thread: add the groups' sums in group order
    if (active) *reinterpret_cast<fv*>(&part_sum[VW * tid]) = acc[0];
    __syncthreads();
    if (grp == 0) {
      fv t = *reinterpret_cast<const fv*>(&part_sum[VW * c0]);
      for (int g2 = 1; g2 < G; ++g2) t += *reinterpret_cast<const fv*>(&part_sum[VW * (g2 * T + c0)]);
      acc[0] = t;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < NCOL; ++k) {
      const int c = c0 + T * k;
      if (c >= C) continue;
#pragma unroll
      for (int v = 0; v < VW; ++v) out[VW * c + v] = M == -INFINITY ? 0.f : acc[k][v] / Z;
    }
  }
  if (tid == 0) *lse_out = M == -INFINITY ? -INFINITY : M + logf(Z);
}

// Row r of the (query, query head) rows: the parts are the query's segments.
template <int VW>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AParams P, int D) {
  const int r = blockIdx.x;
  const int j = r / P.n_q, qh = r - j * P.n_q;
  const AQuery Q = P.queries[j];
  const int64_t base = (int64_t)Q.seg_start * P.n_q + qh;
  merge_row<VW>(P.part_lse + base, P.n_q, P.part_o + base * D, (int64_t)P.n_q * D, Q.n_segs, D,
                P.out + (int64_t)r * D, P.lse + r);
}

template <int VW>
__global__ __launch_bounds__(kMergeThreads) void state_merge_kernel(const float* part_out,
                                                                    const float* part_lse,
                                                                    float* out, float* lse,
                                                                    int n_parts, int n_rows, int D) {
  const int r = blockIdx.x;
  merge_row<VW>(part_lse + r, n_rows, part_out + (int64_t)r * D, (int64_t)n_rows * D, n_parts, D,
                out + (int64_t)r * D, lse + r);
}

// Parts in the workspace start 256-byte aligned and every head width the attention calls take
// is a multiple of 4, so their merges always read 16 bytes at a time.
void launch_attn_merge(const AParams& P, int64_t rows, int D, hipStream_t stream) {
  attn_merge_kernel<4><<<dim3((unsigned)rows), dim3(kMergeThreads), 0, stream>>>(P, D);
}


// ---------------------------------------------------------------------------------------
// chunk_attn_kernel<D>: attention over chunks read in place. Block = (segment of one chunk,
// KV head), 4 waves over 16-token tiles as attn_segment_kernel. The score contraction runs
// over the head's features and then over the key patch's rank:
//   s_t = <q', k_t> + <w, U_K(t)>,   q' = R(-delta) q,   w = V_K^T q,
// both fp32 and split into bf16 high and low parts (two exact-product MFMA passes each). The
// value patch rides along P V: each 16-token V tile in LDS is followed by the tokens' U_V
// rows, so the same MFMAs accumulate z = sum_t p_t U_V(t) next to o; after the wave merge the
// block adds z V_V^T and normalises.
// ---------------------------------------------------------------------------------------

constexpr int kMaxViewRank = 64;

struct alignas(16) VChunk {
  const uint16_t* k;    // canonical K rows of the layer: token t, head h at k + t*k_ts + h*D
  const uint16_t* v;
  const uint16_t* uk;   // U_K of the layer (head h at + h*uk_hs, token t at + t*mk), or NULL
  const uint16_t* vk;   // V_K of the layer (head h at + h*vk_hs, feature f at + f*mk)
  const uint16_t* uv;
  const uint16_t* vv;
  int64_t k_ts, v_ts;
  int64_t uk_hs, vk_hs, uv_hs, vv_hs;
  int64_t delta, delta_s1, delta_s2;
  int32_t n_tokens, mk, mv;
  int32_t vec_u;        // U rows may be read 16 bytes at a time (both channels)
  int32_t vec_v;        // V factors of a head may be copied 16 bytes at a time (both channels)
  int32_t pad0[3];
};

struct alignas(16) VSeg {
  int32_t chunk, t_lo, t_hi, query;
};

struct VParams {
  const VChunk* chunks;
  const VSeg* segs;
  const uint16_t* q;
  float* part_o;
  float* part_lse;
  const double* inv_freq;       // device (workspace) or NULL
  const uint8_t* pair_section;  // device (workspace) or NULL
  double theta;
  float scale;                  // the call's scale times log2(e): scores in base-2 units
  int32_t n_q, n_kv, group, rot_dim, layout;
};

// 8 consecutive bf16 of a U row from element r0 (zeros at and past m).
__device__ __forceinline__ u32x4 load_u8(const uint16_t* row, int r0, int m, bool vec) {
  if (r0 >= m) return u32x4{0u, 0u, 0u, 0u};
  if (vec && r0 + 8 <= m) return *reinterpret_cast<const u32x4*>(row + r0);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = r0 + 2 * e < m ? row[r0 + 2 * e] : 0u;
    const uint32_t hi = r0 + 2 * e + 1 < m ? row[r0 + 2 * e + 1] : 0u;
    w[e] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// n bf16 from src to LDS dst (n a multiple of 8 when vec), 16 bytes per thread when vec.
__device__ __forceinline__ void stage_rows(const uint16_t* src, int n, bool vec, uint16_t* dst) {
  if (vec) {
    for (int i = threadIdx.x; i < n / 8; i += kThreads)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
  } else {
    for (int i = threadIdx.x; i < n; i += kThreads) dst[i] = src[i];
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Eight fp32 values as two bf16x8 terms: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float* x, bf16x8* hi, bf16x8* lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = bf16_rne(x[2 * e]), h1 = bf16_rne(x[2 * e + 1]);
    const float r0 = x[2 * e] - __uint_as_float((uint32_t)h0 << 16);
    const float r1 = x[2 * e + 1] - __uint_as_float((uint32_t)h1 << 16);
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = (uint32_t)bf16_rne(r0) | ((uint32_t)bf16_rne(r1) << 16);
  }
  *hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  *lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// KMAX: the largest patch rank in the launch, rounded up to 16, 32 or 64 (register budget).
template <int D, int KMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 32 ? 3 : 2, 8)))
void chunk_attn_kernel(VParams P) {
  constexpr int KS = D / 32;                 // bf16 k-steps over the features
  constexpr int PK = (KMAX + 31) / 32;       // bf16 k-steps over the key patch rank
  constexpr int NC = D / 16;                 // column blocks of o
  constexpr int NZ = KMAX / 16;              // column blocks of z
  constexpr int VS = D + 32 * PK + 8;        // LDS row: V row, then the token's U_V row (whole k-steps)
  constexpr int PSTR = 17;
  constexpr int MW = D + KMAX;               // merged row: o, then z
  constexpr int NQ = 2 * KS + 2 * PK;        // score A operands of a lane: q' and w, hi and lo
  static_assert(kTile * 4 * VS >= D * KMAX, "V_K and V_V are staged in the V tiles");
  __shared__ __align__(16) uint16_t vt[4][kTile * VS];
  __shared__ float pt[4][kTile * PSTR];
  __shared__ float mrg_m[4][kMaxGroup], mrg_l[4][kMaxGroup];
  __shared__ float mrg_o[kMaxGroup * MW];    // also holds the query rows during set-up
  __shared__ float wsh[kMaxGroup][KMAX + 1];
  __shared__ float2 cs[64];
  // The score operands are the same in every wave: built once, read from LDS at each tile
  // (kept in registers they would cost 40 of them and one wave per SIMD).
  __shared__ __align__(16) u32x4 qop[NQ][64];

  const int sidx = blockIdx.x / P.n_kv;
  const int h = blockIdx.x - sidx * P.n_kv;
  const VSeg S = P.segs[sidx];
  const VChunk& C = P.chunks[S.chunk];
  const int j = S.query;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int mk = C.mk, mv = C.mv;
  const bool vec = C.vec_u != 0;

  const uint16_t* kh = C.k + h * D;
  const uint16_t* vh = C.v + h * D;
  const uint16_t* ukh = mk > 0 ? C.uk + h * C.uk_hs : nullptr;
  const uint16_t* uvh = mv > 0 ? C.uv + h * C.uv_hs : nullptr;
  // software pipeline: the next tile's K, V, U_K and U_V rows are in flight while this one
  // is computed
  struct Tile {
    u32x4 k[KS], v[KS], uk[PK], uv[PK];
  };
  auto load_tile = [&](int t, Tile& x) {
    const bool ok = t < S.t_hi;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      x.k[k] = ok ? *reinterpret_cast<const u32x4*>(kh + (int64_t)t * C.k_ts + 32 * k + 8 * grp)
                  : u32x4{0u, 0u, 0u, 0u};
      x.v[k] = ok ? *reinterpret_cast<const u32x4*>(vh + (int64_t)t * C.v_ts + 32 * k + 8 * grp)
                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      x.uk[s2] = ok && 32 * s2 < mk ? load_u8(ukh + (int64_t)t * mk, 32 * s2 + 8 * grp, mk, vec)
                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      x.uv[s2] = ok && 32 * s2 < mv ? load_u8(uvh + (int64_t)t * mv, 32 * s2 + 8 * grp, mv, vec)
                                    : u32x4{0u, 0u, 0u, 0u};
  };
  // Every global load of the set-up goes out first, with the first tile's, so the set-up waits
  // for one round trip: the phase inputs (pair tid), the query rows (8 bytes per thread) and
  // V_K of head h (16 bytes at a time, up to four per thread, when its rows allow it).
  const int R = P.rot_dim;   // at most D <= 2 * kThreads: one pair per thread
  const int ip = max(0, min(tid, R / 2 - 1));
  const double inv_in = P.inv_freq && R > 0 ? P.inv_freq[ip] : 0.0;
  const int sec_in = P.pair_section && R > 0 ? (int)P.pair_section[ip] : 0;
  const uint16_t* qrow0 = P.q + ((int64_t)j * P.n_q + h * P.group) * D;
  const bool qon = tid < P.group * D / 4;
  const uint2 qpiece = qon ? reinterpret_cast<const uint2*>(qrow0)[tid] : make_uint2(0u, 0u);
  constexpr int kVkPieces = (D * KMAX / 8 + kThreads - 1) / kThreads;   // per thread, 16 B each
  const bool vk_vec = mk > 0 && C.vec_v != 0;
  const uint16_t* vkh = mk > 0 ? C.vk + h * C.vk_hs : nullptr;
  u32x4 vkp[kVkPieces];
#pragma unroll
  for (int q = 0; q < kVkPieces; ++q) {
    const int idx = tid + kThreads * q;
    vkp[q] = vk_vec && idx < D * mk / 8 ? reinterpret_cast<const u32x4*>(vkh)[idx]
                                        : u32x4{0u, 0u, 0u, 0u};
  }
  Tile cur;
  load_tile(S.t_lo + kTile * wave + col, cur);

  // set-up: the chunk's phases, the query rows (fp32, in mrg_o) and w = V_K^T q
  if (tid < R / 2) {
    const double inv = P.inv_freq ? inv_in : pow(P.theta, -2.0 * (double)tid / (double)R);
    const int sec = P.pair_section ? sec_in : 0;
    const int64_t d = sec == 0 ? C.delta : (sec == 1 ? C.delta_s1 : C.delta_s2);
    double sn, cn;
    sincos((double)d * inv, &sn, &cn);
    cs[tid] = make_float2((float)cn, (float)sn);
  }
  float* qs = mrg_o;   // [group][D]
  if (qon) {
    qs[4 * tid] = __uint_as_float(qpiece.x << 16);
    qs[4 * tid + 1] = __uint_as_float(qpiece.x & 0xffff0000u);
    qs[4 * tid + 2] = __uint_as_float(qpiece.y << 16);
    qs[4 * tid + 3] = __uint_as_float(qpiece.y & 0xffff0000u);
  }
  // V_K of head h staged in LDS (the V tiles are not in use yet)
  uint16_t* stage = &vt[0][0];
  if (vk_vec) {
#pragma unroll
    for (int q = 0; q < kVkPieces; ++q) {
      const int idx = tid + kThreads * q;
      if (idx < D * mk / 8) reinterpret_cast<u32x4*>(stage)[idx] = vkp[q];
    }
  } else if (mk > 0) {
    stage_rows(vkh, D * mk, false, stage);
  }
  __syncthreads();
  // w = V_K^T q on v_mfma_f32_16x16x32_bf16 (q and V_K are bf16, so every product is exact;
  // fp32 sums): wave c takes the rank columns 16 c .. 16 c + 15, the query heads are the rows
  if (wave < (mk + 15) / 16) {
    const int r = 16 * wave + col;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      uint16_t a[8], b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = 32 * k + 8 * grp + e;
        a[e] = col < P.group ? (uint16_t)(__builtin_bit_cast(uint32_t, qs[col * D + f]) >> 16) : 0;
        b[e] = r < mk ? stage[f * mk + r] : 0;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    // lane (grp, col): query heads 4 grp + i, rank r
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i < P.group && r < mk) wsh[4 * grp + i][r] = acc[i];
  }
  __syncthreads();

  // operands of lane (col, grp): query row col, features 32k + 8 grp + e, turned by -delta;
  // built by wave 0 into qop: [q' hi, q' lo] per k-step, then [w hi, w lo] per rank step
  if (wave == 0) {
    bf16x8 qh[KS], ql[KS], wh[PK], wl[PK];
    const bool on = col < P.group;
    const bool inter = P.layout != KAMERA_ROPE_HALF_SPLIT;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = 32 * k + 8 * grp + e;
        float v = 0.f;
        if (on) {
          v = qs[col * D + f];
          if (f < R) {
            int pair, other;
            bool first;
            if (inter) {
              pair = f >> 1;
              first = (f & 1) == 0;
              other = first ? f + 1 : f - 1;
            } else {
              first = f < R / 2;
              pair = first ? f : f - R / 2;
              other = first ? f + R / 2 : f - R / 2;
            }
            const float y = qs[col * D + other];
            const float2 r = cs[pair];
            // R(-delta): first' = x c + y s, second' = x c - y s (x: own, y: partner)
            v = first ? v * r.x + y * r.y : v * r.x - y * r.y;
          }
        }
        x[e] = v;
      }
      split8(x, &qh[k], &ql[k]);
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * s2 + 8 * grp + e;
        x[e] = on && r < mk ? wsh[col][r] : 0.f;
      }
      split8(x, &wh[s2], &wl[s2]);
    }
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qop[2 * k][lane] = __builtin_bit_cast(u32x4, qh[k]);
      qop[2 * k + 1][lane] = __builtin_bit_cast(u32x4, ql[k]);
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2) {
      qop[2 * KS + 2 * s2][lane] = __builtin_bit_cast(u32x4, wh[s2]);
      qop[2 * KS + 2 * s2 + 1][lane] = __builtin_bit_cast(u32x4, wl[s2]);
    }
  }
  __syncthreads();   // qs (in mrg_o) is free again; qop is complete

  float m[4], l[4];
  f32x4 o[NC], z[NZ];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NZ; ++c) z[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  Tile nxt;
  for (int t0 = S.t_lo + kTile * wave; t0 < S.t_hi; t0 += 4 * kTile) {
    const int t = t0 + col;
    const bool valid = t < S.t_hi;
    load_tile(t + 4 * kTile, nxt);
    // S = Q' K^T + W U_K^T: lane holds query rows 4 grp + r of token col
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, cur.k[k]);
      const bf16x8 qh = __builtin_bit_cast(bf16x8, qop[2 * k][lane]);
      const bf16x8 ql = __builtin_bit_cast(bf16x8, qop[2 * k + 1][lane]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kb, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kb, sacc, 0, 0, 0);
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2) {
      if (32 * s2 < mk) {
        const bf16x8 ub = __builtin_bit_cast(bf16x8, cur.uk[s2]);
        const bf16x8 wh = __builtin_bit_cast(bf16x8, qop[2 * KS + 2 * s2][lane]);
        const bf16x8 wl = __builtin_bit_cast(bf16x8, qop[2 * KS + 2 * s2 + 1][lane]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, ub, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, ub, sacc, 0, 0, 0);
      }
    }
    // V rows and U_V rows of the tile to LDS (token col)
#pragma unroll
    for (int k = 0; k < KS; ++k)
      *reinterpret_cast<u32x4*>(&vt[wave][col * VS + 32 * k + 8 * grp]) = cur.v[k];
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      *reinterpret_cast<u32x4*>(&vt[wave][col * VS + D + 32 * s2 + 8 * grp]) = cur.uv[s2];
    float s2[4], corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[r] = valid ? sacc[r] * P.scale : -INFINITY;
    softmax_step(s2, m, l, corr, &pt[wave][4 * grp * PSTR + col], PSTR);
    if (any_moved(corr)) {
      rescale_rows(o, corr);
      rescale_rows(z, corr);
    }
    wave_lds_sync();
    // o += P V and z += P U_V (the U_V rows follow the V rows of the tile)
    {
      const PSplit w = split_weights(&pt[wave][col * PSTR + 4 * grp]);
      const uint16_t* vcol = &vt[wave][4 * grp * VS + col];
      pv_accumulate<true>(o, w, vcol, VS);
      pv_accumulate<true>(z, w, vcol + D, VS, (mv + 15) / 16);
    }
    wave_lds_sync();   // the next tile rewrites this wave's P and V tiles
    cur = nxt;
  }

  // merge the four waves' states (as attn_segment_kernel), o and z together
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mrg_m[wave][4 * grp + r] = m[r];
      mrg_l[wave][4 * grp + r] = l[r];
    }
  }
  __syncthreads();
  float wgt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rw = 4 * grp + r;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_m[w][rw]);
    wgt[r] = M == -INFINITY ? 0.f : exp2_hw(m[r] - M);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = &mrg_o[(4 * grp + r) * MW];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const float v = o[c][r] * wgt[r];
          dst[16 * c + col] = w == 0 ? v : dst[16 * c + col] + v;
        }
#pragma unroll
        for (int c = 0; c < NZ; ++c) {
          const float v = z[c][r] * wgt[r];
          dst[D + 16 * c + col] = w == 0 ? v : dst[D + 16 * c + col] + v;
        }
      }
    }
    __syncthreads();
  }
  // V_V of head h staged in LDS (every wave is past its last tile)
  if (mv > 0) stage_rows(C.vv + h * C.vv_hs, D * mv, C.vec_v != 0, stage);
  __syncthreads();
  for (int idx = tid; idx < P.group * D; idx += kThreads) {
    const int rw = idx / D, f = idx - rw * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, mrg_m[w][rw]);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) L += mrg_l[w][rw] * exp2_hw(mrg_m[w][rw] - M);
    }
    float acc = mrg_o[rw * MW + f];
    for (int r = 0; r < mv; ++r) acc += mrg_o[rw * MW + D + r] * bf16_lo(stage[f * mv + r]);
    const int64_t orow = (int64_t)sidx * P.n_q + h * P.group + rw;
    P.part_o[orow * D + f] = M == -INFINITY ? 0.f : acc / L;
    if (f == 0) P.part_lse[orow] = M == -INFINITY ? -INFINITY : M * kLn2 + logf(L);
  }
}

// chunk_rows_kernel<D, KMAX>: the same attention over chunks read in place with a block reading
// whole rows: block = (segment of one chunk, quad of KV heads), wave w takes KV head 4 q + w over
// every 16-token tile of the segment (as attn_rows_kernel) and does its head's set-up and patch
// term itself: w = V_K^T q on bf16 MFMA from V_K staged in the wave's LDS, the score operands
// (q' and w, high and low bf16 parts) held in registers, and at the end o += z V_V^T on bf16
// MFMA with z cut into three exact bf16 terms (as the P V weights) and V_V staged in the wave's
// LDS. Used when n_kv_heads is a multiple of 4 and no patch rank exceeds 32.
template <int D, int KMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void chunk_rows_kernel(VParams P) {
  static_assert(KMAX == 16 || KMAX == 32, "rank classes of the whole-row kernel");
  constexpr int KS = D / 32;                 // bf16 k-steps over the features
  constexpr int PK = 1;                      // bf16 k-steps over the key patch rank
  constexpr int NC = D / 16;                 // column blocks of o
  constexpr int NZ = KMAX / 16;              // column blocks of z
  constexpr int VS = D + 32 * PK + 8;        // LDS row: V row, then the token's U_V row
  constexpr int PSTR = 17;
  constexpr int WS = KMAX + 1;               // LDS row stride of w and z (fp32)
  // One wave's LDS. In the tile loop: its V tile (V rows, then U_V rows) and P tile. In the
  // set-up and at the end: a factor of the head (V_K, then the head's query rows; V_V at the
  // end; bf16) and w or z (16 rows x WS, fp32).
  constexpr int kLoopBytes = kTile * VS * 2 + kTile * PSTR * 4;
  constexpr int kFactorBytes = D * KMAX * 2 > kMaxGroup * D * 2 ? D * KMAX * 2 : kMaxGroup * D * 2;
  constexpr int kSetBytes = kFactorBytes + kMaxGroup * WS * 4;
  constexpr int kWaveBytes = ((kLoopBytes > kSetBytes ? kLoopBytes : kSetBytes) + 15) / 16 * 16;
  __shared__ __align__(16) uint8_t wbuf[4][kWaveBytes];
  __shared__ float2 cs[64];

  const int quads = P.n_kv >> 2;
  const int sidx = blockIdx.x / quads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = 4 * (blockIdx.x - sidx * quads) + wave;
  const VSeg S = P.segs[sidx];
  const VChunk& C = P.chunks[S.chunk];
  const int j = S.query;
  const int mk = C.mk, mv = C.mv;
  const bool vec = C.vec_u != 0;
  uint16_t* vt = reinterpret_cast<uint16_t*>(wbuf[wave]);
  float* pt = reinterpret_cast<float*>(wbuf[wave] + kTile * VS * 2);
  uint16_t* fac = reinterpret_cast<uint16_t*>(wbuf[wave]);
  float* wz = reinterpret_cast<float*>(wbuf[wave] + kFactorBytes);

  const uint16_t* kh = C.k + h * D;
  const uint16_t* vh = C.v + h * D;
  const uint16_t* ukh = mk > 0 ? C.uk + h * C.uk_hs : nullptr;
  const uint16_t* uvh = mv > 0 ? C.uv + h * C.uv_hs : nullptr;
  // software pipeline: the next tile's K, V, U_K and U_V rows are in flight while this one
  // is computed
  struct Tile {
    u32x4 k[KS], v[KS], uk[PK], uv[PK];
  };
  auto load_tile = [&](int t, Tile& x) {
    const bool ok = t < S.t_hi;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      x.k[k] = ok ? *reinterpret_cast<const u32x4*>(kh + (int64_t)t * C.k_ts + 32 * k + 8 * grp)
                  : u32x4{0u, 0u, 0u, 0u};
      x.v[k] = ok ? *reinterpret_cast<const u32x4*>(vh + (int64_t)t * C.v_ts + 32 * k + 8 * grp)
                  : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      x.uk[s2] = ok && 32 * s2 < mk ? load_u8(ukh + (int64_t)t * mk, 32 * s2 + 8 * grp, mk, vec)
                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      x.uv[s2] = ok && 32 * s2 < mv ? load_u8(uvh + (int64_t)t * mv, 32 * s2 + 8 * grp, mv, vec)
                                    : u32x4{0u, 0u, 0u, 0u};
  };
  // The set-up's global loads go out together with the first tile's: the phase inputs (pair
  // tid of the block), the head's query rows as MFMA A operands (query row col, features
  // 32 k + 8 grp ..; zero past the group) and V_K of the head (16 bytes per lane at a time
  // when its rows allow).
  const int R = P.rot_dim;   // at most D <= 2 * kThreads: one pair per thread
  const int ip = max(0, min(tid, R / 2 - 1));
  const double inv_in = P.inv_freq && R > 0 ? P.inv_freq[ip] : 0.0;
  const int sec_in = P.pair_section && R > 0 ? (int)P.pair_section[ip] : 0;
  const bool qon = col < P.group;
  const uint16_t* qrow = P.q + ((int64_t)j * P.n_q + h * P.group + (qon ? col : 0)) * D;
  u32x4 qa[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    qa[k] = qon ? *reinterpret_cast<const u32x4*>(qrow + 32 * k + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
  constexpr int kVkPieces = (D * KMAX / 8 + 63) / 64;   // per lane, 16 bytes each
  const bool vk_vec = mk > 0 && C.vec_v != 0;
  const uint16_t* vkh = mk > 0 ? C.vk + h * C.vk_hs : nullptr;
  u32x4 vkp[kVkPieces];
#pragma unroll
  for (int q = 0; q < kVkPieces; ++q) {
    const int idx = lane + 64 * q;
    vkp[q] = vk_vec && idx < D * mk / 8 ? reinterpret_cast<const u32x4*>(vkh)[idx]
                                        : u32x4{0u, 0u, 0u, 0u};
  }
  Tile cur;
  load_tile(S.t_lo + col, cur);

  // the chunk's phases (shared by the four heads)
  if (tid < R / 2) {
    const double inv = P.inv_freq ? inv_in : pow(P.theta, -2.0 * (double)tid / (double)R);
    const int sec = P.pair_section ? sec_in : 0;
    const int64_t d = sec == 0 ? C.delta : (sec == 1 ? C.delta_s1 : C.delta_s2);
    double sn, cn;
    sincos((double)d * inv, &sn, &cn);
    cs[tid] = make_float2((float)cn, (float)sn);
  }
  // V_K of the head to the wave's LDS, [feature][rank]
  if (vk_vec) {
#pragma unroll
    for (int q = 0; q < kVkPieces; ++q) {
      const int idx = lane + 64 * q;
      if (idx < D * mk / 8) reinterpret_cast<u32x4*>(fac)[idx] = vkp[q];
    }
  } else if (mk > 0) {
    for (int i = lane; i < D * mk; i += 64) fac[i] = vkh[i];
  }
  __syncthreads();   // the phases are complete; so is each wave's V_K
  // w = V_K^T q on v_mfma_f32_16x16x32_bf16 (q and V_K are bf16, so every product is exact;
  // fp32 sums): rows the query heads, columns the ranks 16 c .. 16 c + 15
#pragma unroll
  for (int c = 0; c < NZ; ++c) {
    if (16 * c >= mk) break;
    const int r = 16 * c + col;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint16_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = r < mk ? fac[(32 * k + 8 * grp + e) * mk + r] : 0;
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[k]),
                                                    __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    // lane (grp, col): query heads 4 grp + i, rank r
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i < P.group && r < mk) wz[(4 * grp + i) * WS + r] = acc[i];
  }
  wave_lds_sync();   // V_K is read; w is complete
  // the head's query rows to the wave's LDS in V_K's place (bf16, rows of D)
  if (qon) {
#pragma unroll
    for (int k = 0; k < KS; ++k)
      *reinterpret_cast<u32x4*>(&fac[col * D + 32 * k + 8 * grp]) = qa[k];
  }
  wave_lds_sync();

  // score operands of lane (col, grp), in registers: query row col, features 32 k + 8 grp + e,
  // turned by -delta, then w of the same row, each as high and low bf16 parts
  bf16x8 qh[KS], ql[KS], wh[PK], wl[PK];
  {
    const bool inter = P.layout != KAMERA_ROPE_HALF_SPLIT;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int f = 32 * k + 8 * grp + e;
        float v = 0.f;
        if (qon) {
          v = __uint_as_float((uint32_t)fac[col * D + f] << 16);
          if (f < R) {
            int pair, other;
            bool first;
            if (inter) {
              pair = f >> 1;
              first = (f & 1) == 0;
              other = first ? f + 1 : f - 1;
            } else {
              first = f < R / 2;
              pair = first ? f : f - R / 2;
              other = first ? f + R / 2 : f - R / 2;
            }
            const float y = __uint_as_float((uint32_t)fac[col * D + other] << 16);
            const float2 r = cs[pair];
            // R(-delta): first' = x c + y s, second' = x c - y s (x: own, y: partner)
            v = first ? v * r.x + y * r.y : v * r.x - y * r.y;
          }
        }
        x[e] = v;
      }
      split8(x, &qh[k], &ql[k]);
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * s2 + 8 * grp + e;
        x[e] = qon && r < mk ? wz[col * WS + r] : 0.f;
      }
      split8(x, &wh[s2], &wl[s2]);
    }
  }
  wave_lds_sync();   // the query rows and w are read: the tiles may take the wave's LDS

  float m[4], l[4];
  f32x4 o[NC], z[NZ];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NZ; ++c) z[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  Tile nxt;
  for (int t0 = S.t_lo; t0 < S.t_hi; t0 += kTile) {
    const int t = t0 + col;
    const bool valid = t < S.t_hi;
    load_tile(t + kTile, nxt);
    // S = Q' K^T + W U_K^T: lane holds query rows 4 grp + r of token col
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bf16x8 kb = __builtin_bit_cast(bf16x8, cur.k[k]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[k], kb, sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[k], kb, sacc, 0, 0, 0);
    }
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2) {
      if (32 * s2 < mk) {
        const bf16x8 ub = __builtin_bit_cast(bf16x8, cur.uk[s2]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh[s2], ub, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl[s2], ub, sacc, 0, 0, 0);
      }
    }
    // V rows and U_V rows of the tile to LDS (token col)
#pragma unroll
    for (int k = 0; k < KS; ++k)
      *reinterpret_cast<u32x4*>(&vt[col * VS + 32 * k + 8 * grp]) = cur.v[k];
#pragma unroll
    for (int s2 = 0; s2 < PK; ++s2)
      *reinterpret_cast<u32x4*>(&vt[col * VS + D + 32 * s2 + 8 * grp]) = cur.uv[s2];
    float s2[4], corr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s2[r] = valid ? sacc[r] * P.scale : -INFINITY;
    softmax_step(s2, m, l, corr, &pt[4 * grp * PSTR + col], PSTR);
    if (any_moved(corr)) {
      rescale_rows(o, corr);
      rescale_rows(z, corr);
    }
    wave_lds_sync();
    // o += P V and z += P U_V (the U_V rows follow the V rows of the tile)
    {
      const PSplit w = split_weights(&pt[col * PSTR + 4 * grp]);
      const uint16_t* vcol = &vt[4 * grp * VS + col];
      pv_accumulate<true>(o, w, vcol, VS);
      pv_accumulate<true>(z, w, vcol + D, VS, (mv + 15) / 16);
    }
    wave_lds_sync();   // the next tile rewrites this wave's P and V tiles
    cur = nxt;
  }

  // o += z V_V^T on v_mfma_f32_16x16x16_bf16: z (rows the query heads, columns the ranks) cut
  // into three exact bf16 terms through LDS, V_V of the head staged [feature][rank]; z is zero
  // at ranks past mv (the U_V loads are zero there)
  if (mv > 0) {
    const uint16_t* vvh = C.vv + h * C.vv_hs;
    if (C.vec_v != 0) {
      for (int i = lane; i < D * mv / 8; i += 64)
        reinterpret_cast<u32x4*>(fac)[i] = reinterpret_cast<const u32x4*>(vvh)[i];
    } else {
      for (int i = lane; i < D * mv; i += 64) fac[i] = vvh[i];
    }
#pragma unroll
    for (int c = 0; c < NZ; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) wz[(4 * grp + i) * WS + 16 * c + col] = z[c][i];
    wave_lds_sync();
#pragma unroll
    for (int kb = 0; kb < NZ; ++kb) {
      if (16 * kb >= mv) break;
      float zw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) zw[e] = wz[col * WS + 16 * kb + 4 * grp + e];
      const PSplit zs = split_weights(zw);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        s16x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * kb + 4 * grp + e;
          b[e] = r < mv ? (short)fac[(16 * c + col) * mv + r] : (short)0;
        }
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zs.lo, b, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zs.mid, b, o[c], 0, 0, 0);
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(zs.hi, b, o[c], 0, 0, 0);
      }
    }
  }
  // this wave's state is the segment's for head h: normalised output and lse
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rw = 4 * grp + r;
    if (rw >= P.group) continue;
    const int64_t orow = (int64_t)sidx * P.n_q + h * P.group + rw;
    const bool none = m[r] == -INFINITY;
#pragma unroll
    for (int c = 0; c < NC; ++c) P.part_o[orow * D + 16 * c + col] = none ? 0.f : o[c][r] / l[r];
    if (col == 0) P.part_lse[orow] = none ? -INFINITY : m[r] * kLn2 + logf(l[r]);
  }
}

// ---------------------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------------------

struct APlan {
  std::vector<AQuery> queries;
  std::vector<int32_t> seg_query;
  int32_t seg = KAMERA_ATTN_SEGMENT;
  size_t seg_off = 0, part_o_off = 0, part_lse_off = 0, total = 0;
};

// Blocks per key segment of kamera_decode_attention: one per quad of KV heads where
// attn_rows_kernel runs (GQA/MHA with n_kv_heads a multiple of 4), else one per KV head.
bool rows_kernel_for(const kamera_model* model) {
  return model->family == KAMERA_FAMILY_GQA && model->n_kv_heads % 4 == 0;
}
int32_t blocks_per_segment(const kamera_model* model) {
  return rows_kernel_for(model) ? model->n_kv_heads / 4 : model->n_kv_heads;
}

kamera_status attention_geometry(const kamera_model* model, int32_t n_q_heads,
                                 const kamera_attn_query* queries, int32_t n_queries,
                                 int64_t capacity, APlan* plan) {
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  if (model->dtype != KAMERA_DTYPE_BF16)
    return fail(KAMERA_ERR_UNSUPPORTED, "decode attention supports bf16 caches");
  if (model->family == KAMERA_FAMILY_MLA) {
    if (model->head_dim != kMlaLatent || model->rope_dim != kMlaRope)
      return fail(KAMERA_ERR_UNSUPPORTED,
                  "MLA decode attention needs a %d-wide latent and %d-wide k_rope (got %d, %d)",
                  kMlaLatent, kMlaRope, model->head_dim, model->rope_dim);
  } else if (model->head_dim != 64 && model->head_dim != 128) {
    return fail(KAMERA_ERR_UNSUPPORTED, "decode attention needs head_dim 64 or 128 (got %d)",
                model->head_dim);
  }
  if (n_q_heads <= 0 || n_q_heads % model->n_kv_heads)
    return fail(KAMERA_ERR_INVALID_ARGUMENT,
                "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", n_q_heads,
                model->n_kv_heads);
  if (n_q_heads / model->n_kv_heads > kMaxGroup)
    return fail(KAMERA_ERR_UNSUPPORTED, "more than %d query heads per KV head", kMaxGroup);
  if (n_queries < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_queries must be >= 0");
  if (n_queries > 0 && !queries) return fail(KAMERA_ERR_INVALID_ARGUMENT, "queries is NULL");
  if ((int64_t)n_queries * n_q_heads > INT32_MAX)
    return fail(KAMERA_ERR_UNSUPPORTED, "too many query rows");
  for (int32_t i = 0; i < n_queries; ++i) {
    const kamera_attn_query& a = queries[i];
    if (a.kv_start < 0 || a.kv_len < 0)
      return fail(KAMERA_ERR_INVALID_ARGUMENT, "query %d: kv_start and kv_len must be >= 0", i);
    if (capacity >= 0 && (int64_t)a.kv_start + a.kv_len > capacity)
      return fail(KAMERA_ERR_INVALID_ARGUMENT,
                  "query %d: tokens [%d, %lld) run past the cache's %lld logical tokens", i,
                  a.kv_start, (long long)a.kv_start + a.kv_len, (long long)capacity);
  }
  plan->seg = kSegChoices[3];
  for (int c = rows_kernel_for(model) ? 0 : 1; c < 4; ++c) {
    int64_t blocks = 0;
    for (int32_t i = 0; i < n_queries; ++i)
      blocks += (queries[i].kv_len + kSegChoices[c] - 1) / kSegChoices[c];
    if (blocks * blocks_per_segment(model) >=
        (rows_kernel_for(model) ? kTargetRowBlocks : kTargetSegBlocks)) {
      plan->seg = kSegChoices[c];
      break;
    }
  }
  const int seg = plan->seg;
  int64_t segs = 0;
  plan->queries.resize(n_queries);
  for (int32_t i = 0; i < n_queries; ++i) {
    const kamera_attn_query& a = queries[i];
    const int n = (a.kv_len + seg - 1) / seg;
    plan->queries[i] = AQuery{a.kv_start, a.kv_len, (int32_t)segs, n};
    for (int k = 0; k < n; ++k) plan->seg_query.push_back(i);
    segs += n;
  }
  if (segs * blocks_per_segment(model) > INT32_MAX)
    return fail(KAMERA_ERR_UNSUPPORTED, "too many attention segments");
  const size_t D = model->head_dim;
  plan->seg_off = round_up(plan->queries.size() * sizeof(AQuery), 16);
  plan->part_o_off = round_up(plan->seg_off + plan->seg_query.size() * sizeof(int32_t), 256);
  plan->part_lse_off = round_up(plan->part_o_off + segs * n_q_heads * D * sizeof(float), 256);
  plan->total = round_up(plan->part_lse_off + segs * n_q_heads * sizeof(float), 256);
  plan->total = std::max<size_t>(plan->total, 256);
  return KAMERA_OK;
}


// Relocation-free read: validation and layout of the device tables.
struct VPlan {
  std::vector<VSeg> segs;
  std::vector<AQuery> queries;   // seg_start / n_segs per query, for attn_merge_kernel
  int32_t seg = KAMERA_ATTN_SEGMENT;
  int32_t mmax = 0;      // the largest patch rank of a chunk with tokens
  bool rows = false;     // chunk_rows_kernel (else chunk_attn_kernel)
  size_t freq_off = 0, sec_off = 0, chunk_off = 0, seg_off = 0, query_off = 0;
  size_t part_o_off = 0, part_lse_off = 0, total = 0;
};

kamera_status chunk_attention_geometry(const kamera_model* model, int32_t n_q_heads,
                                       const kamera_attn_chunk* chunks, int32_t n_chunks,
                                       const kamera_chunk_query* queries, int32_t n_queries,
                                       VPlan* plan) {
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  if (model->family != KAMERA_FAMILY_GQA)
    return fail(KAMERA_ERR_UNSUPPORTED, "chunk attention supports GQA/MHA models");
  if (model->dtype != KAMERA_DTYPE_BF16)
    return fail(KAMERA_ERR_UNSUPPORTED, "chunk attention supports bf16 rows");
  if (model->head_dim != 64 && model->head_dim != 128)
    return fail(KAMERA_ERR_UNSUPPORTED, "chunk attention needs head_dim 64 or 128 (got %d)",
                model->head_dim);
  if (n_q_heads <= 0 || n_q_heads % model->n_kv_heads)
    return fail(KAMERA_ERR_INVALID_ARGUMENT,
                "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", n_q_heads,
                model->n_kv_heads);
  if (n_q_heads / model->n_kv_heads > kMaxGroup)
    return fail(KAMERA_ERR_UNSUPPORTED, "more than %d query heads per KV head", kMaxGroup);
  if (n_chunks < 0 || n_queries < 0)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_chunks and n_queries must be >= 0");
  if (n_chunks > 0 && !chunks) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunks is NULL");
  if (n_queries > 0 && !queries) return fail(KAMERA_ERR_INVALID_ARGUMENT, "queries is NULL");
  if ((int64_t)n_queries * n_q_heads > INT32_MAX)
    return fail(KAMERA_ERR_UNSUPPORTED, "too many query rows");
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_attn_chunk& c = chunks[i];
    if (c.n_tokens < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: n_tokens < 0", i);
    for (int ch = 0; ch < 2; ++ch) {
      const kamera_patch_ref& pr = c.patch[ch];
      if (pr.m < 0 || pr.m > kMaxViewRank)
        return fail(pr.m < 0 ? KAMERA_ERR_INVALID_ARGUMENT : KAMERA_ERR_UNSUPPORTED,
                    "chunk %d channel %d: m = %d outside [0, %d]", i, ch, pr.m, kMaxViewRank);
      if (c.n_tokens == 0) continue;
      const kamera_src& sr = c.src[ch];
      if (!sr.ptr) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: src is NULL", i, ch);
      if (!aligned16(sr.ptr) || sr.token_stride % 8 || sr.layer_stride % 8)
        return fail(KAMERA_ERR_UNSUPPORTED,
                    "chunk %d channel %d: canonical rows must start on 16-byte boundaries", i, ch);
      if (sr.token_stride < (int64_t)model->n_kv_heads * model->head_dim)
        return fail(KAMERA_ERR_INVALID_ARGUMENT,
                    "chunk %d channel %d: token stride shorter than a row", i, ch);
      if (pr.m > 0 && (!pr.U || !pr.V))
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: m > 0 needs U and V", i, ch);
    }
  }
  plan->queries.resize(n_queries);
  for (int32_t i = 0; i < n_queries; ++i) {
    const kamera_chunk_query& a = queries[i];
    if (a.first_chunk < 0 || a.n_chunks < 0 || (int64_t)a.first_chunk + a.n_chunks > n_chunks)
      return fail(KAMERA_ERR_INVALID_ARGUMENT, "query %d: chunks [%d, %lld) outside [0, %d)", i,
                  a.first_chunk, (long long)a.first_chunk + a.n_chunks, n_chunks);
  }
  // the kernel: whole-row blocks (a quad of KV heads) where the heads come in quads and no
  // patch rank exceeds 32
  plan->mmax = 0;
  for (int32_t i = 0; i < n_chunks; ++i)
    if (chunks[i].n_tokens > 0)
      plan->mmax = std::max(plan->mmax, std::max(chunks[i].patch[0].m, chunks[i].patch[1].m));
  plan->rows = model->n_kv_heads % 4 == 0 && plan->mmax <= 32;
  const int64_t per_seg = plan->rows ? model->n_kv_heads / 4 : model->n_kv_heads;
  // segment length: as kamera_decode_attention, segments never cross a chunk
  auto blocks_at = [&](int seg) {
    int64_t b = 0;
    for (int32_t i = 0; i < n_queries; ++i)
      for (int32_t c = 0; c < queries[i].n_chunks; ++c)
        b += (chunks[queries[i].first_chunk + c].n_tokens + seg - 1) / seg;
    return b * per_seg;
  };
  plan->seg = kSegChoices[3];
  for (int c = plan->rows ? 0 : 1; c < 4; ++c)
    if (blocks_at(kSegChoices[c]) >= (plan->rows ? kTargetRowBlocks : kTargetSegBlocks)) {
      plan->seg = kSegChoices[c];
      break;
    }
  const int seg = plan->seg;
  for (int32_t i = 0; i < n_queries; ++i) {
    const int32_t first = (int32_t)plan->segs.size();
    int64_t tokens = 0;
    for (int32_t c = 0; c < queries[i].n_chunks; ++c) {
      const int32_t ci = queries[i].first_chunk + c;
      const int32_t n = chunks[ci].n_tokens;
      tokens += n;
      for (int32_t t = 0; t < n; t += seg)
        plan->segs.push_back(VSeg{ci, t, std::min(n, t + seg), i});
    }
    plan->queries[i] = AQuery{0, (int32_t)std::min<int64_t>(tokens, INT32_MAX), first,
                              (int32_t)plan->segs.size() - first};
  }
  if ((int64_t)plan->segs.size() * per_seg > INT32_MAX)
    return fail(KAMERA_ERR_UNSUPPORTED, "too many attention segments");
  const size_t D = model->head_dim;
  plan->freq_off = 0;
  plan->sec_off = plan->freq_off + 64 * sizeof(double);
  plan->chunk_off = round_up(plan->sec_off + 64, 16);
  plan->seg_off = round_up(plan->chunk_off + (size_t)n_chunks * sizeof(VChunk), 16);
  plan->query_off = round_up(plan->seg_off + plan->segs.size() * sizeof(VSeg), 16);
  plan->part_o_off = round_up(plan->query_off + plan->queries.size() * sizeof(AQuery), 256);
  const size_t segs = plan->segs.size();
  plan->part_lse_off = round_up(plan->part_o_off + segs * n_q_heads * D * sizeof(float), 256);
  plan->total = round_up(plan->part_lse_off + segs * n_q_heads * sizeof(float), 256);
  return KAMERA_OK;
}

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

extern "C" {

size_t kamera_attention_workspace_bytes(const kamera_model* model, int32_t n_q_heads,
                                        const kamera_attn_query* queries, int32_t n_queries) {
  APlan plan;
  if (attention_geometry(model, n_q_heads, queries, n_queries, -1, &plan) != KAMERA_OK) return 0;
  return plan.total;
}

kamera_status kamera_decode_attention(const kamera_model* model, const kamera_cache* cache,
                                      int32_t layer, const void* q, int32_t n_q_heads,
                                      const kamera_attn_query* queries, int32_t n_queries,
                                      float scale, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream_ptr) {
  clear_error();
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  st = validate_cache(*model, cache);
  if (st != KAMERA_OK) return st;
  const int64_t capacity = (int64_t)cache->n_logical_pages * cache->page_size;
  APlan plan;
  st = attention_geometry(model, n_q_heads, queries, n_queries, capacity, &plan);
  if (st != KAMERA_OK) return st;
  if (layer < 0 || layer >= model->n_layers)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, model->n_layers);
  if (!std::isfinite(scale) || !std::isfinite((float)((double)scale * 1.4426950408889634)))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "scale must be finite (also times log2(e))");
  if (n_queries > 0 && (!q || !out || !lse))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "q, out and lse must not be NULL");
  if (q && !aligned16(q)) return fail(KAMERA_ERR_UNSUPPORTED, "q must be 16-byte aligned");
  // 16-byte row loads from both pools
  if (!aligned16(cache->pool[0]) || !aligned16(cache->pool[1]) || cache->token_stride % 8 ||
      cache->layer_stride % 8)
    return fail(KAMERA_ERR_UNSUPPORTED, "cache rows must start on 16-byte boundaries");
  const size_t D = model->head_dim;
  const bool mla = model->family == KAMERA_FAMILY_MLA;
  const size_t DQ = mla ? (size_t)kMlaLatent + kMlaRope : D;   // query row length
  const size_t rows = (size_t)n_queries * n_q_heads;
  if (n_queries > 0 && (ranges_overlap(out, rows * D * 4, lse, rows * 4) ||
                        ranges_overlap(out, rows * D * 4, q, rows * DQ * 2) ||
                        ranges_overlap(lse, rows * 4, q, rows * DQ * 2)))
    return fail(KAMERA_ERR_OVERLAP, "q, out and lse must not overlap");
  if (!workspace) return fail(KAMERA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(KAMERA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(KAMERA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                plan.total);
  if (n_queries == 0) return KAMERA_OK;

  std::vector<uint8_t> table(plan.part_o_off, 0);
  std::memcpy(table.data(), plan.queries.data(), plan.queries.size() * sizeof(AQuery));
  if (!plan.seg_query.empty())
    std::memcpy(table.data() + plan.seg_off, plan.seg_query.data(),
                plan.seg_query.size() * sizeof(int32_t));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  st = upload(table, workspace, stream);
  if (st != KAMERA_OK) return st;

  uint8_t* base = static_cast<uint8_t*>(workspace);
  AParams P{};
  P.queries = reinterpret_cast<const AQuery*>(base);
  P.seg_query = reinterpret_cast<const int32_t*>(base + plan.seg_off);
  P.q = static_cast<const uint16_t*>(q);
  P.kpool = static_cast<const uint16_t*>(cache->pool[0]) + (int64_t)layer * cache->layer_stride;
  P.vpool = static_cast<const uint16_t*>(cache->pool[1]) + (int64_t)layer * cache->layer_stride;
  P.page_table = cache->page_table;
  P.part_o = reinterpret_cast<float*>(base + plan.part_o_off);
  P.part_lse = reinterpret_cast<float*>(base + plan.part_lse_off);
  P.out = out;
  P.lse = lse;
  P.pool_ts = cache->token_stride;
  P.scale = (float)((double)scale * 1.4426950408889634);   // scores in base-2 units
  P.n_queries = n_queries;
  P.n_q = n_q_heads;
  P.n_kv = model->n_kv_heads;
  P.group = n_q_heads / model->n_kv_heads;
  P.page_size = cache->page_size;
  P.page_shift = -1;
  for (int b = 0; b < 31; ++b)
    if (cache->page_size == (1 << b)) P.page_shift = b;
  P.n_pages = cache->n_pages;
  P.seg = plan.seg;
  const int64_t seg_blocks = (int64_t)plan.seg_query.size() * blocks_per_segment(model);
  if (seg_blocks > 0) {
    const dim3 grid((unsigned)seg_blocks), block(kThreads);
    const bool rows_kernel = rows_kernel_for(model);
    if (mla) mla_segment_kernel<<<grid, block, 0, stream>>>(P);
    else if (rows_kernel && D == 128) attn_rows_kernel<128><<<grid, block, 0, stream>>>(P);
    else if (rows_kernel) attn_rows_kernel<64><<<grid, block, 0, stream>>>(P);
    else if (D == 128) attn_segment_kernel<128><<<grid, block, 0, stream>>>(P);
    else attn_segment_kernel<64><<<grid, block, 0, stream>>>(P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KAMERA_ERR_HIP, "attention kernel launch: %s", hipGetErrorString(e));
  }
  launch_attn_merge(P, rows, (int)D, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

size_t kamera_chunk_attention_workspace_bytes(const kamera_model* model, int32_t n_q_heads,
                                              const kamera_attn_chunk* chunks, int32_t n_chunks,
                                              const kamera_chunk_query* queries,
                                              int32_t n_queries) {
  VPlan plan;
  if (chunk_attention_geometry(model, n_q_heads, chunks, n_chunks, queries, n_queries, &plan) !=
      KAMERA_OK)
    return 0;
  return plan.total;
}

kamera_status kamera_chunk_attention(const kamera_model* model, int32_t layer,
                                     const kamera_attn_chunk* chunks, int32_t n_chunks,
                                     const kamera_chunk_query* queries, int32_t n_queries,
                                     const void* q, int32_t n_q_heads, float scale, float* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream_ptr) {
  clear_error();
  VPlan plan;
  kamera_status st =
      chunk_attention_geometry(model, n_q_heads, chunks, n_chunks, queries, n_queries, &plan);
  if (st != KAMERA_OK) return st;
  if (layer < 0 || layer >= model->n_layers)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, model->n_layers);
  if (!std::isfinite(scale) || !std::isfinite((float)((double)scale * 1.4426950408889634)))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "scale must be finite (also times log2(e))");
  if (n_queries > 0 && (!q || !out || !lse))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "q, out and lse must not be NULL");
  if (q && !aligned16(q)) return fail(KAMERA_ERR_UNSUPPORTED, "q must be 16-byte aligned");
  const size_t D = model->head_dim;
  const size_t rows = (size_t)n_queries * n_q_heads;
  if (n_queries > 0 && (ranges_overlap(out, rows * D * 4, lse, rows * 4) ||
                        ranges_overlap(out, rows * D * 4, q, rows * D * 2) ||
                        ranges_overlap(lse, rows * 4, q, rows * D * 2)))
    return fail(KAMERA_ERR_OVERLAP, "q, out and lse must not overlap");
  if (!workspace) return fail(KAMERA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(KAMERA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < plan.total)
    return fail(KAMERA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                plan.total);
  if (n_queries == 0) return KAMERA_OK;

  std::vector<uint8_t> table(plan.part_o_off, 0);
  const int pairs = model->rope_dim / 2;
  if (model->inv_freq) std::memcpy(table.data() + plan.freq_off, model->inv_freq, pairs * sizeof(double));
  if (model->pair_section) std::memcpy(table.data() + plan.sec_off, model->pair_section, pairs);
  const int64_t es = 2;
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_attn_chunk& c = chunks[i];
    VChunk v{};
    v.n_tokens = c.n_tokens;
    v.delta = c.delta;
    v.delta_s1 = model->n_sections > 1 ? c.delta_sections[0] : c.delta;
    v.delta_s2 = model->n_sections > 2 ? c.delta_sections[1] : c.delta;
    if (c.n_tokens > 0) {
      v.k = static_cast<const uint16_t*>(c.src[0].ptr) + (int64_t)layer * c.src[0].layer_stride;
      v.v = static_cast<const uint16_t*>(c.src[1].ptr) + (int64_t)layer * c.src[1].layer_stride;
      v.k_ts = c.src[0].token_stride;
      v.v_ts = c.src[1].token_stride;
    }
    bool vec = true, vecv = true;
    for (int ch = 0; ch < 2; ++ch) {
      const kamera_patch_ref& pr = c.patch[ch];
      const int m = c.n_tokens > 0 ? pr.m : 0;
      const uint16_t* U = m ? static_cast<const uint16_t*>(pr.U) + (int64_t)layer * pr.u_layer_stride : nullptr;
      const uint16_t* V = m ? static_cast<const uint16_t*>(pr.V) + (int64_t)layer * pr.v_layer_stride : nullptr;
      if (m && (!aligned16(U) || (pr.u_head_stride * es) % 16 || (m * es) % 16)) vec = false;
      if (m && (!aligned16(V) || (pr.v_head_stride * es) % 16 || (model->head_dim * m) % 8))
        vecv = false;
      if (ch == 0) {
        v.mk = m;
        v.uk = U;
        v.vk = V;
        v.uk_hs = pr.u_head_stride;
        v.vk_hs = pr.v_head_stride;
      } else {
        v.mv = m;
        v.uv = U;
        v.vv = V;
        v.uv_hs = pr.u_head_stride;
        v.vv_hs = pr.v_head_stride;
      }
    }
    v.vec_u = vec ? 1 : 0;
    v.vec_v = vecv ? 1 : 0;
    std::memcpy(table.data() + plan.chunk_off + i * sizeof(VChunk), &v, sizeof v);
  }
  if (!plan.segs.empty())
    std::memcpy(table.data() + plan.seg_off, plan.segs.data(), plan.segs.size() * sizeof(VSeg));
  std::memcpy(table.data() + plan.query_off, plan.queries.data(),
              plan.queries.size() * sizeof(AQuery));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  st = upload(table, workspace, stream);
  if (st != KAMERA_OK) return st;

  uint8_t* base = static_cast<uint8_t*>(workspace);
  VParams P{};
  P.chunks = reinterpret_cast<const VChunk*>(base + plan.chunk_off);
  P.segs = reinterpret_cast<const VSeg*>(base + plan.seg_off);
  P.q = static_cast<const uint16_t*>(q);
  P.part_o = reinterpret_cast<float*>(base + plan.part_o_off);
  P.part_lse = reinterpret_cast<float*>(base + plan.part_lse_off);
  P.inv_freq = model->inv_freq ? reinterpret_cast<const double*>(base + plan.freq_off) : nullptr;
  P.pair_section = model->pair_section ? base + plan.sec_off : nullptr;
  P.theta = model->rope_theta;
  P.scale = (float)((double)scale * 1.4426950408889634);   // scores in base-2 units
  P.n_q = n_q_heads;
  P.n_kv = model->n_kv_heads;
  P.group = n_q_heads / model->n_kv_heads;
  P.rot_dim = model->rope_dim;
  P.layout = model->rope_layout;
  const int64_t seg_blocks =
      (int64_t)plan.segs.size() * (plan.rows ? model->n_kv_heads / 4 : model->n_kv_heads);
  if (seg_blocks > 0) {
    const dim3 grid((unsigned)seg_blocks), block(kThreads);
    const int mmax = plan.mmax;
    if (plan.rows) {
      if (D == 128 && mmax <= 16) chunk_rows_kernel<128, 16><<<grid, block, 0, stream>>>(P);
      else if (D == 128) chunk_rows_kernel<128, 32><<<grid, block, 0, stream>>>(P);
      else if (mmax <= 16) chunk_rows_kernel<64, 16><<<grid, block, 0, stream>>>(P);
      else chunk_rows_kernel<64, 32><<<grid, block, 0, stream>>>(P);
    } else if (D == 128) {
      if (mmax <= 16) chunk_attn_kernel<128, 16><<<grid, block, 0, stream>>>(P);
      else if (mmax <= 32) chunk_attn_kernel<128, 32><<<grid, block, 0, stream>>>(P);
      else chunk_attn_kernel<128, 64><<<grid, block, 0, stream>>>(P);
    } else {
      if (mmax <= 16) chunk_attn_kernel<64, 16><<<grid, block, 0, stream>>>(P);
      else if (mmax <= 32) chunk_attn_kernel<64, 32><<<grid, block, 0, stream>>>(P);
      else chunk_attn_kernel<64, 64><<<grid, block, 0, stream>>>(P);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KAMERA_ERR_HIP, "chunk attention kernel launch: %s", hipGetErrorString(e));
  }
  AParams M{};
  M.queries = reinterpret_cast<const AQuery*>(base + plan.query_off);
  M.part_o = P.part_o;
  M.part_lse = P.part_lse;
  M.out = out;
  M.lse = lse;
  M.n_q = n_q_heads;
  launch_attn_merge(M, rows, (int)D, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

kamera_status kamera_state_merge(int32_t n_parts, int32_t n_rows, int32_t head_dim,
                                 const float* part_out, const float* part_lse, float* out,
                                 float* lse, void* stream_ptr) {
  clear_error();
  if (n_parts < 0 || n_rows < 0)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_parts and n_rows must be >= 0");
  if (head_dim <= 0 || head_dim > 1024)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "head_dim must be in [1, 1024] (got %d)", head_dim);
  if (n_rows == 0) return KAMERA_OK;
  if (!out || !lse || (n_parts > 0 && (!part_out || !part_lse)))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "NULL buffer");
  const size_t po = (size_t)n_parts * n_rows * head_dim * 4, pl = (size_t)n_parts * n_rows * 4;
  const size_t oo = (size_t)n_rows * head_dim * 4, ol = (size_t)n_rows * 4;
  if (ranges_overlap(out, oo, lse, ol) || (n_parts > 0 && (ranges_overlap(out, oo, part_out, po) ||
                                                           ranges_overlap(out, oo, part_lse, pl) ||
                                                           ranges_overlap(lse, ol, part_out, po) ||
                                                           ranges_overlap(lse, ol, part_lse, pl))))
    return fail(KAMERA_ERR_OVERLAP, "out and lse must not overlap the parts or each other");
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool vec = head_dim % 4 == 0 && reinterpret_cast<uintptr_t>(part_out) % 16 == 0;
  if (vec)
    state_merge_kernel<4><<<dim3((unsigned)n_rows), dim3(kMergeThreads), 0, stream>>>(
        part_out, part_lse, out, lse, n_parts, n_rows, head_dim);
  else
    state_merge_kernel<1><<<dim3((unsigned)n_rows), dim3(kMergeThreads), 0, stream>>>(
        part_out, part_lse, out, lse, n_parts, n_rows, head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

}  // extern "C"
