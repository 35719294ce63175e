// kamera_kernels.hip — gfx950 kernels of the Kamera reuse operator.
//
//   out(l, t, h, f) = [R(delta) src](l, t, h, f) + sum_r U(l, h, t, r) V(l, h, f, r)
//
// (technical summary of "Kamera: Unified Position-Invariant Multimodal KV Cache for
// Training-Free Reuse", §2 Methodology, reuse equation; R(delta) is the exact RoPE phase
// shift, the patch is added after it.) The result is stored through the page table into
// the destination pool.
//
// Two kernels:
//   * kamera_mfma_kernel  — bf16, windows of 64 or 128 features. The pass is HBM-bound: each
//     lane streams 16-byte pieces of token rows (several tiles in flight per wave),
//     rotates in fp32 with cos/sin from an LDS table, and, when a patch is present, lets one
//     bf16 MFMA per 16x16 output tile add U V^T onto the rotated values held in the
//     accumulator. The rows of the MFMA A operand (V) are permuted so that the accumulator a
//     lane receives covers exactly the features it loaded: 8 contiguous features per
//     32-feature run, which keeps both RoPE pair layouts lane-local and every load and store
//     16 bytes wide.
//   * kamera_valu_kernel  — fp32 (and bf16 shapes the MFMA path does not take): one thread
//     per pair of features, fp32 FMA for the patch.
//
// Lane map of the MFMA path (one wave, one 16-token tile of one window of width W):
//   lane = 16 g + n   (g = 0..3, n = 0..15): token t0 + n, features 32 r + 8 g + (0..7),
//   r = 0..W/32-1. MFMA tile T = 2 r + q holds, in accumulator i of lane (g, n), feature
//   32 r + 8 g + 4 q + i of token t0 + n (16x16x16 and 16x16x32 bf16 MFMAs share this
//   output layout: lane (g, n) holds rows 4g..4g+3 of column n).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kamera_internal.h"

namespace kamera {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr bool kNT = KAMERA_NONTEMPORAL != 0;
constexpr bool kNTLoad = kNT && (KAMERA_NT_MASK & 1);    // streamed row loads
constexpr bool kNTStore = kNT && (KAMERA_NT_MASK & 2);   // row stores

// Device-memory accesses go through address-space-1 pointers: the row pointers come from the
// job table, so the compiler cannot tell them from LDS and would otherwise emit FLAT
// instructions, whose completion also counts against the LDS wait counter and would make
// every LDS wait of the staging transpose drain the prefetched loads.
#define KGLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const KGLOBAL T* gp(const T* p) { return (const KGLOBAL T*)p; }
template <typename T>
__device__ __forceinline__ KGLOBAL T* gp(T* p) { return (KGLOBAL T*)p; }
// Row staging: global loads and stores use a row-contiguous lane map (each instruction covers
// whole 128-byte lines), and a padded wave-private LDS tile transposes rows to and from the
// MFMA lane map.
constexpr bool kStage = KAMERA_LDS_STAGE != 0;
constexpr int kStageRowBytes = 2 * 128 + 16;                // padded row of a 128-wide window
constexpr int kStageWaveBytes = kTileTokens * kStageRowBytes;

// Orders this wave's LDS accesses across lanes: writes before the fence are seen by reads
// after it (a wave's LDS operations complete in order; this stops the compiler reordering).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t shfl64(int64_t v, int src_lane) {
  const int lo = __shfl((int)(uint32_t)(uint64_t)v, src_lane, 64);
  const int hi = __shfl((int)(uint32_t)((uint64_t)v >> 32), src_lane, 64);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (RNE, hardware conversion) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)b);
  return lo | (hi << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Streamed 16-byte row pieces: read once, written once.
__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
  const KGLOBAL u32x4* q = gp(reinterpret_cast<const u32x4*>(p));
  if constexpr (kNTLoad) return __builtin_nontemporal_load(q);
  else return *q;
}
__device__ __forceinline__ void st_stream(uint16_t* p, u32x4 v) {
  KGLOBAL u32x4* q = gp(reinterpret_cast<u32x4*>(p));
  if constexpr (kNTStore) __builtin_nontemporal_store(v, q);
  else *q = v;
}

// Hardware block -> logical block. Blocks are dealt round-robin over the 8 XCDs, each with its
// own L2. mode 1: each XCD works through one contiguous range of logical blocks. mode T >= 2:
// runs of T consecutive logical blocks stay on one XCD and successive runs go round the XCDs,
// so neighbouring blocks (which share patch factors and page-table lines) meet in one L2 while
// heavy and light jobs stay spread over all XCDs; blocks past the last whole 8 T round keep
// their index.
__device__ __forceinline__ int remap_block(int b, int total, int mode) {
  if (mode <= 0) return b;
  const int xcd = b & 7, idx = b >> 3;
  if (mode == 1) {
    const int per = total >> 3, rem = total & 7;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  }
  const int full = total / (8 * mode) * (8 * mode);
  if (b >= full) return b;
  return ((idx / mode) * 8 + xcd) * mode + idx % mode;
}

// The job whose block range holds `blk`: block_starts is ascending, so the job index is the
// number of starts <= blk, minus one. One ballot over every 64th start finds the group of 64
// jobs, a second ballot the job inside it: two dependent loads however many jobs there are
// (up to 4096; more take one extra ballot per 4096).
__device__ __forceinline__ int find_job(const int32_t* block_starts, int n_jobs, int blk) {
  const int lane = threadIdx.x & 63;
  const KGLOBAL int32_t* bs = gp(block_starts);
  int groups = 0;
  for (int g0 = 0; 64 * g0 < n_jobs; g0 += 64) {
    const int gi = g0 + lane;
    const int c = __popcll(__ballot(64 * gi < n_jobs && bs[64 * gi] <= blk));
    groups += c;
    if (c < 64) break;
  }
  const int base = 64 * (groups - 1);
  const int j = base + lane;
  return base + __popcll(__ballot(j < n_jobs && bs[j] <= blk)) - 1;
}

// cos/sin(delta * theta^(-2i/rot_dim)) for every pair i: angle and range reduction in fp64,
// one rounding to fp32 each.
// The frequency is the model's table entry when one is given, else theta^(-2i/rot_dim); the
// shift is that of the pair's position component (multimodal sections), else the chunk's.
__device__ __forceinline__ void fill_phases(float2* cs, const JobDesc& J, const LaunchParams& P) {
  const int rot_dim = J.rot_dim;
  for (int i = threadIdx.x; i < rot_dim / 2; i += kBlockThreads) {
    const double inv = P.inv_freq ? gp(P.inv_freq)[i]
                                  : pow(P.theta, -2.0 * (double)i / (double)rot_dim);
    const int sec = P.pair_section ? (int)gp(P.pair_section)[i] : 0;
    const int64_t delta = sec == 0 ? J.delta : (sec == 1 ? J.delta_s1 : J.delta_s2);
    double s, c;
    sincos((double)delta * inv, &s, &c);
    cs[i] = make_float2((float)c, (float)s);
  }
}

__device__ __forceinline__ void count_fault(const LaunchParams& P) {
  __hip_atomic_fetch_add(gp(P.fault_counter), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Destination row (element offset of feature 0 of the row's first head) of logical token p,
// or -1 when the page-table entry is outside [0, n_pages).
__device__ __forceinline__ int64_t dst_row(const LaunchParams& P, int64_t p) {
  int64_t page, slot;
  if (P.page_shift >= 0) {
    page = p >> P.page_shift;
    slot = p & ((int64_t(1) << P.page_shift) - 1);
  } else {
    page = p / P.page_size;
    slot = p - page * P.page_size;
  }
  const int64_t phys = P.page_table ? (int64_t)gp(P.page_table)[page] : page;
  if (phys < 0 || phys >= P.n_pages) return -1;
  return (phys * P.page_size + slot) * P.pool_ts;
}

// ---------------------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------------------

// KM: 0 = no patch in the launch; 16 = one 16x16x16 step (m <= 16); 32 / 64 = one / two
// 16x16x32 steps (m <= 32 / 64), V operand in registers; -1 = streamed V, any m <= 256.
template <int KM>
struct KTraits {
  static constexpr bool k16 = KM == 16;
  static constexpr int s32 = KM == 32 ? 1 : (KM == 64 ? 2 : 0);
  static constexpr bool streamed = KM < 0;
};

template <int W, int KM>
struct TileIn {
  u32x4 raw[W / 32];   // token t0+n, features 32r + 8g .. +8 (row staging: row-map pieces)
  short4_t u16;                                       // B operand, KM == 16
  bf16x8 u32[KTraits<KM>::s32 > 0 ? KTraits<KM>::s32 : 1];  // B operand, KM == 32 / 64
  int64_t drow;                                       // destination element offset, -1 = skip
};

struct WindowCtx {
  const uint16_t* src;   // src of this layer/head/window, token 0, feature 0
  uint16_t* pool;        // pool of this layer, + head/window feature offset
  const uint16_t* U;     // U of this layer/head (row t at + t*m)
  const uint16_t* V;     // V of this layer/head, + window feature offset (row f at + f*m)
  uint8_t* stage;        // this wave's LDS tile (row staging)
  int64_t src_ts;
  int32_t n_tokens, dst_offset, m, vec_uv, rotate, copy, patch_mode, steps32;
};

// 8 consecutive bf16 of a U or V row starting at k0 (zeros past m).
__device__ __forceinline__ bf16x8 load_k8(const uint16_t* row, int k0, int m, int vec, bool nt) {
  if (vec) {
    if (k0 < m) {
      const KGLOBAL u32x4* q = gp(reinterpret_cast<const u32x4*>(row + k0));
      return __builtin_bit_cast(bf16x8, nt && kNT ? __builtin_nontemporal_load(q) : *q);
    }
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = (k0 + 2 * j < m) ? gp(row)[k0 + 2 * j] : 0u;
    const uint32_t b = (k0 + 2 * j + 1 < m) ? gp(row)[k0 + 2 * j + 1] : 0u;
    w[j] = a | (b << 16);
  }
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// 4 consecutive bf16 of a U or V row starting at k0 (zeros past m).
__device__ __forceinline__ short4_t load_k4(const uint16_t* row, int k0, int m, int vec) {
  if (vec) {
    if (k0 < m) return __builtin_bit_cast(short4_t, *gp(reinterpret_cast<const u32x2*>(row + k0)));
    return short4_t{0, 0, 0, 0};
  }
  short4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (k0 + j < m) ? (short)gp(row)[k0 + j] : (short)0;
  return r;
}

// Feature (within the window) that MFMA tile T row rho stands for: rows 4g..4g+3 of tile
// T = 2r + q land in lane group g as features 32r + 8g + 4q + (0..3).
__device__ __forceinline__ int tile_row_feature(int T, int rho) {
  return 32 * (T >> 1) + 8 * (rho >> 2) + 4 * (T & 1) + (rho & 3);
}

template <int W, int KM>
__device__ __forceinline__ void load_tile(const LaunchParams& P, const WindowCtx& C, int tile,
                                          int g, int n, TileIn<W, KM>& in) {
  constexpr int NR = W / 32;
  using K = KTraits<KM>;
  const int t = tile * kTileTokens + n;
  const bool valid = t < C.n_tokens;
  in.drow = valid ? dst_row(P, (int64_t)C.dst_offset + t) : -1;
  if constexpr (kStage) {
    // row map: instruction k, lane l -> token TPI*k + l/PR of the tile, 16-byte piece l%PR
    constexpr int PR = W / 8, TPI = 64 / PR;
    const int lane = threadIdx.x & 63;
    const int piece = lane % PR, tsub = lane / PR;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int tl = TPI * k + tsub;
      const int tt = tile * kTileTokens + tl;
      const uint16_t* row;
      if (C.patch_mode) {
        const int64_t d = shfl64(in.drow, tl);
        row = d >= 0 ? C.pool + d : nullptr;
      } else {
        row = C.src + (int64_t)tt * C.src_ts;
      }
      in.raw[k] = (tt < C.n_tokens && row != nullptr) ? ld_stream(row + 8 * piece)
                                                      : u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    const uint16_t* row = C.patch_mode ? (in.drow >= 0 ? C.pool + in.drow : nullptr)
                                       : C.src + (int64_t)t * C.src_ts;
    const bool have = valid && row != nullptr;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      in.raw[r] = have ? ld_stream(row + 32 * r + 8 * g) : u32x4{0u, 0u, 0u, 0u};
  }
  if constexpr (K::k16) {
    // the rank-class variants only run jobs whose U and V rows take 16-byte loads (the host
    // sends the others to the streamed variant), so no scalar fallback sits in the tile loop
    in.u16 = (valid && C.m > 0) ? load_k4(C.U + (int64_t)t * C.m, 4 * g, C.m, 1)
                                : short4_t{0, 0, 0, 0};
  }
  if constexpr (K::s32 > 0) {
#pragma unroll
    for (int s = 0; s < K::s32; ++s)
      in.u32[s] = (s < C.steps32 && valid)
                      ? load_k8(C.U + (int64_t)t * C.m, 32 * s + 8 * g, C.m, 1, true)
                      : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
}

template <int W, int KM>
struct VFrags {
  short4_t a16[KTraits<KM>::k16 ? W / 16 : 1];
  bf16x8 a32[KTraits<KM>::s32 > 0 ? KTraits<KM>::s32 : 1][KTraits<KM>::s32 > 0 ? W / 16 : 1];
};

template <int W, int KM>
__device__ __forceinline__ void load_vfrags(const WindowCtx& C, int g, int n, VFrags<W, KM>& vf) {
  constexpr int NT = W / 16;
  using K = KTraits<KM>;
  if (C.m == 0) return;
  if constexpr (K::k16) {
#pragma unroll
    for (int T = 0; T < NT; ++T)
      vf.a16[T] = load_k4(C.V + (int64_t)tile_row_feature(T, n) * C.m, 4 * g, C.m, 1);
  }
  if constexpr (K::s32 > 0) {
#pragma unroll
    for (int s = 0; s < K::s32; ++s)
#pragma unroll
      for (int T = 0; T < NT; ++T)
        vf.a32[s][T] = s < C.steps32 ? load_k8(C.V + (int64_t)tile_row_feature(T, n) * C.m,
                                               32 * s + 8 * g, C.m, 1, false)
                                     : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
}

// Rotate, patch, round and store one tile whose rows are in `in`.
template <int W, int KM>
__device__ __forceinline__ void compute_store(const LaunchParams& P, const WindowCtx& C,
                                              const float2* cs, const VFrags<W, KM>& vf,
                                              int tile, int g, int n, const TileIn<W, KM>& in) {
  constexpr int NR = W / 32;   // 32-feature runs per lane
  constexpr int NT = W / 16;   // MFMA tiles per window
  using K = KTraits<KM>;
  constexpr int PR = W / 8, TPI = 64 / PR;
  const int lane = threadIdx.x & 63;
  const int piece = lane % PR, tsub = lane / PR;
  constexpr int RS = 2 * W + 16;   // padded LDS row (bytes): conflict-free column reads
  u32x4 mraw[NR];                  // the tile in the MFMA lane map
  if constexpr (kStage) {
    if (!C.copy) {
#pragma unroll
      for (int k = 0; k < NR; ++k)
        *reinterpret_cast<u32x4*>(C.stage + (TPI * k + tsub) * RS + 16 * piece) = in.raw[k];
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < NR; ++r)
        mraw[r] = *reinterpret_cast<const u32x4*>(C.stage + n * RS + 64 * r + 16 * g);
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) mraw[r] = in.raw[r];
  }
  u32x4 out[NR];
  if (C.copy) {
#pragma unroll
    for (int r = 0; r < NR; ++r) out[r] = in.raw[r];   // either lane map: stored as loaded
  } else {
    float v[NR][8];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[r][2 * j] = bf_lo(mraw[r][j]);
        v[r][2 * j + 1] = bf_hi(mraw[r][j]);
      }
    }
    if (C.rotate) {
      if (P.layout != 0) {
        // interleaved: pair 16r + 4g + j owns features 32r + 8g + (2j, 2j+1)
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = v[r][2 * j], y = v[r][2 * j + 1];
            const float2 p = cs[16 * r + 4 * g + j];
            v[r][2 * j] = fmaf(x, p.x, -(y * p.y));
            v[r][2 * j + 1] = fmaf(y, p.x, x * p.y);
          }
      } else {
        // half-split: pair 32r + 8g + jj owns features (i, i + W/2) = runs r and r + NR/2
#pragma unroll
        for (int r = 0; r < NR / 2; ++r)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float x = v[r][jj], y = v[r + NR / 2][jj];
            const float2 p = cs[32 * r + 8 * g + jj];
            v[r][jj] = fmaf(x, p.x, -(y * p.y));
            v[r + NR / 2][jj] = fmaf(y, p.x, x * p.y);
          }
      }
    }
    if constexpr (KM != 0) {
      if (C.m > 0) {
        f32x4 acc[NT];
#pragma unroll
        for (int T = 0; T < NT; ++T)
          acc[T] = f32x4{v[T >> 1][4 * (T & 1)], v[T >> 1][4 * (T & 1) + 1],
                         v[T >> 1][4 * (T & 1) + 2], v[T >> 1][4 * (T & 1) + 3]};
        if constexpr (K::k16) {
#pragma unroll
          for (int T = 0; T < NT; ++T)
            acc[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf.a16[T], in.u16, acc[T], 0, 0, 0);
        } else if constexpr (K::s32 > 0) {
#pragma unroll
          for (int s = 0; s < K::s32; ++s) {
            if (s < C.steps32) {
#pragma unroll
              for (int T = 0; T < NT; ++T)
                acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf.a32[s][T], in.u32[s], acc[T],
                                                                 0, 0, 0);
            }
          }
        } else {
          // streamed: any m <= 256, both operands read per tile (V from L1/L2)
          const int t = tile * kTileTokens + n;
          const bool valid = t < C.n_tokens;
          for (int s = 0; s < C.steps32; ++s) {
            const bf16x8 b = valid ? load_k8(C.U + (int64_t)t * C.m, 32 * s + 8 * g, C.m,
                                             C.vec_uv, true)
                                   : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
            for (int T = 0; T < NT; ++T) {
              const bf16x8 a = load_k8(C.V + (int64_t)tile_row_feature(T, n) * C.m,
                                       32 * s + 8 * g, C.m, C.vec_uv, false);
              acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[T], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int T = 0; T < NT; ++T)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[T >> 1][4 * (T & 1) + i] = acc[T][i];
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
      out[r] = u32x4{pack_bf16(v[r][0], v[r][1]), pack_bf16(v[r][2], v[r][3]),
                     pack_bf16(v[r][4], v[r][5]), pack_bf16(v[r][6], v[r][7])};
  }

  const int t = tile * kTileTokens + n;
  if constexpr (kStage) {
    u32x4 orow[NR];
    if (C.copy) {
#pragma unroll
      for (int k = 0; k < NR; ++k) orow[k] = out[k];
    } else {
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < NR; ++r)
        *reinterpret_cast<u32x4*>(C.stage + n * RS + 64 * r + 16 * g) = out[r];
      wave_lds_sync();
#pragma unroll
      for (int k = 0; k < NR; ++k)
        orow[k] = *reinterpret_cast<const u32x4*>(C.stage + (TPI * k + tsub) * RS + 16 * piece);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int tl = TPI * k + tsub;
      const int64_t d = shfl64(in.drow, tl);
      if (tile * kTileTokens + tl < C.n_tokens && d >= 0) st_stream(C.pool + d + 8 * piece, orow[k]);
    }
    if (t < C.n_tokens && in.drow < 0 && g == 0) count_fault(P);
  } else {
    if (t < C.n_tokens) {
      if (in.drow >= 0) {
        uint16_t* row = C.pool + in.drow;
#pragma unroll
        for (int r = 0; r < NR; ++r) st_stream(row + 32 * r + 8 * g, out[r]);
      } else if (g == 0) {
        count_fault(P);
      }
    }
  }
}

// One wave's share of a block: one window, tiles [tile_lo, tile_hi). Every thread of the
// block calls this (the phase table barrier is inside); inactive waves only join the barrier.
template <int W, int KM>
__device__ __forceinline__ void run_window(const LaunchParams& P, const WindowCtx& C,
                                           const JobDesc& J, float2* cs, bool active,
                                           int tile_lo, int tile_hi) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  // tiles loaded ahead of the one computed, and the ring of tile buffers
  constexpr int kDepth = KM == 64 ? KAMERA_PREFETCH_TILES_RANK64 : KAMERA_PREFETCH_TILES;
  constexpr int R = kDepth + 1;

  VFrags<W, KM> vf;
  TileIn<W, KM> ring[R];
  if (active) {
    // first loads go out before the phase table is built, so their latency overlaps it
#pragma unroll
    for (int k = 0; k < kDepth; ++k)
      if (tile_lo + k < tile_hi) load_tile<W, KM>(P, C, tile_lo + k, g, n, ring[k]);
    if constexpr (KM != 0) load_vfrags<W, KM>(C, g, n, vf);
  }
  if (C.rotate) {
    fill_phases(cs, J, P);
    __syncthreads();
  }
  if (!active) return;

#if KAMERA_RING_SHIFT
  // one copy of the tile body; the ring advances by register moves
#pragma unroll 1
  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    if (tile + kDepth < tile_hi) load_tile<W, KM>(P, C, tile + kDepth, g, n, ring[kDepth]);
    compute_store<W, KM>(P, C, cs, vf, tile, g, n, ring[0]);
#pragma unroll
    for (int k = 0; k < kDepth; ++k) ring[k] = ring[k + 1];
  }
#else
  for (int base = tile_lo; base < tile_hi; base += R) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int tile = base + k;
      if (tile + kDepth < tile_hi)
        load_tile<W, KM>(P, C, tile + kDepth, g, n, ring[(k + kDepth) % R]);
      if (tile < tile_hi) compute_store<W, KM>(P, C, cs, vf, tile, g, n, ring[k]);
    }
  }
#endif
}

// Waves per SIMD the compiler must fit: the m <= 64 variant keeps 64 more registers of V
// operand and stays at 2; the others fit 3 once the accumulators live in VGPRs.
#if KAMERA_WAVES_PER_EU > 0
#define KAMERA_OCCUPANCY(KM) \
  __attribute__((amdgpu_waves_per_eu((KM) == 64 ? 2 : KAMERA_WAVES_PER_EU, 8)))
#else
#define KAMERA_OCCUPANCY(KM)
#endif

template <int W, int KM>
__global__ __launch_bounds__(kBlockThreads) KAMERA_OCCUPANCY(KM) void kamera_mfma_kernel(const LaunchParams P) {
  __shared__ float2 cs[64];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStage ? 4 * kStageWaveBytes : 16];
  const int blk = P.block_base + remap_block((int)blockIdx.x, P.total_blocks, P.xcd_remap);
  const JobDesc& J = P.jobs[find_job(P.block_starts, P.n_jobs, blk)];

  int local = blk - J.block_start;
  int tg, wg, layer;
  if (P.block_order == 0) {          // token groups fastest
    tg = local % J.n_tgroups;
    local /= J.n_tgroups;
    wg = local % J.n_wgroups;
    layer = local / J.n_wgroups;
  } else if (P.block_order == 1) {   // layers fastest
    layer = local % P.n_layers;
    local /= P.n_layers;
    wg = local % J.n_wgroups;
    tg = local / J.n_wgroups;
  } else {                           // window groups, then layers, token groups slowest
    wg = local % J.n_wgroups;
    local /= J.n_wgroups;
    layer = local % P.n_layers;
    tg = local / P.n_layers;
  }

  const int wave = threadIdx.x >> 6;
  const int nwin = min(4, J.n_windows - 4 * wg);
  const int sub = 4 / nwin;                       // waves sharing one window
  const bool active = wave < nwin * sub;
  const int win = 4 * wg + wave % nwin;
  const int part = wave / nwin;

  const int g_lo = (int)((int64_t)tg * J.n_tiles / J.n_tgroups);
  const int g_hi = (int)((int64_t)(tg + 1) * J.n_tiles / J.n_tgroups);
  const int tile_lo = g_lo + (g_hi - g_lo) * part / sub;
  const int tile_hi = g_lo + (g_hi - g_lo) * (part + 1) / sub;

  const int head = win / J.wph;
  const int f0 = (win % J.wph) * J.win_width;
  const int64_t feat = (int64_t)head * J.head_stride + f0;

  WindowCtx C;
  C.rotate = P.mode == MODE_PATCH ? 0 : J.rotate;
  C.src = J.src ? static_cast<const uint16_t*>(J.src) + layer * J.src_ls + feat : nullptr;
  C.pool = static_cast<uint16_t*>(J.pool) + layer * P.pool_ls + feat;
  C.U = J.m > 0 ? static_cast<const uint16_t*>(J.U) + layer * J.u_ls + head * J.u_hs : nullptr;
  C.V = J.m > 0 ? static_cast<const uint16_t*>(J.V) + layer * J.v_ls + head * J.v_hs +
                      (int64_t)f0 * J.m
                : nullptr;
  C.src_ts = J.src_ts;
  C.n_tokens = J.n_tokens;
  C.dst_offset = J.dst_offset;
  C.m = J.m;
  C.steps32 = (J.m + 31) / 32;
  C.vec_uv = J.vec_uv;
  C.copy = (!C.rotate && J.m == 0) ? 1 : 0;
  C.patch_mode = P.mode == MODE_PATCH;
  C.stage = stage + (kStage ? wave * kStageWaveBytes : 0);

  run_window<W, KM>(P, C, J, cs, active, tile_lo, tile_hi);
}

// ---------------------------------------------------------------------------------------
// VALU path
// ---------------------------------------------------------------------------------------

template <typename T> __device__ __forceinline__ float ld(const KGLOBAL T* p);
template <> __device__ __forceinline__ float ld<float>(const KGLOBAL float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const KGLOBAL uint16_t* p) {
  return bf16_to_f32(*p);
}
template <typename T> __device__ __forceinline__ void st(KGLOBAL T* p, float v);
template <> __device__ __forceinline__ void st<float>(KGLOBAL float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<uint16_t>(KGLOBAL uint16_t* p, float v) {
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void kamera_valu_kernel(const LaunchParams P) {
  __shared__ float2 cs[kMaxPairs];
  const int blk = P.block_base + remap_block((int)blockIdx.x, P.total_blocks, P.xcd_remap);
  const JobDesc& J = P.jobs[find_job(P.block_starts, P.n_jobs, blk)];

  int local = blk - J.block_start;
  const int tg = local % J.n_tgroups;
  local /= J.n_tgroups;
  const int wg = local % J.n_wgroups;
  const int layer = local / J.n_wgroups;

  const int rotate = P.mode == MODE_PATCH ? 0 : J.rotate;
  if (rotate) {
    fill_phases(cs, J, P);
    __syncthreads();
  }
  const bool interleaved = P.layout != 0;
  const int D = J.head_width;
  const int half = D / 2;
  const int h_lo = 4 * wg;
  const int nh = min(4, J.n_windows - h_lo);
  const int t_lo = (int)((int64_t)tg * J.n_tokens / J.n_tgroups);
  const int t_hi = (int)((int64_t)(tg + 1) * J.n_tokens / J.n_tgroups);
  const int nt = t_hi - t_lo;
  const int64_t items = (int64_t)nh * nt * half;
  const int m = J.m;

  const KGLOBAL T* src = gp(static_cast<const T*>(J.src));
  KGLOBAL T* pool = gp(static_cast<T*>(J.pool)) + layer * P.pool_ls;
  const KGLOBAL T* U = gp(static_cast<const T*>(J.U));
  const KGLOBAL T* V = gp(static_cast<const T*>(J.V));

  for (int64_t it = threadIdx.x; it < items; it += kBlockThreads) {
    const int q = (int)(it % half);
    const int64_t rest = it / half;
    const int t = t_lo + (int)(rest % nt);
    const int head = h_lo + (int)(rest / nt);
    // the two features this item owns
    int fa, fb;
    if (rotate && !interleaved) { fa = q; fb = q + half; } else { fa = 2 * q; fb = 2 * q + 1; }

    const int64_t drow = dst_row(P, (int64_t)J.dst_offset + t);
    if (drow < 0) {
      if (q == 0) count_fault(P);
      continue;
    }
    KGLOBAL T* out = pool + drow + (int64_t)head * J.head_stride;
    const KGLOBAL T* in = P.mode == MODE_PATCH ? out
                                       : src + layer * J.src_ls + (int64_t)t * J.src_ts +
                                             (int64_t)head * J.head_stride;
    if (!rotate && m == 0) {   // bit copy through an integer type of the element's width
      using Bits = std::conditional_t<sizeof(T) == 4, uint32_t, uint16_t>;
      const KGLOBAL Bits* ib = reinterpret_cast<const KGLOBAL Bits*>(in);
      KGLOBAL Bits* ob = reinterpret_cast<KGLOBAL Bits*>(out);
      ob[fa] = ib[fa];
      ob[fb] = ib[fb];
      continue;
    }
    float xa = ld<T>(in + fa), xb = ld<T>(in + fb);
    if (rotate) {
      const float2 p = cs[q];
      const float ra = fmaf(xa, p.x, -(xb * p.y));
      const float rb = fmaf(xb, p.x, xa * p.y);
      xa = ra;
      xb = rb;
    }
    if (m > 0) {
      const KGLOBAL T* urow = U + layer * J.u_ls + head * J.u_hs + (int64_t)t * m;
      const KGLOBAL T* vbase = V + layer * J.v_ls + head * J.v_hs;
      float pa = 0.f, pb = 0.f;
      for (int r = 0; r < m; ++r) {
        const float u = ld<T>(urow + r);
        pa = fmaf(u, ld<T>(vbase + (int64_t)fa * m + r), pa);
        pb = fmaf(u, ld<T>(vbase + (int64_t)fb * m + r), pb);
      }
      xa += pa;
      xb += pb;
    }
    st<T>(out + fa, xa);
    st<T>(out + fb, xb);
  }
}

}  // namespace

template <int W>
void launch_mfma_w(const LaunchParams& p, int kmode, hipStream_t stream) {
  const dim3 grid(p.total_blocks), block(kBlockThreads);
  switch (kmode) {
    case 0: hipLaunchKernelGGL((kamera_mfma_kernel<W, 0>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((kamera_mfma_kernel<W, 16>), grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL((kamera_mfma_kernel<W, 32>), grid, block, 0, stream, p); break;
    case 64: hipLaunchKernelGGL((kamera_mfma_kernel<W, 64>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((kamera_mfma_kernel<W, -1>), grid, block, 0, stream, p); break;
  }
}

hipError_t launch_mfma(const LaunchParams& p, int win_width, int kmode, hipStream_t stream) {
  if (win_width == 128) launch_mfma_w<128>(p, kmode, stream);
  else launch_mfma_w<64>(p, kmode, stream);
  return hipGetLastError();
}

hipError_t launch_valu(const LaunchParams& p, int dtype, hipStream_t stream) {
  const dim3 grid(p.total_blocks), block(kBlockThreads);
  if (dtype == 0) hipLaunchKernelGGL(kamera_valu_kernel<float>, grid, block, 0, stream, p);
  else hipLaunchKernelGGL(kamera_valu_kernel<uint16_t>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace kamera
