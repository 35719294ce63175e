// kamera_internal.h — types shared by the reuse path's host runtime (kamera_api.cpp) and its
// kernels (kamera_kernels.hip), and the workspace layout constants. Not part of the public
// ABI. Host helpers shared by every entry point are in kamera_host.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kamera.h"

namespace kamera {

// One unit of work packed by the host: one chunk, one channel, every layer.
// The kernels split it into blocks of (layer, window group, token group).
struct alignas(16) JobDesc {
  const void* src;   // canonical rows of the channel (unused in patch-only mode)
  const void* U;     // patch factors (m > 0)
  const void* V;
  void* pool;        // destination pool of the channel
  int64_t src_ls;    // src layer stride (elements)
  int64_t src_ts;    // src token stride
  int64_t u_ls, u_hs;
  int64_t v_ls, v_hs;
  int64_t delta;       // shift of section 0 (of every pair when the model has no sections)
  int64_t delta_s1;    // shifts of sections 1 and 2
  int64_t delta_s2;
  int32_t n_tokens;
  int32_t dst_offset;
  int32_t m;
  int32_t rotate;      // 1: R(delta) on this job's features
  int32_t head_width;  // features per head this job covers (src, pool, V already offset to them)
  int32_t head_stride; // features between consecutive heads of the channel's rows
  int32_t win_width;   // features one wave handles at a time (a window of a head)
  int32_t wph;         // windows per head
  int32_t n_windows;   // heads * wph
  int32_t n_wgroups;   // windows are taken 4 at a time (one per wave)
  int32_t n_tgroups;   // token groups
  int32_t n_tiles;     // token tiles (16 tokens on the MFMA path, 1 token on the VALU path)
  int32_t block_start; // first block of this job in the launch
  int32_t vec_uv;      // U and V rows may be read with 16-byte loads
  int32_t rot_dim;     // length of the frequency ladder (2 x pairs)
  int32_t pad0;
};

enum Mode : int32_t { MODE_REUSE = 0, MODE_PATCH = 1 };

struct LaunchParams {
  const JobDesc* jobs;      // device (inside the workspace)
  const int32_t* block_starts;  // device: jobs[i].block_start, compact (one int per job)
  int32_t n_jobs;
  int32_t total_blocks;
  int32_t block_base;       // block_start of jobs[0]: job block ranges are offset by it
  const int32_t* page_table;
  int32_t n_logical_pages;
  int32_t page_size;
  int32_t page_shift;       // log2(page_size) when it is a power of two, else -1
  int32_t n_pages;
  int32_t layout;           // kamera_rope_layout
  int64_t pool_ls;          // pool layer stride (elements)
  int64_t pool_ts;          // pool token stride
  double theta;
  const double* inv_freq;       // device (workspace): rot_dim/2 frequencies, or NULL (ladder)
  const uint8_t* pair_section;  // device (workspace): section of each pair, or NULL
  uint32_t* fault_counter;  // device (workspace header)
  int32_t mode;             // Mode
  int32_t n_layers;
  int32_t block_order;      // MFMA path: how a job's blocks map to (layer, window group, tokens)
  int32_t xcd_remap;        // 0: none; 1: contiguous range per XCD; T >= 2: runs of T blocks
};

// Kernel geometry
constexpr int kBlockThreads = 256;      // 4 waves of 64
constexpr int kTileTokens = 16;         // MFMA N dimension
constexpr int kValuTokensPerBlock = 64; // tokens per block on the VALU path (at most)
constexpr int kValuMinBlocks = 1024;    // fewer tokens per block until a VALU launch has this many
constexpr int kMaxPairs = 512;          // LDS phase table (rot_dim <= 1024)
// Workspace front: [header (fault counter) | inv_freq table (kMaxPairs doubles) |
// pair sections (kMaxPairs bytes) | job tables ...]
constexpr size_t kHeaderBytes = 256;
constexpr size_t kFreqOffset = kHeaderBytes;
constexpr size_t kSectionOffset = kFreqOffset + kMaxPairs * sizeof(double);
constexpr size_t kTablesEnd = kSectionOffset + kMaxPairs;

// Build-time knobs; the defaults are the measured best on MI355X.
//   KAMERA_PREFETCH_TILES(_RANK64): tiles a wave keeps loaded ahead of the one it computes
//     (ring of PREFETCH+1 tile buffers in registers). Deeper rings cost occupancy and did
//     not pay.
//   KAMERA_NONTEMPORAL: streamed rows use nontemporal loads and stores (pays only once rows
//     are staged: half-line accesses defeat L2 merging).
//   KAMERA_LDS_STAGE: rows go through a padded LDS tile so every global access instruction
//     covers whole 128-byte lines.
//   KAMERA_RING_SHIFT: one copy of the tile body per loop iteration, the ring advancing by
//     register moves (instead of one unrolled body per ring slot).
//   KAMERA_WAVES_PER_EU: occupancy the compiler is asked to fit (0 = its own choice). At 3 the
//     m <= 16 and m <= 32 variants keep their accumulators in VGPRs and fit 3 waves per SIMD
//     (measured +2 % at m = 16, neutral elsewhere); the m <= 64 variant stays at 2.
#ifndef KAMERA_PREFETCH_TILES
#define KAMERA_PREFETCH_TILES 1
#endif
#ifndef KAMERA_PREFETCH_TILES_RANK64
#define KAMERA_PREFETCH_TILES_RANK64 1
#endif
#ifndef KAMERA_NONTEMPORAL
#define KAMERA_NONTEMPORAL 1
#endif
#ifndef KAMERA_NT_MASK
#define KAMERA_NT_MASK 3   // bit 0: nontemporal row loads, bit 1: nontemporal row stores
#endif
#ifndef KAMERA_LDS_STAGE
#define KAMERA_LDS_STAGE 1
#endif
#ifndef KAMERA_RING_SHIFT
#define KAMERA_RING_SHIFT 1
#endif
#ifndef KAMERA_WAVES_PER_EU
#define KAMERA_WAVES_PER_EU 3
#endif

// One launch covers jobs of one window width (64 or 128). kmode: largest rank in the launch,
// rounded up: 0 (no patch), 16, 32 or 64 keep the V operand in registers; -1 streams it from
// memory for any m <= 256.
hipError_t launch_mfma(const LaunchParams& p, int win_width, int kmode, hipStream_t stream);
// dtype: 0 = fp32, 1 = bf16
hipError_t launch_valu(const LaunchParams& p, int dtype, hipStream_t stream);

// kamera_reuse_batch with its device tables at `tables` (tables_bytes long, 256-byte aligned)
// and no staging set-up (kamera_api.cpp).
kamera_status reuse_batch_tables_at(const kamera_model* model, const kamera_cache* cache,
                                    const kamera_chunk* chunks, int32_t n_chunks, void* tables,
                                    size_t tables_bytes, void* stream);
// Looks up this device's copy of the no-allocation entry point's scratch array (once per
// device; kamera_noalloc.hip). Called by kamera_init().
kamera_status scratch_setup();

}  // namespace kamera
