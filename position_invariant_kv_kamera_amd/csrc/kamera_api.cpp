// kamera_api.cpp — host runtime behind include/kamera.h: argument validation, work packing
// and kernel launch. Every check runs before anything is enqueued (the optional deep check of
// the page table only reads it), so a rejected call has no side effect on the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kamera.h"
#include "kamera_host.h"
#include "kamera_internal.h"

using kamera::JobDesc;
using kamera::LaunchParams;

using kamera::kHeaderBytes;
using kamera::kFreqOffset;
using kamera::kSectionOffset;
using kamera::kTablesEnd;
using namespace kamera::host;

namespace {

// Largest grid of one launch: 2^23 blocks of 256 threads keeps the work-item count of the
// dispatch (a 32-bit quantity) below 2^31.
constexpr int64_t kMaxGridBlocks = int64_t(1) << 23;

enum class Op { Reuse, Relocate, Patch };

kamera_status validate_chunks(const kamera_model& m, const kamera_cache& c,
                              const kamera_chunk* chunks, int32_t n_chunks, Op op) {
  if (n_chunks < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_chunks must be >= 0");
  if (n_chunks > 0 && !chunks) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunks is NULL");
  const int64_t es = m.dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  const int64_t capacity = (int64_t)c.n_logical_pages * c.page_size;
  const int64_t slots = (int64_t)c.n_pages * c.page_size;
  Range pools[2];
  for (int ch = 0; ch < 2; ++ch) {
    const Channel g = channel_of(m, ch);
    pools[ch] = view_range(c.pool[ch], c.layer_stride, m.n_layers, c.token_stride, slots,
                           (int64_t)g.heads * g.width, es);
  }
  std::vector<std::pair<int64_t, int64_t>> spans;
  spans.reserve(n_chunks);
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_chunk& k = chunks[i];
    if (k.n_tokens < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: n_tokens < 0", i);
    if (k.n_tokens == 0) continue;
    if (k.dst_token_offset < 0)
      return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: dst_token_offset < 0", i);
    if ((int64_t)k.dst_token_offset + k.n_tokens > capacity)
      return fail(KAMERA_ERR_INVALID_ARGUMENT,
                  "chunk %d: tokens [%d, %lld) run past the cache's %lld logical tokens", i,
                  k.dst_token_offset, (long long)k.dst_token_offset + k.n_tokens,
                  (long long)capacity);
    if (op != Op::Patch) {
      auto big = [](int64_t d) { return d >= (int64_t(1) << 31) || d <= -(int64_t(1) << 31); };
      if (big(k.delta)) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d: |delta| must be < 2^31", i);
      for (int sct = 1; sct < m.n_sections; ++sct)
        if (big(k.delta_sections[sct - 1]))
          return fail(KAMERA_ERR_INVALID_ARGUMENT,
                      "chunk %d: |delta_sections[%d]| must be < 2^31", i, sct - 1);
    }
    spans.emplace_back(k.dst_token_offset, (int64_t)k.dst_token_offset + k.n_tokens);
    for (int ch = 0; ch < 2; ++ch) {
      const Channel g = channel_of(m, ch);
      const int64_t row = (int64_t)g.heads * g.width;
      if (op != Op::Patch) {
        const kamera_src& s = k.src[ch];
        if (!s.ptr) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: src is NULL", i, ch);
        if (s.layer_stride < 0 || s.token_stride < row)
          return fail(KAMERA_ERR_INVALID_ARGUMENT,
                      "chunk %d channel %d: src token_stride %lld shorter than the row (%lld)",
                      i, ch, (long long)s.token_stride, (long long)row);
        const Range sr = view_range(s.ptr, s.layer_stride, m.n_layers, s.token_stride,
                                    k.n_tokens, row, es);
        if (overlaps(sr, pools[0]) || overlaps(sr, pools[1]))
          return fail(KAMERA_ERR_OVERLAP, "chunk %d channel %d: src overlaps the cache", i, ch);
      }
      const kamera_patch_ref& p = k.patch[ch];
      if (op == Op::Relocate) continue;
      if (p.m < 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: m < 0", i, ch);
      if (p.m > KAMERA_MAX_RANK)
        return fail(KAMERA_ERR_UNSUPPORTED, "chunk %d channel %d: m = %d exceeds %d", i, ch,
                    p.m, KAMERA_MAX_RANK);
      if (p.m == 0) continue;
      if (!p.U || !p.V)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: m > 0 but U or V is NULL",
                    i, ch);
      if (p.u_layer_stride < 0 || p.u_head_stride < 0 || p.v_layer_stride < 0 ||
          p.v_head_stride < 0)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "chunk %d channel %d: negative patch stride", i, ch);
      // U: layers x heads x (n_tokens x m); V: layers x heads x (width x m)
      const Range ur = view_range(p.U, p.u_layer_stride, m.n_layers, p.u_head_stride, g.heads,
                                  (int64_t)k.n_tokens * p.m, es);
      const Range vr = view_range(p.V, p.v_layer_stride, m.n_layers, p.v_head_stride, g.heads,
                                  (int64_t)g.width * p.m, es);
      if (overlaps(ur, pools[0]) || overlaps(ur, pools[1]) || overlaps(vr, pools[0]) ||
          overlaps(vr, pools[1]))
        return fail(KAMERA_ERR_OVERLAP, "chunk %d channel %d: patch factors overlap the cache",
                    i, ch);
    }
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second)
      return fail(KAMERA_ERR_INVALID_ARGUMENT,
                  "two chunks write logical cache token %lld", (long long)spans[i].first);
  return KAMERA_OK;
}

// Deep validation (environment variable KAMERA_VALIDATE non-zero): the page table lives in
// device memory, so the argument checks above cannot see its entries. This copies it to the
// host (after the stream's earlier work, which may have written it) and checks that every
// logical page a chunk writes maps into [0, n_pages) and that no two written tokens share a
// physical slot. It synchronises the stream, so it refuses a capturing one. Nothing is
// written to the device.
kamera_status validate_table_contents(const kamera_cache& c, const kamera_chunk* chunks,
                                      int32_t n_chunks, hipStream_t stream) {
  if (!c.page_table) return KAMERA_OK;   // identity table: checked against n_pages already
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(KAMERA_ERR_UNSUPPORTED,
                "KAMERA_VALIDATE reads the page table and synchronises; the stream is capturing");
  std::vector<int32_t> table(c.n_logical_pages);
  e = hipMemcpyAsync(table.data(), c.page_table, table.size() * sizeof(int32_t),
                     hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(KAMERA_ERR_HIP, "reading the page table: %s", hipGetErrorString(e));
  struct Use {
    int32_t phys, slot_lo, slot_hi, logical, chunk;
  };
  std::vector<Use> uses;
  const int32_t ps = c.page_size;
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_chunk& k = chunks[i];
    if (k.n_tokens <= 0) continue;
    const int64_t first = k.dst_token_offset, end = first + k.n_tokens;
    for (int64_t lp = first / ps; lp * ps < end; ++lp) {
      const int32_t phys = table[lp];
      if (phys < 0 || phys >= c.n_pages)
        return fail(KAMERA_ERR_INVALID_ARGUMENT,
                    "chunk %d: page_table[%lld] = %d is outside [0, %d)", i, (long long)lp, phys,
                    c.n_pages);
      const int64_t lo = std::max(first, lp * ps), hi = std::min(end, (lp + 1) * ps);
      uses.push_back({phys, (int32_t)(lo - lp * ps), (int32_t)(hi - lp * ps), (int32_t)lp, i});
    }
  }
  std::sort(uses.begin(), uses.end(), [](const Use& a, const Use& b) {
    return a.phys != b.phys ? a.phys < b.phys : a.slot_lo < b.slot_lo;
  });
  for (size_t j = 1; j < uses.size(); ++j) {
    const Use &a = uses[j - 1], &b = uses[j];
    if (a.phys == b.phys && b.slot_lo < a.slot_hi)
      return fail(KAMERA_ERR_INVALID_ARGUMENT,
                  "logical pages %d (chunk %d) and %d (chunk %d) both write slot %d of physical "
                  "page %d",
                  a.logical, a.chunk, b.logical, b.chunk, b.slot_lo, b.phys);
  }
  return KAMERA_OK;
}



// ---------------------------------------------------------------------------------------
// packing
// ---------------------------------------------------------------------------------------

struct Plan {
  std::vector<JobDesc> mfma, valu;
  int mfma_max_m = 0;
  int xcd_remap = 0;   // LaunchParams::xcd_remap of the MFMA launches
  int64_t mfma_blocks = 0, valu_blocks = 0;
};

// Kernel variant for the largest rank in an MFMA launch (see launch_mfma).
int kmode_for(int max_m) {
  if (max_m == 0) return 0;
  if (max_m <= 16) return 16;
  if (max_m <= 32) return 32;
  if (max_m <= 64) return 64;
  return -1;
}

// Can this job use the MFMA path? Sets the window width.
bool mfma_eligible(const kamera_model& m, const kamera_cache& c, const kamera_chunk& k,
                   const Channel& g, Op op, int ch, int f_base, int* win_width) {
  if (m.dtype != KAMERA_DTYPE_BF16) return false;
  if (env_int("KAMERA_FORCE_VALU", 0)) return false;
  int w;
  if (g.rotate && op != Op::Patch) {
    if (g.width != 64 && g.width != 128) return false;
    w = g.width;
  } else if (g.width % 128 == 0) {
    w = 128;
  } else if (g.width % 64 == 0) {
    w = 64;
  } else {
    return false;
  }
  // 16-byte loads and stores of token rows (of the job's sub-head, and of every head)
  const int64_t off = (int64_t)f_base * 2;
  if (f_base % 8 || channel_of(m, ch).width % 8) return false;
  if (!aligned16(static_cast<const uint8_t*>(c.pool[ch]) + off) || c.layer_stride % 8 ||
      c.token_stride % 8)
    return false;
  if (op != Op::Patch) {
    const kamera_src& s = k.src[ch];
    if (!aligned16(static_cast<const uint8_t*>(s.ptr) + off) || s.layer_stride % 8 ||
        s.token_stride % 8)
      return false;
  }
  *win_width = w;
  return true;
}

kamera_status build_plan(const kamera_model& m, const kamera_cache& c, const kamera_chunk* chunks,
                         int32_t n_chunks, Op op, Plan* plan) {
  const int64_t es = m.dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  for (int32_t i = 0; i < n_chunks; ++i) {
    const kamera_chunk& k = chunks[i];
    if (k.n_tokens == 0) continue;
    for (int ch = 0; ch < 2; ++ch) {
      const Channel g = channel_of(m, ch);
      const kamera_patch_ref& p = k.patch[ch];
      const int mm = op == Op::Relocate ? 0 : p.m;
      if (op == Op::Patch && mm == 0) continue;
      // A partially rotary key head is two jobs: features [0, rope_dim) turn, the rest pass
      // through. Each job sees its sub-head through offset pointers and the head stride.
      const bool partial = g.rotate && m.family == KAMERA_FAMILY_GQA && m.rope_dim < g.width;
      const int n_parts = partial ? 2 : 1;
      for (int part = 0; part < n_parts; ++part) {
        const int f_base = part == 0 ? 0 : m.rope_dim;
        const int width = partial ? (part == 0 ? m.rope_dim : g.width - m.rope_dim) : g.width;
        const bool rot = g.rotate && part == 0;
        JobDesc j;
        std::memset(&j, 0, sizeof j);
        j.src = op == Op::Patch ? nullptr
                                : static_cast<const uint8_t*>(k.src[ch].ptr) + f_base * es;
        j.src_ls = op == Op::Patch ? 0 : k.src[ch].layer_stride;
        j.src_ts = op == Op::Patch ? 0 : k.src[ch].token_stride;
        j.pool = static_cast<uint8_t*>(c.pool[ch]) + f_base * es;
        j.m = mm;
        if (mm > 0) {
          j.U = p.U;
          j.V = static_cast<const uint8_t*>(p.V) + (int64_t)f_base * mm * es;
          j.u_ls = p.u_layer_stride;
          j.u_hs = p.u_head_stride;
          j.v_ls = p.v_layer_stride;
          j.v_hs = p.v_head_stride;
        }
        j.delta = k.delta;
        j.delta_s1 = m.n_sections > 1 ? k.delta_sections[0] : k.delta;
        j.delta_s2 = m.n_sections > 2 ? k.delta_sections[1] : k.delta;
        j.n_tokens = k.n_tokens;
        j.dst_offset = k.dst_token_offset;
        j.rotate = (rot && op != Op::Patch) ? 1 : 0;
        j.head_width = width;
        j.head_stride = g.width;
        j.rot_dim = m.rope_dim;
        const Channel sub{g.heads, width, rot};
        int w = 0;
        if (mfma_eligible(m, c, k, sub, op, ch, f_base, &w)) {
          j.win_width = w;
          j.wph = width / w;
          j.n_windows = g.heads * j.wph;
          j.n_wgroups = (j.n_windows + 3) / 4;
          j.n_tiles = (k.n_tokens + kamera::kTileTokens - 1) / kamera::kTileTokens;
          // n_tgroups is set below, once the whole batch's size is known
          j.vec_uv = mm > 0 && mm % 8 == 0 && aligned16(j.U) && aligned16(j.V) &&
                     p.u_layer_stride % 8 == 0 && p.u_head_stride % 8 == 0 &&
                     p.v_layer_stride % 8 == 0 && p.v_head_stride % 8 == 0;
          plan->mfma.push_back(j);
          plan->mfma_max_m = std::max(plan->mfma_max_m, mm);
        } else {
          j.win_width = width;
          j.wph = 1;
          j.n_windows = g.heads;
          j.n_wgroups = (g.heads + 3) / 4;
          j.n_tiles = k.n_tokens;   // n_tgroups is set below, as for the MFMA jobs
          plan->valu.push_back(j);
        }
      }
    }
  }
  // Token groups of the MFMA jobs: each wave gets `tpw` tiles of one window. Short waves
  // (many small blocks) keep the chip evenly loaded to the end; but every block reloads its V
  // operand (16 KB per window at m = 64), so rank > 32 takes long waves. Measured on MI355X:
  // 4 tiles for m <= 32 (2 and 8 tiles were 1-7 % slower, 16 and 32 up to 8 %), 32 for
  // m <= 64 (4 tiles: -18 %); larger only when the grid would exceed kMaxGridBlocks.
  // With the short-wave default of 4 tiles, a job whose tile count splits evenly into 3s but
  // not into 4s takes 3 (81-tile chunks of 1296 tokens: 27 equal token groups instead of 21
  // of 3 or 4 tiles).
  const int even_tpw = env_int("KAMERA_EVEN_TPW", 1);
  auto tgroups = [even_tpw](const JobDesc& j, int64_t tpw) {
    const int64_t sub = 4 / std::min(4, j.n_windows);
    const int64_t t = (even_tpw && tpw == 4 && sub == 1 && j.n_tiles % 4 != 0 &&
                       j.n_tiles % 3 == 0) ? 3 : tpw;
    return std::max<int64_t>(1, (j.n_tiles + t * sub - 1) / (t * sub));
  };
  auto blocks_at = [&](int64_t tpw) {
    int64_t b = 0;
    for (const JobDesc& j : plan->mfma) b += (int64_t)m.n_layers * j.n_wgroups * tgroups(j, tpw);
    return b;
  };
  int64_t tpw = plan->mfma_max_m > 32 ? 32 : 4;
  tpw = std::max(1, env_int("KAMERA_TILES_PER_WAVE", (int)tpw));
  while (tpw < (int64_t(1) << 30) && blocks_at(tpw) > kMaxGridBlocks) tpw *= 2;
  for (JobDesc& j : plan->mfma) j.n_tgroups = (int32_t)tgroups(j, tpw);
  // Short waves mean many blocks per (layer, window group), each loading the same V operand:
  // runs of 4 blocks kept on one XCD then find it in that XCD's L2 (measured +1 % on 4 KV
  // heads x 1296-token chunks at m = 16, neutral at m = 32; with long waves it cost 1-5 %).
  plan->xcd_remap = env_int("KAMERA_XCD_REMAP", tpw <= 4 ? 4 : 0);
  // VALU token groups: up to kValuTokensPerBlock tokens per block, fewer while the launch
  // would have under kValuMinBlocks blocks (a thread walks its items one after another, so a
  // small batch on a few blocks is one long latency chain; results do not depend on it).
  auto valu_blocks_at = [&](int64_t tpb) {
    int64_t b = 0;
    for (const JobDesc& j : plan->valu)
      b += (int64_t)m.n_layers * j.n_wgroups * ((j.n_tiles + tpb - 1) / tpb);
    return b;
  };
  int64_t tpb = kamera::kValuTokensPerBlock;
  while (tpb > 1 && valu_blocks_at(tpb) < kamera::kValuMinBlocks) tpb /= 2;
  for (JobDesc& j : plan->valu) j.n_tgroups = (int32_t)std::max<int64_t>(1, (j.n_tiles + tpb - 1) / tpb);

  // grouped by window width (one launch each), heaviest jobs first inside a group so that a
  // mixed batch does not end on a tail of patched work
  auto heavier = [](const JobDesc& a, const JobDesc& b) {
    if (a.win_width != b.win_width) return a.win_width > b.win_width;
    return a.m > b.m;
  };
  std::stable_sort(plan->mfma.begin(), plan->mfma.end(), heavier);
  std::stable_sort(plan->valu.begin(), plan->valu.end(), heavier);
  auto assign = [&](std::vector<JobDesc>& jobs, int64_t* total) -> bool {
    // block_start counts from the first job of the vector; a launch over a sub-range of it
    // numbers its blocks from that range's first start (LaunchParams::block_base)
    int64_t b = 0;
    for (JobDesc& j : jobs) {
      j.block_start = (int32_t)b;
      b += (int64_t)m.n_layers * j.n_wgroups * j.n_tgroups;
      if (b > kMaxGridBlocks) return false;
    }
    *total = b;
    return true;
  };
  if (!assign(plan->mfma, &plan->mfma_blocks) || !assign(plan->valu, &plan->valu_blocks))
    return fail(KAMERA_ERR_UNSUPPORTED,
                "batch needs more than 2^23 blocks in one launch: split it into smaller calls");
  return KAMERA_OK;
}

// The reuse path: validation, planning, table upload and launches. The device tables go to
// `workspace` (the caller's, or the no-allocation entry point's static scratch); with
// allow_setup false the upload refuses to set up a staging ring that kamera_init() did not.
kamera_status run(const kamera_model* model, const kamera_cache* cache, const kamera_chunk* chunks,
                  int32_t n_chunks, void* workspace, size_t workspace_bytes, void* stream_ptr,
                  Op op, bool allow_setup = true) {
  clear_error();
  kamera_status st = validate_model(model);
  if (st != KAMERA_OK) return st;
  st = validate_cache(*model, cache);
  if (st != KAMERA_OK) return st;
  st = validate_chunks(*model, *cache, chunks, n_chunks, op);
  if (st != KAMERA_OK) return st;
  if (!workspace) return fail(KAMERA_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(KAMERA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = kamera_workspace_bytes(n_chunks);
  if (workspace_bytes < need)
    return fail(KAMERA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (env_int("KAMERA_VALIDATE", 0)) {
    st = validate_table_contents(*cache, chunks, n_chunks, stream);
    if (st != KAMERA_OK) return st;
  }

  Plan plan;
  st = build_plan(*model, *cache, chunks, n_chunks, op, &plan);
  if (st != KAMERA_OK) return st;

  // workspace: [header | inv_freq | pair sections | MFMA jobs | VALU jobs | MFMA block starts |
  //             VALU block starts]
  const size_t mfma_off = kTablesEnd;
  const size_t valu_off = mfma_off + plan.mfma.size() * sizeof(JobDesc);
  const size_t mfma_bs_off = valu_off + plan.valu.size() * sizeof(JobDesc);
  const size_t valu_bs_off = mfma_bs_off + plan.mfma.size() * sizeof(int32_t);
  const size_t bytes = valu_bs_off + plan.valu.size() * sizeof(int32_t);
  std::vector<uint8_t> staging(bytes, 0);
  auto put = [&](size_t off, const std::vector<JobDesc>& jobs, size_t bs_off) {
    if (jobs.empty()) return;
    std::memcpy(staging.data() + off, jobs.data(), jobs.size() * sizeof(JobDesc));
    for (size_t i = 0; i < jobs.size(); ++i)
      std::memcpy(staging.data() + bs_off + i * sizeof(int32_t), &jobs[i].block_start,
                  sizeof(int32_t));
  };
  put(mfma_off, plan.mfma, mfma_bs_off);
  put(valu_off, plan.valu, valu_bs_off);
  const int pairs = model->rope_dim / 2;
  if (model->inv_freq)
    std::memcpy(staging.data() + kFreqOffset, model->inv_freq, pairs * sizeof(double));
  if (model->pair_section)
    std::memcpy(staging.data() + kSectionOffset, model->pair_section, pairs);

  st = upload(staging, workspace, stream, allow_setup);
  if (st != KAMERA_OK) return st;

  LaunchParams lp;
  std::memset(&lp, 0, sizeof lp);
  lp.page_table = cache->page_table;
  lp.n_logical_pages = cache->n_logical_pages;
  lp.page_size = cache->page_size;
  lp.page_shift = -1;
  for (int b = 0; b < 31; ++b)
    if (cache->page_size == (1 << b)) lp.page_shift = b;
  lp.n_pages = cache->n_pages;
  lp.layout = model->rope_layout;
  lp.pool_ls = cache->layer_stride;
  lp.pool_ts = cache->token_stride;
  lp.theta = model->rope_theta;
  lp.inv_freq = model->inv_freq
                    ? reinterpret_cast<const double*>(static_cast<uint8_t*>(workspace) + kFreqOffset)
                    : nullptr;
  lp.pair_section = model->pair_section ? static_cast<uint8_t*>(workspace) + kSectionOffset
                                        : nullptr;
  lp.fault_counter = static_cast<uint32_t*>(workspace);
  lp.mode = op == Op::Patch ? kamera::MODE_PATCH : kamera::MODE_REUSE;
  lp.xcd_remap = plan.xcd_remap;
  lp.n_layers = model->n_layers;
  lp.block_order = env_int("KAMERA_BLOCK_ORDER", 0);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // MFMA jobs: one launch per window width (jobs are grouped by width in build_plan)
  for (size_t lo = 0; lo < plan.mfma.size();) {
    size_t hi = lo;
    int max_m = 0;
    bool scalar_uv = false;   // a patched job whose U or V rows cannot take 16-byte loads
    while (hi < plan.mfma.size() && plan.mfma[hi].win_width == plan.mfma[lo].win_width) {
      scalar_uv |= plan.mfma[hi].m > 0 && !plan.mfma[hi].vec_uv;
      max_m = std::max(max_m, plan.mfma[hi++].m);
    }
    lp.jobs = reinterpret_cast<const JobDesc*>(ws + mfma_off) + lo;
    lp.block_starts = reinterpret_cast<const int32_t*>(ws + mfma_bs_off) + lo;
    lp.n_jobs = (int32_t)(hi - lo);
    const int32_t first = plan.mfma[lo].block_start;
    const int64_t last = hi < plan.mfma.size() ? plan.mfma[hi].block_start : plan.mfma_blocks;
    lp.block_base = first;
    lp.total_blocks = (int32_t)(last - first);
    // the rank-class variants read U and V with 16-byte loads only; the streamed one takes any
    const int kmode = scalar_uv ? -1 : kmode_for(max_m);
    hipError_t e = kamera::launch_mfma(lp, plan.mfma[lo].win_width, kmode, stream);
    if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "MFMA kernel launch: %s", hipGetErrorString(e));
    lo = hi;
  }
  lp.block_base = 0;
  lp.xcd_remap = 0;
  if (!plan.valu.empty()) {
    lp.jobs = reinterpret_cast<const JobDesc*>(ws + valu_off);
    lp.block_starts = reinterpret_cast<const int32_t*>(ws + valu_bs_off);
    lp.n_jobs = (int32_t)plan.valu.size();
    lp.total_blocks = (int32_t)plan.valu_blocks;
    hipError_t e = kamera::launch_valu(lp, model->dtype == KAMERA_DTYPE_F32 ? 0 : 1, stream);
    if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "VALU kernel launch: %s", hipGetErrorString(e));
  }
  return KAMERA_OK;
}

}  // namespace

namespace kamera {
kamera_status reuse_batch_tables_at(const kamera_model* model, const kamera_cache* cache,
                                    const kamera_chunk* chunks, int32_t n_chunks, void* tables,
                                    size_t tables_bytes, void* stream) {
  return run(model, cache, chunks, n_chunks, tables, tables_bytes, stream, Op::Reuse, false);
}
}  // namespace kamera

extern "C" {

kamera_status kamera_init(void) {
  clear_error();
  const kamera_status st = init_current_device();
  return st != KAMERA_OK ? st : kamera::scratch_setup();
}

size_t kamera_workspace_bytes(int32_t n_chunks) {
  if (n_chunks < 0) return 0;
  // up to three jobs per chunk: channel 0 (two when a key head is partially rotary), channel 1
  return round_up(kTablesEnd + (size_t)n_chunks * 3 * (sizeof(JobDesc) + sizeof(int32_t)), 256);
}

kamera_status kamera_reuse_batch(const kamera_model* model, const kamera_cache* cache,
                                 const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream, Op::Reuse);
}

kamera_status kamera_relocate(const kamera_model* model, const kamera_cache* cache,
                              const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return run(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream, Op::Relocate);
}

kamera_status kamera_patch(const kamera_model* model, const kamera_cache* cache,
                           const kamera_chunk* chunks, int32_t n_chunks, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return run(model, cache, chunks, n_chunks, workspace, workspace_bytes, stream, Op::Patch);
}

kamera_status kamera_read_fault_count(const void* workspace, void* stream, uint32_t* count) {
  clear_error();
  if (!workspace || !count) return fail(KAMERA_ERR_INVALID_ARGUMENT, "NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(count, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "reading the fault count: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

size_t kamera_patch_bytes(const kamera_model* model, int32_t n_tokens, int32_t m) {
  if (!model || n_tokens < 0 || m < 0) return 0;
  if (validate_model(model) != KAMERA_OK) return 0;
  const size_t es = model->dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  size_t total = 0;
  for (int ch = 0; ch < 2; ++ch) {
    const Channel g = channel_of(*model, ch);
    total += (size_t)model->n_layers * g.heads * ((size_t)n_tokens + g.width) * m * es;
  }
  return total;
}

size_t kamera_kv_bytes(const kamera_model* model, int32_t n_tokens) {
  if (!model || n_tokens < 0) return 0;
  if (validate_model(model) != KAMERA_OK) return 0;
  const size_t es = model->dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  size_t total = 0;
  for (int ch = 0; ch < 2; ++ch) {
    const Channel g = channel_of(*model, ch);
    total += (size_t)model->n_layers * n_tokens * g.heads * g.width * es;
  }
  return total;
}

const char* kamera_status_string(kamera_status status) {
  switch (status) {
    case KAMERA_OK: return "ok";
    case KAMERA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KAMERA_ERR_UNSUPPORTED: return "unsupported";
    case KAMERA_ERR_OVERLAP: return "source overlaps destination";
    case KAMERA_ERR_WORKSPACE: return "workspace missing or too small";
    case KAMERA_ERR_HIP: return "HIP runtime error";
    case KAMERA_ERR_BUSY: return "staging ring busy";
  }
  return "unknown status";
}

const char* kamera_last_error(void) { return last_error(); }

int32_t kamera_version(void) { return KAMERA_VERSION; }

}  // extern "C"
