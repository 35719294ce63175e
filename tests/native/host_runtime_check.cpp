// host_runtime_check.cpp — CPU check of libkamera's host runtime (argument validation, work
// planning and the pinned staging ring of kamera_api.cpp / kamera_host.cpp), built with g++
// under AddressSanitizer and UndefinedBehaviorSanitizer against a counting stand-in for the
// HIP runtime. No GPU is involved: device pointers are host addresses the host code never
// dereferences, kernel launches are recorded, and "device" copies land in host buffers.
//
// What it shows:
//   * the staging ring is allocated once per device (kamera_init or the first call) and never
//     again: no compute call allocates, frees or waits on the host after that;
//   * when every ring region still feeds an unfinished copy, a call returns KAMERA_ERR_BUSY and
//     enqueues nothing; once the copies complete, calls go through again, wrapping the ring;
//   * a capturing stream is rejected before anything is enqueued;
//   * rejected calls (invalid descriptors) enqueue nothing;
//   * the table a call uploads describes its chunks (header cleared, one job per channel).
// Exit status 0 when every check passes; each failure prints a line.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/kamera.h"
#include "../../position_invariant_kv_kamera_amd/csrc/kamera_internal.h"

// ------------------------------------------------------------------------------------------
// counting stand-in for the HIP runtime calls the host code makes
// ------------------------------------------------------------------------------------------
struct ihipEvent_t {
  bool recorded = false;
  bool done = false;
  const uint8_t* lo = nullptr;   // staging bytes the copy recorded before this event reads
  const uint8_t* hi = nullptr;
};

namespace mock {
int device = 0;
int host_mallocs = 0, host_frees = 0, event_creates = 0, event_destroys = 0;
int memcpys = 0, event_records = 0, stream_syncs = 0, launches = 0;
hipStream_t capturing = nullptr;   // stream reported as capturing
std::vector<ihipEvent_t*> events;
kamera::LaunchParams last_launch;
int last_kmode = -99, last_width = 0;
std::vector<uint8_t> last_copy;     // bytes of the last host -> device copy
const uint8_t* copy_lo = nullptr;   // staging range of the last copy
const uint8_t* copy_hi = nullptr;
const uint8_t* prev_lo = nullptr;
int wraps = 0;                      // copies that started below the previous one
int overlaps_in_flight = 0;         // copies that read bytes an unfinished copy still reads
std::vector<ihipEvent_t*> record_order;

void complete_all() {
  for (ihipEvent_t* e : events)
    if (e->recorded) e->done = true;
}
void complete_oldest(int k) {
  for (ihipEvent_t* e : record_order)
    if (k > 0 && e->recorded && !e->done) {
      e->done = true;
      --k;
    }
}
int pending() {
  int n = 0;
  for (ihipEvent_t* e : events) n += e->recorded && !e->done;
  return n;
}
}  // namespace mock

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = mock::device;
  return hipSuccess;
}
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  ++mock::host_mallocs;
  *p = std::malloc(n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* p) {
  ++mock::host_frees;
  std::free(p);
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  ++mock::event_creates;
  *e = new ihipEvent_t();
  mock::events.push_back(*e);
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) {
  ++mock::event_destroys;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  ++mock::event_records;
  e->recorded = true;
  e->done = false;
  e->lo = mock::copy_lo;
  e->hi = mock::copy_hi;
  mock::record_order.push_back(e);
  return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t e) {
  return (!e->recorded || e->done) ? hipSuccess : hipErrorNotReady;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  ++mock::memcpys;
  const uint8_t* lo = static_cast<const uint8_t*>(src);
  for (ihipEvent_t* e : mock::events)
    if (e->recorded && !e->done && lo < e->hi && e->lo < lo + n) ++mock::overlaps_in_flight;
  if (mock::prev_lo && lo < mock::prev_lo) ++mock::wraps;
  mock::prev_lo = lo;
  mock::copy_lo = lo;
  mock::copy_hi = lo + n;
  mock::last_copy.assign(lo, lo + n);
  std::memcpy(dst, src, n);   // the "device" workspace is a host buffer here
  return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t s, hipStreamCaptureStatus* st) {
  *st = (s != nullptr && s == mock::capturing) ? hipStreamCaptureStatusActive
                                               : hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) {
  ++mock::stream_syncs;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "mock error"; }
}

namespace mock {
int scratch_setups = 0;
}
namespace kamera {
kamera_status scratch_setup() {   // the no-allocation entry point's symbol lookup
  ++mock::scratch_setups;
  return KAMERA_OK;
}
hipError_t launch_mfma(const LaunchParams& p, int win_width, int kmode, hipStream_t) {
  ++mock::launches;
  mock::last_launch = p;
  mock::last_kmode = kmode;
  mock::last_width = win_width;
  return hipSuccess;
}
hipError_t launch_valu(const LaunchParams& p, int, hipStream_t) {
  ++mock::launches;
  mock::last_launch = p;
  return hipSuccess;
}
}  // namespace kamera

// ------------------------------------------------------------------------------------------
// checks
// ------------------------------------------------------------------------------------------
static int failures = 0;
#define CHECK(cond)                                                           \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::printf("FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond,          \
                  kamera_last_error());                                       \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

// A GQA bf16 model (4 heads x 128, 2 layers) and a dense cache; device buffers are host memory
// that only the (recorded, never run) kernels would touch.
struct Fixture {
  kamera_model model{};
  kamera_cache cache{};
  std::vector<uint16_t> pool_k, pool_v, src;
  std::vector<uint16_t> U, V;
  std::vector<uint8_t> ws;
  uint8_t* ws_ptr = nullptr;
  int n_tokens = 64;

  explicit Fixture(int max_chunks) {
    model.family = KAMERA_FAMILY_GQA;
    model.dtype = KAMERA_DTYPE_BF16;
    model.n_layers = 2;
    model.n_kv_heads = 4;
    model.head_dim = 128;
    model.rope_dim = 128;
    model.rope_layout = KAMERA_ROPE_HALF_SPLIT;
    model.rope_theta = 1e6;
    const int row = 4 * 128;
    const int64_t slots = (int64_t)max_chunks * n_tokens;
    pool_k.assign(2 * slots * row + 64, 0);
    pool_v.assign(2 * slots * row + 64, 0);
    src.assign(2 * (size_t)n_tokens * 2 * row + 64, 0);
    U.assign(2 * 4 * n_tokens * 16 + 64, 0);
    V.assign(2 * 4 * 128 * 16 + 64, 0);
    cache.pool[0] = align(pool_k.data());
    cache.pool[1] = align(pool_v.data());
    cache.layer_stride = slots * row;
    cache.token_stride = row;
    cache.page_table = nullptr;
    cache.page_size = 16;
    cache.n_logical_pages = (int32_t)(slots / 16);
    cache.n_pages = cache.n_logical_pages;
    ws.assign(kamera_workspace_bytes(max_chunks) + 512, 0xAB);
    ws_ptr = reinterpret_cast<uint8_t*>((reinterpret_cast<uintptr_t>(ws.data()) + 255) / 256 * 256);
  }
  static void* align(void* p) {
    return reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(p) + 15) / 16 * 16);
  }
  std::vector<kamera_chunk> chunks(int n, int m) {
    std::vector<kamera_chunk> v(n);
    const int row = 4 * 128;
    for (int i = 0; i < n; ++i) {
      kamera_chunk& k = v[i];
      std::memset(&k, 0, sizeof k);
      k.n_tokens = n_tokens;
      k.dst_token_offset = i * n_tokens;
      k.delta = 1000 + i;
      for (int ch = 0; ch < 2; ++ch) {
        // the two channels read disjoint halves of the same source buffer
        k.src[ch].ptr = static_cast<uint16_t*>(align(src.data())) + (size_t)ch * 2 * n_tokens * row;
        k.src[ch].layer_stride = (int64_t)n_tokens * row;
        k.src[ch].token_stride = row;
        k.patch[ch].m = m;
        if (m > 0) {
          k.patch[ch].U = align(U.data());
          k.patch[ch].u_layer_stride = 4 * (int64_t)n_tokens * m;
          k.patch[ch].u_head_stride = (int64_t)n_tokens * m;
          k.patch[ch].V = align(V.data());
          k.patch[ch].v_layer_stride = 4 * 128 * (int64_t)m;
          k.patch[ch].v_head_stride = 128 * (int64_t)m;
        }
      }
    }
    return v;
  }
  kamera_status reuse(const std::vector<kamera_chunk>& c, size_t ws_bytes, hipStream_t s) {
    return kamera_reuse_batch(&model, &cache, c.data(), (int32_t)c.size(), ws_ptr, ws_bytes, s);
  }
};

int main() {
  hipStream_t stream = reinterpret_cast<hipStream_t>(0x1000);

  // set-up: one pinned allocation and the event pool, once per device
  CHECK(kamera_init() == KAMERA_OK);
  CHECK(mock::host_mallocs == 1);
  CHECK(mock::event_creates == 256);
  CHECK(mock::scratch_setups == 1);
  CHECK(kamera_init() == KAMERA_OK);
  CHECK(mock::host_mallocs == 1 && mock::event_creates == 256);

  Fixture fx(512);
  const size_t wsb = kamera_workspace_bytes(512);

  // a normal call: one copy, one event, one launch; no allocation, free or host wait
  {
    auto c = fx.chunks(3, 16);
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_OK);
    CHECK(mock::memcpys == 1 && mock::event_records == 1 && mock::launches == 1);
    CHECK(mock::last_kmode == 16 && mock::last_width == 128);
    CHECK(mock::last_launch.n_jobs == 6);   // 3 chunks x 2 channels
    // the uploaded table: a cleared header (the fault counter), then the jobs
    uint32_t counter = 0xFFFFFFFFu;
    std::memcpy(&counter, fx.ws_ptr, sizeof counter);
    CHECK(counter == 0);
    CHECK(mock::last_copy.size() >= kamera::kTablesEnd + 6 * sizeof(kamera::JobDesc));
  }

  // many calls while the device never catches up: 256 may be in flight, then BUSY with
  // nothing enqueued; after the copies complete, calls go through again
  {
    auto c = fx.chunks(2, 0);
    int ok = 0, busy = 0;
    const int copies0 = mock::memcpys, launches0 = mock::launches;
    for (int i = 0; i < 300; ++i) {
      const kamera_status st = fx.reuse(c, wsb, stream);
      if (st == KAMERA_OK) ++ok;
      else if (st == KAMERA_ERR_BUSY) ++busy;
    }
    CHECK(ok == 255 && busy == 45);   // one entry was already in flight from the call above
    CHECK(mock::memcpys - copies0 == ok && mock::launches - launches0 == ok);
    CHECK(mock::pending() == 256);
    mock::complete_all();
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_OK);
    CHECK(mock::pending() == 1);
  }

  // large tables: the ring wraps round; a region is handed out again only after the copy
  // that read it completed (the device retires the oldest copies first)
  {
    auto c = fx.chunks(512, 16);
    const size_t table = mock::last_copy.size();
    int ok = 0, busy = 0;
    for (int i = 0; i < 5000 && ok < 1000; ++i) {
      const kamera_status st = fx.reuse(c, wsb, stream);
      if (st == KAMERA_OK) {
        ++ok;
      } else {
        CHECK(st == KAMERA_ERR_BUSY);
        ++busy;
        mock::complete_oldest(40);
      }
    }
    CHECK(ok == 1000 && busy > 0);
    CHECK(mock::last_copy.size() > table);
    CHECK(mock::wraps >= 4);
  }
  CHECK(mock::overlaps_in_flight == 0);

  // a capturing stream is rejected before anything is enqueued
  {
    auto c = fx.chunks(2, 16);
    mock::complete_all();
    const int copies0 = mock::memcpys, launches0 = mock::launches;
    mock::capturing = stream;
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_ERR_UNSUPPORTED);
    mock::capturing = nullptr;
    CHECK(mock::memcpys == copies0 && mock::launches == launches0);
  }

  // invalid descriptors: rejected on the host, nothing enqueued
  {
    const int copies0 = mock::memcpys, launches0 = mock::launches;
    auto c = fx.chunks(2, 16);
    c[1].dst_token_offset = c[0].dst_token_offset;   // two chunks write the same tokens
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_ERR_INVALID_ARGUMENT);
    c = fx.chunks(2, 16);
    c[0].patch[1].m = KAMERA_MAX_RANK + 1;
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_ERR_UNSUPPORTED);
    c = fx.chunks(2, 16);
    c[0].src[0].ptr = fx.cache.pool[0];               // source inside the cache
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_ERR_OVERLAP);
    c = fx.chunks(2, 16);
    CHECK(fx.reuse(c, 64, stream) == KAMERA_ERR_WORKSPACE);
    CHECK(kamera_reuse_batch(&fx.model, &fx.cache, c.data(), 2, fx.ws_ptr + 16, wsb, stream) ==
          KAMERA_ERR_WORKSPACE);
    kamera_model bad = fx.model;
    bad.rope_theta = 0.5;
    CHECK(kamera_relocate(&bad, &fx.cache, c.data(), 2, fx.ws_ptr, wsb, stream) ==
          KAMERA_ERR_INVALID_ARGUMENT);
    CHECK(mock::memcpys == copies0 && mock::launches == launches0);
  }

  // relocate and patch take the same path
  {
    mock::complete_all();
    auto c = fx.chunks(4, 32);
    CHECK(kamera_relocate(&fx.model, &fx.cache, c.data(), 4, fx.ws_ptr, wsb, stream) == KAMERA_OK);
    CHECK(mock::last_kmode == 0);
    CHECK(kamera_patch(&fx.model, &fx.cache, c.data(), 4, fx.ws_ptr, wsb, stream) == KAMERA_OK);
    CHECK(mock::last_kmode == 32);
  }

  // a second device gets a ring of its own at its first call; the first device's is kept
  {
    mock::device = 1;
    auto c = fx.chunks(2, 16);
    CHECK(fx.reuse(c, wsb, stream) == KAMERA_OK);
    CHECK(mock::host_mallocs == 2 && mock::event_creates == 512);
    mock::device = 0;
  }

  // the no-allocation path never sets a ring up: on a device kamera_init() has not seen it is
  // refused with nothing allocated or enqueued
  {
    mock::device = 2;
    auto c = fx.chunks(2, 16);
    const int mallocs0 = mock::host_mallocs, copies0 = mock::memcpys, launches0 = mock::launches;
    CHECK(kamera::reuse_batch_tables_at(&fx.model, &fx.cache, c.data(), 2, fx.ws_ptr, wsb,
                                        stream) == KAMERA_ERR_UNSUPPORTED);
    CHECK(mock::host_mallocs == mallocs0 && mock::memcpys == copies0 &&
          mock::launches == launches0);
    mock::device = 0;
    CHECK(kamera::reuse_batch_tables_at(&fx.model, &fx.cache, c.data(), 2, fx.ws_ptr, wsb,
                                        stream) == KAMERA_OK);
    CHECK(mock::host_mallocs == mallocs0);
  }

  // nothing above allocated after set-up, freed, or waited on the host
  CHECK(mock::host_frees == 0 && mock::event_destroys == 0 && mock::stream_syncs == 0);

  // the fault-count reader is the one call that synchronises (documented)
  uint32_t count = 7;
  CHECK(kamera_read_fault_count(fx.ws_ptr, stream, &count) == KAMERA_OK);
  CHECK(mock::stream_syncs == 1);

  std::printf("host runtime checks: %d failure(s); %d copies, %d launches, %d pinned "
              "allocations\n",
              failures, mock::memcpys, mock::launches, mock::host_mallocs);
  for (ihipEvent_t* e : mock::events) delete e;
  return failures == 0 ? 0 : 1;
}
