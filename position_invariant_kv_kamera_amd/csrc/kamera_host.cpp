// kamera_host.cpp — host helpers shared by every entry point of libkamera.so: the per-thread
// error message, model and cache validation, view ranges, and the pinned staging ring that
// copies job tables into the caller's workspace.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kamera_host.h"
#include "kamera_internal.h"

namespace kamera {
namespace host {

thread_local std::string g_last_error;

kamera_status fail(kamera_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }
const char* last_error() { return g_last_error.c_str(); }


size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Channel channel_of(const kamera_model& m, int c) {
  if (m.family == KAMERA_FAMILY_MLA)
    return c == KAMERA_CH_ROT ? Channel{1, m.rope_dim, true} : Channel{1, m.head_dim, false};
  return Channel{m.n_kv_heads, m.head_dim, c == KAMERA_CH_ROT};
}

Range view_range(const void* p, int64_t ls, int64_t n_layers, int64_t ts, int64_t n_tokens,
                 int64_t row_elems, int64_t esize) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  const int64_t last = (n_layers - 1) * ls + (n_tokens - 1) * ts + row_elems;
  return Range{b, b + static_cast<uintptr_t>(last * esize)};
}

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

kamera_status validate_model(const kamera_model* m) {
  if (!m) return fail(KAMERA_ERR_INVALID_ARGUMENT, "model is NULL");
  if (m->family != KAMERA_FAMILY_GQA && m->family != KAMERA_FAMILY_MLA)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "unknown model family %d", m->family);
  if (m->dtype != KAMERA_DTYPE_F32 && m->dtype != KAMERA_DTYPE_BF16)
    return fail(KAMERA_ERR_UNSUPPORTED, "unsupported dtype %d", m->dtype);
  if (m->n_layers <= 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_layers must be > 0");
  if (m->rope_layout != KAMERA_ROPE_HALF_SPLIT && m->rope_layout != KAMERA_ROPE_INTERLEAVED)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "unknown rope_layout %d", m->rope_layout);
  if (!std::isfinite(m->rope_theta) || !(m->rope_theta > 1.0))
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 1");
  if (m->head_dim <= 0 || m->head_dim % 2)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "head_dim must be even and > 0 (got %d)",
                m->head_dim);
  if (m->rope_dim <= 0 || m->rope_dim % 2)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "rope_dim must be even and > 0 (got %d)",
                m->rope_dim);
  if (m->rope_dim > 2 * kamera::kMaxPairs)
    return fail(KAMERA_ERR_UNSUPPORTED, "rope_dim %d exceeds %d", m->rope_dim,
                2 * kamera::kMaxPairs);
  if (m->family == KAMERA_FAMILY_GQA) {
    if (m->n_kv_heads <= 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_kv_heads must be > 0");
    if (m->rope_dim > m->head_dim)
      return fail(KAMERA_ERR_INVALID_ARGUMENT, "rope_dim (%d) exceeds head_dim (%d)",
                  m->rope_dim, m->head_dim);
  } else if (m->n_kv_heads != 1) {
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "MLA needs n_kv_heads == 1 (got %d)",
                m->n_kv_heads);
  }
  const int pairs = m->rope_dim / 2;
  if (m->inv_freq) {
    for (int i = 0; i < pairs; ++i)
      if (!std::isfinite(m->inv_freq[i]) || m->inv_freq[i] < 0.0)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "inv_freq[%d] must be finite and >= 0", i);
  }
  if (m->n_sections < 0 || m->n_sections > KAMERA_MAX_SECTIONS)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_sections must be in [0, %d] (got %d)",
                KAMERA_MAX_SECTIONS, m->n_sections);
  if ((m->n_sections > 0) != (m->pair_section != nullptr))
    return fail(KAMERA_ERR_INVALID_ARGUMENT,
                "pair_section must be given exactly when n_sections > 0");
  if (m->pair_section) {
    for (int i = 0; i < pairs; ++i)
      if (m->pair_section[i] >= m->n_sections)
        return fail(KAMERA_ERR_INVALID_ARGUMENT, "pair_section[%d] = %d is not below n_sections",
                    i, (int)m->pair_section[i]);
  }
  return KAMERA_OK;
}

kamera_status validate_cache(const kamera_model& m, const kamera_cache* c) {
  if (!c) return fail(KAMERA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!c->pool[0] || !c->pool[1]) return fail(KAMERA_ERR_INVALID_ARGUMENT, "cache pool is NULL");
  if (c->page_size <= 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "page_size must be > 0");
  if (c->n_pages <= 0) return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_pages must be > 0");
  if (c->n_logical_pages <= 0)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "n_logical_pages must be > 0");
  if (!c->page_table && c->n_logical_pages > c->n_pages)
    return fail(KAMERA_ERR_INVALID_ARGUMENT,
                "identity page table needs n_logical_pages (%d) <= n_pages (%d)",
                c->n_logical_pages, c->n_pages);
  if ((int64_t)c->n_logical_pages * c->page_size > INT32_MAX)
    return fail(KAMERA_ERR_UNSUPPORTED, "cache holds more than 2^31-1 logical tokens");
  if (c->token_stride <= 0 || c->layer_stride < 0)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "cache strides must be positive");
  const int64_t slots = (int64_t)c->n_pages * c->page_size;
  for (int ch = 0; ch < 2; ++ch) {
    const Channel g = channel_of(m, ch);
    if ((int64_t)g.heads * g.width > c->token_stride)
      return fail(KAMERA_ERR_INVALID_ARGUMENT,
                  "cache token_stride (%lld) is shorter than channel %d's row (%d)",
                  (long long)c->token_stride, ch, g.heads * g.width);
  }
  if (m.n_layers > 1 && c->layer_stride < slots * c->token_stride)
    return fail(KAMERA_ERR_INVALID_ARGUMENT, "cache layer_stride overlaps the next layer");
  // the two channel pools may share rows (MLA), but must not write the same elements
  const int64_t es = m.dtype == KAMERA_DTYPE_F32 ? 4 : 2;
  const Channel g0 = channel_of(m, 0), g1 = channel_of(m, 1);
  const Range r0 = view_range(c->pool[0], c->layer_stride, m.n_layers, c->token_stride, slots,
                              (int64_t)g0.heads * g0.width, es);
  const Range r1 = view_range(c->pool[1], c->layer_stride, m.n_layers, c->token_stride, slots,
                              (int64_t)g1.heads * g1.width, es);
  if (overlaps(r0, r1)) {
    const int64_t d = ((int64_t)reinterpret_cast<intptr_t>(c->pool[0]) -
                       (int64_t)reinterpret_cast<intptr_t>(c->pool[1]));
    const int64_t w0 = (int64_t)g0.heads * g0.width * es, w1 = (int64_t)g1.heads * g1.width * es;
    const int64_t row = c->token_stride * es;
    const bool disjoint_rows = (d >= w1 && d + w0 <= row) || (-d >= w0 && -d + w1 <= row);
    if (!disjoint_rows)
      return fail(KAMERA_ERR_OVERLAP, "the two channel pools write the same elements");
  }
  return KAMERA_OK;
}

// ---------------------------------------------------------------------------------------
// pinned staging ring for the job tables (host -> workspace copies)
// ---------------------------------------------------------------------------------------
//
// One ring per device, set up once (kamera_init, or the first compute call on the device):
// kStagingBytes of pinned host memory and kMaxInFlight events. Every call copies its table
// into the next free region of the ring and enqueues one hipMemcpyAsync from there, followed by
// an event. A region is handed out again only once its event has completed, which is checked
// with hipEventQuery and never waited for: when the regions a call needs are all still in
// flight the call fails with KAMERA_ERR_BUSY and enqueues nothing. After set-up nothing here
// allocates or frees, and nothing blocks the host.

struct Ring {
  std::mutex mu;
  bool ready = false;
  uint8_t* host = nullptr;
  hipEvent_t ev[kMaxInFlight];
  size_t lo[kMaxInFlight], hi[kMaxInFlight];  // byte range of each in-flight entry
  int first = 0, count = 0;                   // FIFO of in-flight entries
  size_t head = 0;                            // where the next region starts
};

Ring* ring_for(int device) {
  static Ring rings[kMaxDevices];   // process lifetime; never torn down (no exit-time HIP calls)
  return (device >= 0 && device < kMaxDevices) ? &rings[device] : nullptr;
}

namespace {

// Allocates the ring of the current device (caller holds r.mu).
kamera_status ring_setup(Ring& r) {
  if (r.ready) return KAMERA_OK;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, kStagingBytes, hipHostMallocDefault);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipHostMalloc: %s", hipGetErrorString(e));
  for (int i = 0; i < kMaxInFlight; ++i) {
    e = hipEventCreateWithFlags(&r.ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int k = 0; k < i; ++k) (void)hipEventDestroy(r.ev[k]);
      (void)hipHostFree(h);
      return fail(KAMERA_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  r.host = static_cast<uint8_t*>(h);
  r.first = r.count = 0;
  r.head = 0;
  r.ready = true;
  return KAMERA_OK;
}

kamera_status current_ring(Ring** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  Ring* r = ring_for(dev);
  if (!r) return fail(KAMERA_ERR_UNSUPPORTED, "device index %d is not below %d", dev, kMaxDevices);
  *out = r;
  return KAMERA_OK;
}

}  // namespace

kamera_status init_current_device() {
  Ring* r = nullptr;
  kamera_status st = current_ring(&r);
  if (st != KAMERA_OK) return st;
  std::lock_guard<std::mutex> lock(r->mu);
  return ring_setup(*r);
}

kamera_status check_stream(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(KAMERA_ERR_UNSUPPORTED,
                "the stream is being captured: a captured call would replay a copy from a "
                "staging region later calls reuse");
  return KAMERA_OK;
}

kamera_status upload(const std::vector<uint8_t>& bytes, void* workspace, hipStream_t stream,
                     bool allow_setup) {
  const size_t n = bytes.size();
  if (n > kStagingBytes)
    return fail(KAMERA_ERR_UNSUPPORTED,
                "a table of %zu bytes exceeds the staging ring (%zu bytes): split the batch", n,
                kStagingBytes);
  kamera_status st = check_stream(stream);
  if (st != KAMERA_OK) return st;
  Ring* r = nullptr;
  st = current_ring(&r);
  if (st != KAMERA_OK) return st;
  std::lock_guard<std::mutex> lock(r->mu);
  if (!r->ready && !allow_setup)
    return fail(KAMERA_ERR_UNSUPPORTED,
                "kamera_init() has not been called on this device (this call allocates nothing, "
                "so it cannot set up the staging ring)");
  st = ring_setup(*r);
  if (st != KAMERA_OK) return st;
  // retire the entries whose copies have completed (oldest first)
  while (r->count > 0) {
    const hipError_t q = hipEventQuery(r->ev[r->first]);
    if (q == hipErrorNotReady) break;
    if (q != hipSuccess) return fail(KAMERA_ERR_HIP, "hipEventQuery: %s", hipGetErrorString(q));
    r->first = (r->first + 1) % kMaxInFlight;
    --r->count;
  }
  if (r->count == 0) r->head = 0;
  size_t lo = r->head;
  if (lo + n > kStagingBytes) lo = 0;   // wrap: regions are contiguous
  const size_t hi = lo + n;
  bool clash = r->count == kMaxInFlight;
  for (int k = 0; k < r->count && !clash; ++k) {
    const int i = (r->first + k) % kMaxInFlight;
    clash = lo < r->hi[i] && r->lo[i] < hi;
  }
  if (clash)
    return fail(KAMERA_ERR_BUSY,
                "the staging ring holds the tables of %d calls the device has not reached; "
                "synchronise the stream (or wait) and call again",
                r->count);
  std::memcpy(r->host + lo, bytes.data(), n);
  hipError_t e = hipMemcpyAsync(workspace, r->host + lo, n, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  const int slot = (r->first + r->count) % kMaxInFlight;
  e = hipEventRecord(r->ev[slot], stream);
  if (e != hipSuccess) return fail(KAMERA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  r->lo[slot] = lo;
  r->hi[slot] = hi;
  ++r->count;
  r->head = round_up(hi, 256);
  return KAMERA_OK;
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return v && *v ? std::atoi(v) : dflt;
}

}  // namespace host
}  // namespace kamera
