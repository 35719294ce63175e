// kamera_host.h — host helpers shared by the entry points (kamera_host.cpp). Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/kamera.h"
#include <string>
#include <vector>

namespace kamera {
namespace host {

// Geometry of one channel: heads and features per head.
struct Channel {
  int32_t heads;
  int32_t width;
  bool rotate;
};
// Byte range [lo, hi) touched by a (layer, token, row) view.
struct Range {
  uintptr_t lo, hi;
};

kamera_status fail(kamera_status st, const char* fmt, ...);
void clear_error();
const char* last_error();
size_t round_up(size_t x, size_t a);
bool aligned16(const void* p);
Channel channel_of(const kamera_model& m, int c);
Range view_range(const void* p, int64_t ls, int64_t n_layers, int64_t ts, int64_t n_tokens,
                 int64_t row_elems, int64_t esize);
bool overlaps(const Range& a, const Range& b);
kamera_status validate_model(const kamera_model* m);
kamera_status validate_cache(const kamera_model& m, const kamera_cache* c);
// Staging ring of one device: pinned host bytes and the most calls whose copies may be in
// flight at once.
constexpr size_t kStagingBytes = size_t(32) << 20;
constexpr int kMaxInFlight = 256;
constexpr int kMaxDevices = 64;
// Sets up the current device's staging ring (the library's one allocation; idempotent).
kamera_status init_current_device();
// KAMERA_ERR_UNSUPPORTED when `stream` is being captured into a graph.
kamera_status check_stream(hipStream_t stream);
// Copies `bytes` into the device workspace through the current device's staging ring, on
// `stream` (sets the ring up on first use when allow_setup, else KAMERA_ERR_UNSUPPORTED if
// kamera_init() has not run on the device). Never allocates after set-up and never waits:
// KAMERA_ERR_BUSY when every region it could use is still in flight.
kamera_status upload(const std::vector<uint8_t>& bytes, void* workspace, hipStream_t stream,
                     bool allow_setup = true);
int env_int(const char* name, int dflt);

}  // namespace host
}  // namespace kamera
