// kamera_noalloc.hip — kamera_reuse_batch_noalloc: the reuse operator for callers that cannot
// allocate (code that must not call hipMalloc: tight serving loops, harnesses that forbid it).
//
// It is kamera_reuse_batch (same validation, planning, kernels and results, bit for bit) with
// the device tables — fault counter, frequency table, pair sections, job records and block
// starts, i.e. what kamera_reuse_batch puts in the caller's workspace — in a file-scope
// device array of fixed size instead. Each GPU the library runs on holds its own copy of the
// array until the process ends. kamera_init() looks up this device's address of it once
// (hipGetSymbolAddress, with the device current) and keeps it per device; host code uses that
// address, never the array's name, which in host code is only a stand-in.
//
// Every call on one GPU shares that GPU's array and overwrites it: the table upload writes
// the whole table, header included, so the fault counter starts from zero in every call.
// Calls on one GPU whose work can overlap (different streams without ordering between them,
// or several host threads at once) race on the array; calls on one stream are ordered.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kamera_host.h"
#include "kamera_internal.h"

static_assert(sizeof(kamera::JobDesc) == 176, "the chunk limit below assumes 176-byte job records");

namespace kamera {
// 1 MiB: the header (4.6 KB) and up to three job entries of 180 bytes (a 176-byte record and
// its block start) per chunk, so up to 1932 chunks per call.
constexpr size_t kScratchBytes = size_t(1) << 20;
}  // namespace kamera

static __device__ __align__(256) uint8_t scratch[kamera::kScratchBytes];

namespace kamera {
namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[host::kMaxDevices] = {};

}  // namespace

kamera_status scratch_setup() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return host::fail(KAMERA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= host::kMaxDevices)
    return host::fail(KAMERA_ERR_UNSUPPORTED, "device index %d is not below %d", dev,
                      host::kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return KAMERA_OK;
  void* ptr = nullptr;
  e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return host::fail(KAMERA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  g_scratch_ptr[dev] = ptr;
  return KAMERA_OK;
}

}  // namespace kamera

extern "C" kamera_status kamera_reuse_batch_noalloc(const kamera_model* model,
                                                    const kamera_cache* cache,
                                                    const kamera_chunk* chunks, int32_t n_chunks,
                                                    void* stream) {
  kamera::host::clear_error();
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return kamera::host::fail(KAMERA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  void* ptr = nullptr;
  if (dev >= 0 && dev < kamera::host::kMaxDevices) {
    std::lock_guard<std::mutex> lock(kamera::g_scratch_mu);
    ptr = kamera::g_scratch_ptr[dev];
  }
  if (!ptr)
    return kamera::host::fail(KAMERA_ERR_UNSUPPORTED,
                              "kamera_init() has not been called on device %d", dev);
  if (n_chunks > 0 && kamera_workspace_bytes(n_chunks) > kamera::kScratchBytes)
    return kamera::host::fail(
        KAMERA_ERR_UNSUPPORTED,
        "%d chunks need %zu bytes of tables; this entry point's scratch holds %zu "
        "(at most %zu chunks per call)",
        n_chunks, kamera_workspace_bytes(n_chunks), kamera::kScratchBytes,
        (kamera::kScratchBytes - kamera::kTablesEnd) /
            (3 * (sizeof(kamera::JobDesc) + sizeof(int32_t))));
  return kamera::reuse_batch_tables_at(model, cache, chunks, n_chunks, ptr, kamera::kScratchBytes,
                                       stream);
}
