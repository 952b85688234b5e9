// Device-side report of bad table data.  The kernels never read outside the
// caller's buffers: a page id outside the pool skips (or re-reads page 0 for)
// its block, and lengths beyond what the host bounds and the lookup table
// allow are clipped.  The sequence concerned then gets an undefined result
// while every other sequence's stays exact.  So that such data does not go
// unnoticed, the kernels also set a bit in a per-device error word, which
// msa_device_errors reads and clears.
//
// The word is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy.  Its device address is resolved once per device with
// hipGetSymbolAddress (with that device current) and handed to the kernels
// in their parameter blocks; a kernel whose pointer is null reports nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "msa.h"
#include "msa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ uint32_t error_word;

std::mutex g_err_mu;
std::atomic<uint32_t*> g_err_ptr[kMaxDevices];

}  // namespace

namespace msa {

uint32_t* device_error_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint32_t* p = g_err_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_err_mu);
  p = g_err_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(error_word)) != hipSuccess || !q) {
      (void)hipGetLastError();
      return nullptr;
    }
    p = static_cast<uint32_t*>(q);
    g_err_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace msa

extern "C" int msa_device_errors(uint32_t* bits, int clear, void* stream) {
  if (!bits) return MSA_ERR_NULL;
  uint32_t* word = msa::device_error_word();
  if (!word) return MSA_ERR_DEVICE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return MSA_ERR_LAUNCH;
  if (clear) {
    static const uint32_t zero = 0;
    if (hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess)
      return MSA_ERR_LAUNCH;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return MSA_ERR_LAUNCH;
  *bits = v;
  return MSA_OK;
}
