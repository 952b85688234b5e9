// msa_attention_paged_noalloc: msa_attention_paged for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its kernels take their workspace (the
// split-K partials, the union-tile plan and the scheduler state) from one
// fixed device array instead of a caller buffer.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, allocated when the code object is loaded on that
// device and kept until the process ends.  In host code the variable's name
// only stands in for the symbol; the device address of each GPU's copy comes
// from hipGetSymbolAddress with that GPU current, taken once per device and
// cached.  Every call on one GPU shares that GPU's copy and finds the last
// call's contents in it; nothing in it has to start at any value (the plan
// kernels write every entry they read, and the scheduler resets its own
// counter), and calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "msa.h"
#include "msa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's copy of `scratch`, resolved once per
// device; null (with the status in *st) when it cannot be resolved.
void* scratch_of_current_device(int* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = MSA_ERR_DEVICE;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *st = MSA_ERR_DEVICE;
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int msa_attention_paged_noalloc(void* output, const void* q, const int32_t* d_indices,
                                           const msa_paged_cache* k_cache,
                                           const msa_paged_cache* v_cache, const msa_ragged* rg,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t top_k, float scale, int32_t num_partitions,
                                           void* stream) {
  // The workspace this shape needs, as msa_attention_paged would be given;
  // the size query returns 0 for invalid arguments, which the entry below
  // then reports.
  const size_t need = msa_attention_workspace_bytes(rg, num_q_heads, num_kv_heads, top_k,
                                                    num_partitions);
  if (need > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int st = MSA_OK;
    ws = scratch_of_current_device(&st);
    if (!ws) {
      // no array on this device: report argument errors first (the entry
      // validates everything before it asks for its workspace), else st
      const int v = msa::attention_paged_entry(output, q, d_indices, k_cache, v_cache, rg,
                                               num_q_heads, num_kv_heads, top_k, scale,
                                               num_partitions, nullptr, 0, stream, false);
      return v == MSA_ERR_NULL ? st : v;
    }
  }
  return msa::attention_paged_entry(output, q, d_indices, k_cache, v_cache, rg, num_q_heads,
                                    num_kv_heads, top_k, scale, num_partitions, ws,
                                    ws ? (size_t)MSA_NOALLOC_SCRATCH_BYTES : 0, stream, false);
}
