// das_noalloc.hip -- das_decode_attention_noalloc: das_decode_attention with
// its workspace in a static device array instead of a caller's buffer, for
// callers that cannot allocate device memory.
//
// The array lives in this file: each GPU the library runs on holds its own
// copy (kScratchBytes) from the first use until the process ends.  Host code
// never passes the array's name to a kernel -- in host code that name is a
// host-side stand-in, not a device address.  The device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// only that address is used afterwards.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "das.h"
#include "das_internal.h"

namespace {

// Largest workspace the no-allocation entry point serves (see das.h).
constexpr size_t kScratchBytes = DAS_NOALLOC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_init;

// Zeroes n 32-bit words (the arrival counters) with plain vector stores.
__global__ void zero_words(unsigned int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of this device's scratch array.  On the first call for
// a device: look it up with the device current, and zero its arrival
// counters with a fill kernel on `st`, ordered before the caller's kernels.
int scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DAS_ELAUNCH;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_init);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return DAS_ELAUNCH;
      constexpr int kWords = DAS_WORKSPACE_COUNTER_BYTES / 4;
      hipLaunchKernelGGL(zero_words, dim3((kWords + 255) / 256), dim3(256), 0, st,
                         static_cast<unsigned int*>(ptr), kWords);
      if (hipGetLastError() != hipSuccess) return DAS_ELAUNCH;
      g_scratch[dev].store(ptr, std::memory_order_release);
      p = ptr;
    }
  }
  *out = p;
  return DAS_OK;
}

}  // namespace

extern "C" int das_decode_attention_noalloc(const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* seq_lens,
                                            int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax,
                                            int32_t D, float scale, void* out, int32_t out_dtype,
                                            float* lse_out, int32_t num_splits, void* stream) {
  static_assert(kScratchBytes > DAS_WORKSPACE_COUNTER_BYTES, "scratch holds the counters");
  const size_t need = das_decode_workspace_bytes(B, Hq, Hkv, Smax, D, num_splits, 0);
  // invalid shapes: das_decode_attention reports them (and launches nothing)
  if (need == (size_t)-1 || need == 0)
    return das_decode_attention(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Smax, D, scale, out,
                                out_dtype, lse_out, num_splits, nullptr, 0, stream);
  if (need > kScratchBytes) return DAS_EWORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (rc != DAS_OK) return rc;
  return das_decode_attention(q, k_cache, v_cache, seq_lens, B, Hq, Hkv, Smax, D, scale, out,
                              out_dtype, lse_out, num_splits, ws, kScratchBytes, stream);
}
