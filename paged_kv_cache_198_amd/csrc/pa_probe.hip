// Diagnostic: the device-memory read rate a plain streaming kernel reaches
// on this GPU, measured with the same 16-byte non-temporal loads the decode
// kernels use.  It is the practical ceiling the decode kernels' fraction of
// the nominal HBM peak is read against; it computes nothing the decode path
// needs.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;

// Grid-stride read of n16 16-byte chunks; every thread folds what it read
// into one word and stores it (a plain vector store per thread), so the
// loads cannot be dropped.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* src,
                                                                   size_t n16, uint32_t* out) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace pa

extern "C" int pa_probe_read_bandwidth(const void* src, size_t bytes, uint32_t* out,
                                       int32_t out_words, void* stream) {
  if (!src || !out || bytes == 0 || (bytes & 15u) || !pa::aligned16(src)) return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(out) & 3u) || out_words < pa::kProbeThreads)
    return PA_ERR_INVALID;
  const int32_t blocks = std::min<int32_t>(out_words / pa::kProbeThreads, 4096);
  hipLaunchKernelGGL(pa::read_probe_kernel, dim3(static_cast<uint32_t>(blocks)),
                     dim3(pa::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const pa::u32x4_t*>(src), bytes / 16, out);
  return pa::launch_status();
}
