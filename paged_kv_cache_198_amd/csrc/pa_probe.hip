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

// Read of n16 16-byte chunks in contiguous 32 KB slices, workgroups
// striding over the slices: within a slice each wavefront instruction reads
// 1 KB of consecutive bytes and eight are in flight per thread, the access
// shape of the decode kernels' row loads.  Every thread folds what it read
// into one word and stores it (a plain vector store per thread), so the
// loads cannot be dropped.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* src,
                                                                   size_t n16, uint32_t* out) {
  constexpr int kUnroll = 8;
  constexpr size_t kSlice = static_cast<size_t>(kProbeThreads) * kUnroll;   // chunks
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kSlice; base < n16;
       base += static_cast<size_t>(gridDim.x) * kSlice) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kProbeThreads + tid;
      v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
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
