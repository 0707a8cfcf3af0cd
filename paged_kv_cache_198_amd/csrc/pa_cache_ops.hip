// Cache write and copy-on-write block copy for the paged KV cache (gfx950).
//
// Both are pure data movement: every thread moves one 16-byte chunk with a
// dwordx4 load and store, so a wavefront touches 1 KiB of contiguous row data
// per instruction.  Element type does not matter (rows are copied as bytes).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

// Bytes of K and V rows up to which the cache write streams its stores out
// with the non-temporal hint: the 8 XCDs' L2s hold 32 MiB.  A decode step's
// rows (a few MB scattered over the pool) stored the default way stay dirty
// in the L2s and are written back when the launch ends; streamed, the
// two-call decode step measured about 1% faster.  A prompt fill (hundreds of
// MB) keeps the default policy, under which the prefill step that follows
// measured faster.
constexpr int64_t kStreamWriteMax = int64_t(32) << 20;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// "Virtual memory for attention": a new token's key and value rows go to the
// slot its sequence's block table gives it.  One thread per 16-byte chunk of
// the [T][Hkv][D] inputs; chunk c of (t, h) lands at
// ((slot/bs * Hkv + h) * bs + slot%bs) * cpr + c in the [NB][Hkv][bs][D] pool.
template <bool NT>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value,
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int64_t* __restrict__ slot_mapping, int64_t total_chunks, int32_t hkv_cpr,
    int32_t cpr, int32_t Hkv, int32_t bs, int64_t num_slots) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total_chunks) return;
  const int64_t t = i / hkv_cpr;
  const int32_t rem = static_cast<int32_t>(i - t * hkv_cpr);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int32_t h = rem / cpr;
  const int32_t c = rem - h * cpr;
  const int64_t blk = slot / bs;
  const int64_t off = slot - blk * bs;
  const int64_t dst = ((blk * Hkv + h) * bs + off) * cpr + c;
  if constexpr (NT) {
    const uint4 k = key[i], v = value[i];
    __builtin_nontemporal_store(u32x4_t{k.x, k.y, k.z, k.w},
                                reinterpret_cast<u32x4_t*>(key_cache + dst));
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                reinterpret_cast<u32x4_t*>(value_cache + dst));
  } else {
    key_cache[dst] = key[i];
    value_cache[dst] = value[i];
  }
}

// Copy-on-write: pairs and per-layer pool pointers travel in the kernel
// arguments (they come from the host allocator), so a copy needs no
// host-to-device transfer of metadata.
constexpr int kCopyMaxLayers = 16;
constexpr int kCopyMaxPairs = 96;

struct CopyArgs {
  uint4* pools[2 * kCopyMaxLayers];  // layer l: [2l] keys, [2l+1] values
  int64_t src[kCopyMaxPairs];
  int64_t dst[kCopyMaxPairs];
  int64_t chunks_per_block;          // block_bytes / 16
};

// grid: x = chunk groups of one block, y = pair, z = pool (2 per layer)
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= a.chunks_per_block) return;
  uint4* pool = a.pools[blockIdx.z];
  const int64_t n = a.chunks_per_block;
  pool[a.dst[blockIdx.y] * n + c] = pool[a.src[blockIdx.y] * n + c];
}

}  // namespace pa

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int32_t T,
                                    int32_t Hkv, int32_t D, int32_t bs, int32_t NB,
                                    int32_t dtype, void* stream) {
  const int eb = pa::elem_bytes(dtype);
  if (eb == 0) return PA_ERR_INVALID;
  if (T < 0 || Hkv < 1 || D < 1 || bs < 1 || NB < 0) return PA_ERR_INVALID;
  if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
  if (T == 0 || NB == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PA_ERR_INVALID;
  if (!pa::aligned16(key) || !pa::aligned16(value) || !pa::aligned16(key_cache) ||
      !pa::aligned16(value_cache))
    return PA_ERR_INVALID;
  const int32_t cpr = D * eb / 16;
  const int64_t total = static_cast<int64_t>(T) * Hkv * cpr;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return PA_ERR_INVALID;
  const bool stream_out = 2 * total * 16 <= pa::kStreamWriteMax;
  hipLaunchKernelGGL(stream_out ? pa::cache_write_kernel<true> : pa::cache_write_kernel<false>,
                     dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), static_cast<uint4*>(key_cache),
                     static_cast<uint4*>(value_cache), slot_mapping, total, Hkv * cpr, cpr, Hkv,
                     bs, static_cast<int64_t>(NB) * bs);
  return pa::launch_status();
}

extern "C" int pa_copy_blocks(void* const* key_caches, void* const* value_caches, int32_t L,
                              const int64_t* block_mapping, int32_t n, int32_t NB,
                              int64_t block_bytes, void* stream) {
  if (L < 0 || n < 0 || NB < 0) return PA_ERR_INVALID;
  if (L == 0 || n == 0) return PA_OK;
  if (!key_caches || !value_caches || !block_mapping) return PA_ERR_INVALID;
  if (block_bytes <= 0 || block_bytes % 16) return PA_ERR_INVALID;
  for (int32_t l = 0; l < L; ++l) {
    if (!key_caches[l] || !value_caches[l]) return PA_ERR_INVALID;
    if (!pa::aligned16(key_caches[l]) || !pa::aligned16(value_caches[l])) return PA_ERR_INVALID;
  }
  // Independence rules: blocks in range, src != dst, dsts distinct, no dst
  // used as a src.  Quadratic in n only for small n; pair lists here are short.
  std::vector<char> is_dst(static_cast<size_t>(NB), 0), is_src(static_cast<size_t>(NB), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = block_mapping[2 * i], d = block_mapping[2 * i + 1];
    if (s < 0 || s >= NB || d < 0 || d >= NB || s == d) return PA_ERR_INVALID;
    if (is_dst[d]) return PA_ERR_INVALID;
    is_dst[d] = 1;
    is_src[s] = 1;
  }
  for (int32_t i = 0; i < n; ++i)
    if (is_src[block_mapping[2 * i + 1]]) return PA_ERR_INVALID;

  const int64_t chunks = block_bytes / 16;
  const int64_t gx = (chunks + 255) / 256;
  if (gx > 0x7fffffff) return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int32_t l0 = 0; l0 < L; l0 += pa::kCopyMaxLayers) {
    const int32_t nl = std::min(pa::kCopyMaxLayers, L - l0);
    for (int32_t p0 = 0; p0 < n; p0 += pa::kCopyMaxPairs) {
      const int32_t np = std::min(pa::kCopyMaxPairs, n - p0);
      pa::CopyArgs a{};
      for (int32_t l = 0; l < nl; ++l) {
        a.pools[2 * l] = static_cast<uint4*>(key_caches[l0 + l]);
        a.pools[2 * l + 1] = static_cast<uint4*>(value_caches[l0 + l]);
      }
      for (int32_t i = 0; i < np; ++i) {
        a.src[i] = block_mapping[2 * (p0 + i)];
        a.dst[i] = block_mapping[2 * (p0 + i) + 1];
      }
      a.chunks_per_block = chunks;
      hipLaunchKernelGGL(pa::copy_blocks_kernel,
                         dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(np),
                              static_cast<uint32_t>(2 * nl)),
                         dim3(256), 0, st, a);
      const int rc = pa::launch_status();
      if (rc != PA_OK) return rc;
    }
  }
  return PA_OK;
}
