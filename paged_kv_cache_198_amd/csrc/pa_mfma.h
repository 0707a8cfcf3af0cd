// Matrix-core helpers shared by the decode and prefill kernels (gfx950):
// the 16x16x32 and 16x16x16 bf16/f16 MFMA, 16-bit KV bit patterns, raw
// buffer loads that return zero past a resource's end, and same-wavefront
// LDS ordering.
#pragma once

#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"

namespace pa {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

template <int DT>
__device__ __forceinline__ f32x4_t mma(const u16x8_t& a, const u16x8_t& b, const f32x4_t& c) {
  if constexpr (DT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// The 16x16x16 product (K = 16): A and B carry 4 16-bit values per lane.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mma16(const u16x4_t& a, const u16x4_t& b, const f32x4_t& c) {
  if constexpr (DT == PA_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                     __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// float -> 16-bit pattern of the KV type (round to nearest even) and back.
template <int DT>
__device__ __forceinline__ uint16_t to_bits(float x) {
  if constexpr (DT == PA_BF16) return narrow<PA_BF16>(x);
  else return __builtin_bit_cast(uint16_t, narrow<PA_F16>(x));
}
template <int DT>
__device__ __forceinline__ float from_bits(uint16_t b) {
  if constexpr (DT == PA_BF16) return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ u16x8_t as_u16x8(const uint4& v) {
  return __builtin_bit_cast(u16x8_t, v);
}

// bok[i] for a lane-dependent i < N (wave-uniform entries)
template <int N>
__device__ __forceinline__ bool pick_ok(const bool (&v)[N], int i) {
  bool r = v[0];
#pragma unroll
  for (int k = 1; k < N; ++k) r = (i == k) ? v[k] : r;
  return r;
}

// The per-wavefront LDS tile is written and read by the same wavefront,
// whose LDS operations the hardware performs in order; this only stops the
// compiler from moving LDS accesses across the point.
__device__ __forceinline__ void lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Max of x over lanes l, l^16, l^32 and l^48 (the four lane groups that hold
// one MFMA column), on the VALU: v_permlane16_swap exchanges rows 1 and 3
// of one copy with rows 0 and 2 of the other (a row is 16 lanes), so the
// max of the two copies is the max over lanes l and l^16; the 32-lane
// halves the same way.  Needs every lane active.
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a16 = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
  x = fmaxf(__builtin_bit_cast(float, a16[0]), __builtin_bit_cast(float, a16[1]));
  const auto a32 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, a32[0]), __builtin_bit_cast(float, a32[1]));
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x7ffffff0u;   // past every resource's end

// Raw buffer resource over [base, base + bytes): stride 0, the gfx9 data
// format word.  Loads at offsets >= bytes return zero and access nothing.
__device__ __forceinline__ rsrc_t make_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// 16-byte load; K/V are read once, so the non-temporal bit is set (cache
// policy operand: sc0 = 1, nt = 2, sc1 = 16).
__device__ __forceinline__ uint4 buffer_load16(rsrc_t r, uint32_t voff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), 0,
                                                          PA_DECODE_NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i receives element i%4 (16-bit) of the 8-byte chunks that the
// group's lanes 4e + i/4 (e = 0..3) point at.  For a row-major tile
// (token rows, 16-bit dims), lane j of group q pointing at row 4q + j/4,
// dims c + 4(j%4), gives lane i the values of dim c + i in rows 4q .. 4q+3:
// an MFMA operand column read across token rows.
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ v4s_t ds_read_tr16(const char* p) {   // p: LDS, 8-byte aligned
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(const_cast<char*>(p)));
}

// A operand of O^T += V^T P^T from a row-major 32-row tile of 16-bit rows
// (row stride `stride` bytes): lane (n, q) gets dims 16dt + n of rows
// 4q .. 4q+3 and 16+4q .. 16+4q+3 (the order the score tile leaves P^T in).
__device__ __forceinline__ u16x8_t vt_operand(const char* tile, int stride, int dt, int n,
                                              int q) {
  const char* p0 = tile + (4 * q + (n >> 2)) * stride + (16 * dt + 4 * (n & 3)) * 2;
  const v4s_t lo = ds_read_tr16(p0);
  const v4s_t hi = ds_read_tr16(p0 + 16 * stride);
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand of O^T += V^T P^T for a 16-row tile (the 16x16x16 product):
// lane (n, q) gets dims 16dt + n of rows 4q .. 4q+3.
__device__ __forceinline__ u16x4_t vt_operand16(const char* tile, int stride, int dt, int n,
                                                int q) {
  const char* p0 = tile + (4 * q + (n >> 2)) * stride + (16 * dt + 4 * (n & 3)) * 2;
  return __builtin_bit_cast(u16x4_t, ds_read_tr16(p0));
}

}  // namespace mfma
}  // namespace pa
