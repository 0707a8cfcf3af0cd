// Device-side helpers shared by the decode kernels (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "pa.h"

namespace pa {

constexpr float kLog2e = 1.44269504088896340736f;
// Tuning (measured on the 13B- and 7B-shaped batches, see profiles/): 8
// waves per workgroup and 3 rows per lane per tile (12 tokens per wave at
// D = 128, 2 bytes: 68 VGPRs, 3 workgroups per CU; 8 rows hold 113 VGPRs and
// allow 2, with more bytes in flight per CU than the memory system serves
// best); non-temporal K/V loads raise the achieved read bandwidth by about
// 12%.
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 8
#endif
#ifndef PA_DECODE_ROWS
#define PA_DECODE_ROWS 3
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif



typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// K/V rows are read exactly once: optionally mark the loads non-temporal.
__device__ __forceinline__ uint4 load_kv(const void* p) {
#if PA_DECODE_NT
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

template <int DT> struct KV;
template <> struct KV<PA_F32> { using T = float; static constexpr int kBytes = 4; };
template <> struct KV<PA_F16> { using T = _Float16; static constexpr int kBytes = 2; };
template <> struct KV<PA_BF16> { using T = uint16_t; static constexpr int kBytes = 2; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// 16 bytes of stored elements -> float32.
template <int DT>
__device__ __forceinline__ void widen16(const uint4& c, float* f) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  if constexpr (DT == PA_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(float, w[i]);
  } else if constexpr (DT == PA_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t h = __builtin_bit_cast(half2_t, w[i]);
      f[2 * i] = static_cast<float>(h.x);
      f[2 * i + 1] = static_cast<float>(h.y);
    }
  } else {
    // bfloat16 is the upper half of a float32.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
}

// float32 -> stored element, round to nearest even.
template <int DT>
__device__ __forceinline__ typename KV<DT>::T narrow(float x) {
  if constexpr (DT == PA_F32) {
    return x;
  } else if constexpr (DT == PA_F16) {
    return static_cast<_Float16>(x);
  } else {
    // round to nearest even; a NaN stays a (quiet) NaN.  Both results are
    // formed and one selected, so no lane branches.
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? nan : rne);
  }
}

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Sum over the RL consecutive lanes of a token row; every lane of the row
// ends with the same value (each step adds a value and its partner's, and
// float addition is commutative).
template <int RL>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(RL == 8 || RL == 16 || RL == 32, "row width");
  x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: quads 0<->1 of each 8
  if constexpr (RL >= 16) x += dpp<0x140>(x);  // row_mirror: halves of a 16-lane row
  if constexpr (RL >= 32)                      // lane ^ 16 inside each 32
    x += __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS accesses only.  On this architecture one
// counter tracks both vector-memory loads and stores, so a full
// __syncthreads() makes a wavefront wait there until its global stores (the
// fused step's new row) have completed; this barrier does not, and nothing
// in the workgroup reads those stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A block-table entry at a wavefront-uniform index, read through the
// constant address space: the table is never written during a launch, and
// loads from that space at uniform addresses become scalar loads even after
// stores or memory barriers in the kernel (a vector load of the entry would
// wait on the vector-memory counter, i.e. for every K/V load issued before it).
__device__ __forceinline__ int32_t table_entry(const int32_t* row, int i) {
  return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(row))[i];
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  // Fused step (pa_decode_step): the token at position ctx-1 of each
  // sequence, [S][Hkv][D]; null for plain attention.  The workgroup that
  // owns that position writes it into its slot and uses it without reading
  // the pool.
  const void* new_key;
  const void* new_value;
  // Prefix sharing (pa_decode_cascade), null otherwise: sequence s's own
  // tokens start at seq_start[s]; its partitions write workspace slots from
  // slot_base[s] on, the slots below holding shared-prefix partials.
  const int32_t* seq_start;
  const int32_t* slot_base;
  // Shared-prefix work items, kItemInts ints each (see pa_cascade_plan).
  const int32_t* items;
  int32_t n_items;

  int32_t S, Hq, Hkv, NB, MB, max_ctx;
  int32_t part_tokens;  // 0: one pass over the whole context
  int32_t pmax;         // workspace slots per (sequence, query head)
  int32_t grid_parts;   // partitions per sequence in the main grid
  float qscale;         // scale * log2(e)
};

// Shared-prefix work item: table row, token start, token end, workspace
// slot, member count, then up to kItemMembers member rows (-1 = unused).
constexpr int kItemMembers = 16;
constexpr int kItemInts = 5 + kItemMembers;

// Token range [start, end) and workspace slot of partition p of sequence s.
// Plain decode: [p*PT, (p+1)*PT) clipped to ctx, slot p; a sequence that has
// one partition is written straight to the output (total == 1), and one
// with no tokens still gets a partition that writes zeros.  With prefix
// sharing, partitions cover [seq_start[s], ctx) and use slots from
// slot_base[s] on.
struct PartRange {
  int start, end, slot, nparts, total;
};

// `align` (a multiple of the caller's tile and of bs) rounds seq_start
// down, so tiles and row groups always start on the boundaries the kernels
// assume.
__device__ __forceinline__ PartRange part_range(const DecodeArgs& a, int s, int p, int ctx,
                                                int align) {
  const int s0 = a.seq_start ? min(max(a.seq_start[s], 0) / align * align, ctx) : 0;
  const int base = a.slot_base ? min(max(a.slot_base[s], 0), a.pmax) : 0;
  const int len = ctx - s0;
  const int PT = a.part_tokens > 0 ? a.part_tokens : max(len, 1);
  int nparts = (len + PT - 1) / PT;
  if (base == 0) nparts = max(nparts, 1);
  PartRange r;
  r.nparts = nparts;
  r.total = min(base + nparts, a.pmax);   // never more slots than the workspace holds
  r.start = s0 + p * PT;
  r.end = min(ctx, r.start + PT);
  r.slot = base + p;
  return r;
}

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int s, int bs) {
  const int c = a.context_lens[s];
  return max(0, min(c, min(a.max_ctx, a.MB * bs)));
}

// Launches the grouped-query MFMA main pass (bf16 / f16, D = 128, G = 8)
// for the partitions in `a`; returns PA_ERR_UNSUPPORTED for other shapes.
int launch_decode_gqa_mfma(const DecodeArgs& a, int32_t dtype, int32_t bs, hipStream_t st);

// Launches the work items in a.items (bf16 / f16, D = 128).
int launch_items_mfma(const DecodeArgs& a, int32_t dtype, int32_t bs, hipStream_t st);

}  // namespace pa
