// Paged single-query decode attention for gfx950 (CDNA4).
//
// "PagedAttention: the KV cache was the bottleneck all along", section
// "Virtual memory for attention": each sequence's keys and values sit in
// fixed-size blocks scattered over the pool, found through its block table,
// and the attention kernel gathers them from there.  The attention itself is
// the textbook single-query softmax(scale * q.K^T).V.
//
// Work decomposition.  One workgroup of kWaves wavefronts per
// (KV head, sequence, context partition); the G query heads that share the KV
// head are all handled by that workgroup, so each K/V byte is read once.
//
// Data path inside a workgroup.  A token row of one head is D*elem bytes =
// RL lanes x 16 bytes (RL = 16 for D=128 at 2 bytes), so one dwordx4 load
// instruction of a wavefront fetches RPW = 64/RL whole token rows, contiguous
// inside one block.  Each lane keeps, for its 16-byte column chunk, the query
// elements of the G heads (pre-multiplied by scale*log2(e) so exp2 can be
// used), and an online-softmax state (running max m, sum l, output acc) per
// row group: the RPW row groups of a wave and the waves of a workgroup are
// independent partial softmaxes, merged once at the end (first across row
// groups with cross-lane shuffles, then across waves through LDS).  The q.k
// partial dot products are summed over the RL lanes of a row with DPP
// (quad_perm, row_half_mirror, row_mirror; ds_swizzle for 32 lanes), which
// leaves the full dot product in every lane of the row.
//
// A wavefront's token rows never straddle a block, so the block-table entry
// of each row group is wave-uniform.  The fused step's store in the loop
// could alias the table as far as the compiler knows, so it reads each entry
// with a vector load and waits for it before the tile's K/V loads; that
// paces each wavefront's requests, and measured faster than scalar reads of
// all of a tile's entries at once.  K/V rows go straight from HBM to
// registers (each byte is consumed by exactly one lane, so an LDS hop would
// add traffic without reuse).  Tiles wholly inside the context load without
// predication; in the last tile, tokens past the context are never loaded
// and their weights are exactly zero.
//
// Split context.  With partition_tokens > 0 each partition writes
// (m, l, unnormalised acc) in float32 to the workspace and reduce_kernel
// combines them: M = max_p m_p, out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.
// A sequence that fits in one partition is written directly.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = PA_DECODE_WAVES;   // wavefronts per workgroup
constexpr int kRows = PA_DECODE_ROWS;     // token rows per lane per tile (G < 4)
constexpr int kWideReduceParts = 16;      // reduce_wide_kernel from this many partitions on

template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeArgs a) {
  using T = typename KV<DT>::T;
  constexpr int EB = KV<DT>::kBytes;
  constexpr int VEC = 16 / EB;           // elements per lane chunk
  constexpr int RL = D * EB / 16;        // lanes per token row
  constexpr int RPW = 64 / RL;           // token rows per wave load
  constexpr int NL = (G >= 4) ? 4 : kRows;  // rows per lane per tile
  constexpr int TILE = NL * RPW;         // tokens per wave per tile
  constexpr float kNegInf = -INFINITY;

  __shared__ float red_acc[kWaves][G][D];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];

  const int g = blockIdx.x;
  const int p = blockIdx.z;
  const int tid = threadIdx.x;
  const int s = blockIdx.y;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane / RL;
  const int c = lane - r * RL;

  const int ctx = clamp_ctx(a, s, BS);
  const PartRange pr = part_range(a, s, p, ctx, BS > 32 ? BS : 32);
  const int nparts = pr.nparts;
  if (p >= nparts) return;
  const int start = pr.start;
  const int end = pr.end;

  float qf[G][VEC];
  {
    const T* qb = static_cast<const T*>(a.q) + (static_cast<size_t>(s) * a.Hq + g * G) * D + c * VEC;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      widen16<DT>(*reinterpret_cast<const uint4*>(qb + gi * D), qf[gi]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qf[gi][e] *= a.qscale;
    }
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = kNegInf;
    l[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[gi][e] = 0.f;
  }

  // Row group j of a tile starting at t0 holds tokens t0 + j*RPW + [0, RPW):
  // t0 is a multiple of RPW and RPW divides bs, so those RPW tokens share one
  // block and the block number is the same for the whole wavefront; the only
  // per-lane address term is the lane's row and 16-byte column.
  const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.MB;
  const size_t bstride = static_cast<size_t>(a.Hkv) * BS * D * EB;  // bytes per block
  const char* kb = static_cast<const char*>(a.key_cache) + static_cast<size_t>(g) * BS * D * EB;
  const char* vb = static_cast<const char*>(a.value_cache) + static_cast<size_t>(g) * BS * D * EB;
  const uint32_t lane_off = static_cast<uint32_t>((r * D + c * VEC) * EB);
  const int last_lb = end > 0 ? (end - 1) / BS : 0;
  const int wv = __builtin_amdgcn_readfirstlane(w);

  // Fused step: the last partition owns the new token at position c-1,
  // c = context_lens[s].  When c is the attended length (not clamped), the
  // lanes of that row, in the tile that holds it, take the new K/V rows of
  // head g from the inputs instead of the pool and store them into the slot.
  // A clamped length attends fewer tokens; the row is then only stored, after
  // the loop, as a separate cache write would store it.
  const int raw_ctx = a.context_lens[s];
  const bool owns_new = a.new_key != nullptr && raw_ctx > 0 && p == nparts - 1;
  const bool append = owns_new && raw_ctx == ctx;

  for (int t0 = start + wv * TILE; t0 < end; t0 += kWaves * TILE) {
    size_t off[NL];
    bool bok[NL];
    bool whole = t0 + TILE <= end;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int tj = t0 + j * RPW;
      const int blk = trow[min(tj / BS, last_lb)];
      bok[j] = static_cast<unsigned>(blk) < static_cast<unsigned>(a.NB);
      whole = whole && bok[j];
      off[j] = static_cast<size_t>(blk) * bstride + static_cast<size_t>(tj % BS) * (D * EB);
    }
    uint4 kr[NL], vr[NL];
    bool ok[NL];
    if (whole) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        kr[j] = load_kv(kb + off[j] + lane_off);
        vr[j] = load_kv(vb + off[j] + lane_off);
        ok[j] = true;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        ok[j] = bok[j] && t0 + j * RPW + r < end;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (ok[j]) {
          kv = load_kv(kb + off[j] + lane_off);
          vv = load_kv(vb + off[j] + lane_off);
        }
        kr[j] = kv;
        vr[j] = vv;
      }
    }
    if (append && t0 <= ctx - 1 && ctx - 1 < t0 + TILE) {
      const int rel = ctx - 1 - t0;
      if (r == rel % RPW) {
        const size_t src = (static_cast<size_t>(s) * a.Hkv + g) * D * EB + c * 16;
        const uint4 nk = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.new_key) + src);
        const uint4 nv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.new_value) + src);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          if (j == rel / RPW) {
            kr[j] = nk;
            vr[j] = nv;
            if (bok[j]) {
              *reinterpret_cast<uint4*>(const_cast<char*>(kb) + off[j] + lane_off) = nk;
              *reinterpret_cast<uint4*>(const_cast<char*>(vb) + off[j] + lane_off) = nv;
            }
          }
        }
      }
    }

    // logits (log2 domain) for the NL rows of this lane, every head
    float sc[NL][G];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float kf[VEC];
      widen16<DT>(kr[j], kf);
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qf[gi][e], kf[e], d);
        sc[j][gi] = row_sum<RL>(d);
      }
    }

    // online softmax: rescale once per tile, then accumulate
    float pw[NL][G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float mt = kNegInf;
#pragma unroll
      for (int j = 0; j < NL; ++j) mt = ok[j] ? fmaxf(mt, sc[j][gi]) : mt;
      const float mn = fmaxf(m[gi], mt);
      const float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m[gi] - mn);
      l[gi] *= alpha;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[gi][e] *= alpha;
      m[gi] = mn;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        pw[j][gi] = ok[j] ? fast_exp2(sc[j][gi] - mn) : 0.f;
        l[gi] += pw[j][gi];
      }
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float vf[VEC];
      widen16<DT>(vr[j], vf);
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[gi][e] = fmaf(pw[j][gi], vf[e], acc[gi][e]);
    }
  }

  if (owns_new && raw_ctx > ctx && w == 0 && r == 0) {
    // the new token lies past the attended range: store only
    const int pos = raw_ctx - 1;
    if (pos / BS < a.MB) {
      const int blk = trow[pos / BS];
      if (static_cast<unsigned>(blk) < static_cast<unsigned>(a.NB)) {
        const size_t src = (static_cast<size_t>(s) * a.Hkv + g) * D * EB + c * 16;
        const size_t dst = static_cast<size_t>(blk) * bstride +
                           static_cast<size_t>(pos % BS) * (D * EB) + c * 16;
        *reinterpret_cast<uint4*>(const_cast<char*>(kb) + dst) =
            *reinterpret_cast<const uint4*>(static_cast<const char*>(a.new_key) + src);
        *reinterpret_cast<uint4*>(const_cast<char*>(vb) + dst) =
            *reinterpret_cast<const uint4*>(static_cast<const char*>(a.new_value) + src);
      }
    }
  }

  // merge the RPW row groups of the wave
#pragma unroll
  for (int off = RL; off < 64; off <<= 1) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float mo = __shfl_xor(m[gi], off);
      const float lo = __shfl_xor(l[gi], off);
      const float mn = fmaxf(m[gi], mo);
      const float sa = (m[gi] == kNegInf) ? 0.f : fast_exp2(m[gi] - mn);
      const float sb = (mo == kNegInf) ? 0.f : fast_exp2(mo - mn);
      l[gi] = l[gi] * sa + lo * sb;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = __shfl_xor(acc[gi][e], off);
        acc[gi][e] = acc[gi][e] * sa + ao * sb;
      }
      m[gi] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) red_acc[w][gi][c * VEC + e] = acc[gi][e];
      if (c == 0) {
        red_m[w][gi] = m[gi];
        red_l[w][gi] = l[gi];
      }
    }
  }
  lds_barrier();

  // merge the waves; one thread per (head, element)
  for (int i = tid; i < G * D; i += kWaves * 64) {
    const int gi = i / D;
    const int d = i - gi * D;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, red_m[v][gi]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float mv = red_m[v][gi];
      const float sw = (mv == kNegInf) ? 0.f : fast_exp2(mv - M);
      num = fmaf(red_acc[v][gi][d], sw, num);
      den = fmaf(red_l[v][gi], sw, den);
    }
    const int h = g * G + gi;
    if (pr.total == 1) {
      static_cast<T*>(a.out)[(static_cast<size_t>(s) * a.Hq + h) * D + d] =
          narrow<DT>(den > 0.f ? num / den : 0.f);
    } else if (pr.slot < a.pmax) {
      const size_t idx = (static_cast<size_t>(s) * a.Hq + h) * a.pmax + pr.slot;
      a.ws_o[idx * D + d] = num;
      if (d == 0) {
        a.ws_m[idx] = M;
        a.ws_l[idx] = den;
      }
    }
  }
}

// Combine the partitions of sequences longer than one partition.  One
// workgroup per (query head, sequence) and one thread per output element.
// The per-partition max and sum are the same for the whole workgroup (read
// with scalar loads); the partial outputs are summed with eight independent
// accumulators so that eight loads are in flight per thread.
template <int DT, int D, int BS>
__global__ __launch_bounds__(D) void reduce_kernel(DecodeArgs a) {
  using T = typename KV<DT>::T;
  constexpr float kNegInf = -INFINITY;
  constexpr int U = 8;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int ctx = clamp_ctx(a, s, BS);
  const int nparts = part_range(a, s, 0, ctx, BS > 32 ? BS : 32).total;
  if (nparts <= 1) return;
  const size_t base = (static_cast<size_t>(s) * a.Hq + h) * a.pmax;
  const float* mp = a.ws_m + base;
  const float* lp = a.ws_l + base;
  const float* op = a.ws_o + base * D + d;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, mp[p]);
  float num[U], den[U];
#pragma unroll
  for (int k = 0; k < U; ++k) num[k] = den[k] = 0.f;
  int p = 0;
  for (; p + U <= nparts; p += U) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const float mk = mp[p + k];
      const float sw = (mk == kNegInf) ? 0.f : fast_exp2(mk - M);
      num[k] = fmaf(op[static_cast<size_t>(p + k) * D], sw, num[k]);
      den[k] = fmaf(lp[p + k], sw, den[k]);
    }
  }
  for (; p < nparts; ++p) {
    const float mk = mp[p];
    const float sw = (mk == kNegInf) ? 0.f : fast_exp2(mk - M);
    num[0] = fmaf(op[static_cast<size_t>(p) * D], sw, num[0]);
    den[0] = fmaf(lp[p], sw, den[0]);
  }
  float nt = 0.f, dn = 0.f;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    nt += num[k];
    dn += den[k];
  }
  static_cast<T*>(a.out)[(static_cast<size_t>(s) * a.Hq + h) * D + d] =
      narrow<DT>(dn > 0.f ? nt / dn : 0.f);
}

// The (query head, sequence) a wide-reduce workgroup combines.  With Hkv a
// multiple of 8 the main pass writes every partial of KV head g on XCD
// g % 8 (the hardware hands consecutive workgroups to the XCDs in turn), so
// (s, h) goes to the workgroup that runs on XCD (h / G) % 8, the one that
// wrote its partials.  On the long-context batch that took 2 us off the
// step, with the same bytes fetched from memory (the partials are not L2
// hits; the gain is in the placement's timing, not in traffic).  For the few
// partials of reduce_kernel the grid's own order measured faster.
__device__ __forceinline__ void wide_reduce_item(const DecodeArgs& a, int& h, int& s) {
  if (a.Hkv % 8) {
    h = blockIdx.x;
    s = blockIdx.y;
    return;
  }
  const int id = blockIdx.x + gridDim.x * blockIdx.y;
  const int x = id & 7, k = id >> 3, per = a.Hq >> 3, G = a.Hq / a.Hkv;
  s = k / per;
  const int j = k - s * per;
  h = (x + 8 * (j / G)) * G + j % G;
}

// The same combination for many partitions (long contexts).  One workgroup
// of 256 threads per (query head, sequence): a partition's row of D floats is
// read by D/4 threads with 16-byte loads, and the 256/(D/4) thread groups
// take every NG-th partition, four at a time, so 4 NG partition rows of a
// (sequence, head) are in flight at once (32 at D = 128, 64 at D = 64).  The
// groups' partial sums meet in LDS.  With few partitions most groups would idle behind the barrier, so
// the host picks this kernel only from kWideReduceParts partitions on.
template <int DT, int D, int BS>
__global__ __launch_bounds__(256) void reduce_wide_kernel(DecodeArgs a) {
  using T = typename KV<DT>::T;
  constexpr float kNegInf = -INFINITY;
  constexpr int TPR = D / 4;               // threads per partition row
  constexpr int NG = 256 / TPR;            // partition groups
  constexpr int U = 4;                     // partitions per group in flight
  __shared__ float4 gnum[NG][TPR];
  __shared__ float gden[NG];
  int h, s;
  wide_reduce_item(a, h, s);
  const int t = threadIdx.x;
  const int grp = t / TPR;
  const int c = t - grp * TPR;
  const int ctx = clamp_ctx(a, s, BS);
  const int nparts = part_range(a, s, 0, ctx, BS > 32 ? BS : 32).total;
  if (nparts <= 1) return;
  const size_t base = (static_cast<size_t>(s) * a.Hq + h) * a.pmax;
  const float* mp = a.ws_m + base;
  const float* lp = a.ws_l + base;
  const float4* op = reinterpret_cast<const float4*>(a.ws_o + base * D) + c;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, mp[p]);
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  auto add = [&](const float4& v, float mk, float lk) {
    const float sw = (mk == kNegInf) ? 0.f : fast_exp2(mk - M);
    num.x = fmaf(v.x, sw, num.x);
    num.y = fmaf(v.y, sw, num.y);
    num.z = fmaf(v.z, sw, num.z);
    num.w = fmaf(v.w, sw, num.w);
    den = fmaf(lk, sw, den);
  };
  int p = grp;
  for (; p + (U - 1) * NG < nparts; p += U * NG) {
    float4 v[U];
    float mk[U], lk[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      v[k] = op[static_cast<size_t>(p + k * NG) * TPR];
      mk[k] = mp[p + k * NG];
      lk[k] = lp[p + k * NG];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) add(v[k], mk[k], lk[k]);
  }
  for (; p < nparts; p += NG) add(op[static_cast<size_t>(p) * TPR], mp[p], lp[p]);
  gnum[grp][c] = num;
  if (c == 0) gden[grp] = den;
  __syncthreads();
  if (t < TPR) {
    float4 nt = make_float4(0.f, 0.f, 0.f, 0.f);
    float dn = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      nt.x += gnum[k][t].x;
      nt.y += gnum[k][t].y;
      nt.z += gnum[k][t].z;
      nt.w += gnum[k][t].w;
      dn += gden[k];
    }
    const float inv = dn > 0.f ? 1.f / dn : 0.f;
    T* o = static_cast<T*>(a.out) + (static_cast<size_t>(s) * a.Hq + h) * D + 4 * t;
    o[0] = narrow<DT>(nt.x * inv);
    o[1] = narrow<DT>(nt.y * inv);
    o[2] = narrow<DT>(nt.z * inv);
    o[3] = narrow<DT>(nt.w * inv);
  }
}

template <int DT, int D, int BS, int G>
int launch_decode(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<DT, D, BS, G>),
                     dim3(static_cast<uint32_t>(a.Hkv), static_cast<uint32_t>(a.S),
                          static_cast<uint32_t>(a.grid_parts)),
                     dim3(kWaves * 64), 0, st, a);
  return launch_status();
}

template <int DT, int D, int BS>
int launch_reduce(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(a.Hq), static_cast<uint32_t>(a.S));
  if (a.pmax >= kWideReduceParts)
    hipLaunchKernelGGL((reduce_wide_kernel<DT, D, BS>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((reduce_kernel<DT, D, BS>), grid, dim3(D), 0, st, a);
  return launch_status();
}

template <int DT, int D>
int dispatch_reduce(const DecodeArgs& a, int bs, hipStream_t st) {
  switch (bs) {
    case 8: return launch_reduce<DT, D, 8>(a, st);
    case 16: return launch_reduce<DT, D, 16>(a, st);
    case 32: return launch_reduce<DT, D, 32>(a, st);
    case 64: return launch_reduce<DT, D, 64>(a, st);
    case 128: return launch_reduce<DT, D, 128>(a, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <int DT>
int dispatch_reduce_d(const DecodeArgs& a, int D, int bs, hipStream_t st) {
  return D == 64 ? dispatch_reduce<DT, 64>(a, bs, st) : dispatch_reduce<DT, 128>(a, bs, st);
}

template <int DT, int D, int BS>
int dispatch_g(const DecodeArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_decode<DT, D, BS, 1>(a, st);
    case 2: return launch_decode<DT, D, BS, 2>(a, st);
    case 4: return launch_decode<DT, D, BS, 4>(a, st);
    case 8: return launch_decode<DT, D, BS, 8>(a, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <int DT, int D>
int dispatch_bs(const DecodeArgs& a, int bs, int G, hipStream_t st) {
  switch (bs) {
    case 8: return dispatch_g<DT, D, 8>(a, G, st);
    case 16: return dispatch_g<DT, D, 16>(a, G, st);
    case 32: return dispatch_g<DT, D, 32>(a, G, st);
    case 64: return dispatch_g<DT, D, 64>(a, G, st);
    case 128: return dispatch_g<DT, D, 128>(a, G, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

template <int DT>
int dispatch_d(const DecodeArgs& a, int D, int bs, int G, hipStream_t st) {
  switch (D) {
    case 64: return dispatch_bs<DT, 64>(a, bs, G, st);
    case 128: return dispatch_bs<DT, 128>(a, bs, G, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

inline int32_t num_partitions(int32_t max_ctx, int32_t part_tokens) {
  return part_tokens > 0 ? (max_ctx + part_tokens - 1) / part_tokens : 1;
}

}  // namespace pa

extern "C" size_t pa_decode_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                            int32_t max_context_len, int32_t partition_tokens) {
  if (S <= 0 || Hq <= 0 || D <= 0 || max_context_len <= 0 || partition_tokens <= 0) return 0;
  const int32_t pmax = pa::num_partitions(max_context_len, partition_tokens);
  if (pmax <= 1) return 0;
  const size_t n = static_cast<size_t>(S) * Hq * pmax;
  return 2 * pa::align256(n * sizeof(float)) + pa::align256(n * D * sizeof(float));
}

extern "C" size_t pa_cascade_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                             int32_t slots_max) {
  if (S <= 0 || Hq <= 0 || D <= 0 || slots_max <= 1) return 0;
  const size_t n = static_cast<size_t>(S) * Hq * slots_max;
  return 2 * pa::align256(n * sizeof(float)) + pa::align256(n * D * sizeof(float));
}

namespace pa {
namespace {

// A cascade plan on the device (seq_start[S], slot_base[S], items) and its
// host-side sizes.
struct Cascade {
  const int32_t* plan;
  int32_t n_items, slots_max;
};

int decode_impl(void* out, const void* query, const void* new_key, const void* new_value,
                const void* key_cache, const void* value_cache, const int32_t* block_tables,
                const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                int32_t bs, int32_t NB, int32_t MB, int32_t max_context_len, float scale,
                int32_t partition_tokens, void* workspace, size_t workspace_bytes, int32_t dtype,
                void* stream, const Cascade* cas = nullptr) {
  if (pa::elem_bytes(dtype) == 0) return PA_ERR_INVALID;
  if (S < 0 || Hq < 1 || Hkv < 1 || D < 1 || bs < 1 || NB < 1 || MB < 1) return PA_ERR_INVALID;
  if (max_context_len < 1 || partition_tokens < 0) return PA_ERR_INVALID;
  if (partition_tokens > 0 && partition_tokens % bs) return PA_ERR_INVALID;
  if (Hq % Hkv) return PA_ERR_INVALID;
  if (!std::isfinite(scale)) return PA_ERR_INVALID;
  if (S == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID;
  if (!pa::aligned16(out) || !pa::aligned16(query) || !pa::aligned16(key_cache) ||
      !pa::aligned16(value_cache))
    return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PA_ERR_INVALID;
  const int G = Hq / Hkv;
  if (D != 64 && D != 128) return PA_ERR_UNSUPPORTED;
  if (bs != 8 && bs != 16 && bs != 32 && bs != 64 && bs != 128) return PA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  const int32_t eff_ctx = static_cast<int32_t>(
      std::min<int64_t>(max_context_len, static_cast<int64_t>(MB) * bs));
  int32_t pmax = pa::num_partitions(eff_ctx, partition_tokens);
  int32_t grid_parts = pmax;
  if (cas) {
    // the prefix pass runs on the matrix cores only
    if ((dtype != PA_BF16 && dtype != PA_F16) || D != 128) return PA_ERR_UNSUPPORTED;
    if (!cas->plan || (reinterpret_cast<uintptr_t>(cas->plan) & 3u)) return PA_ERR_INVALID;
    if (cas->n_items < 0 || cas->slots_max < 1) return PA_ERR_INVALID;
    if (cas->n_items > 65535) return PA_ERR_UNSUPPORTED;
    pmax = cas->slots_max;
    grid_parts = 1;
  }
  if (S > 65535 || pmax > 65535) return PA_ERR_UNSUPPORTED;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.NB = NB;
  a.MB = MB;
  a.max_ctx = eff_ctx;
  a.part_tokens = (pmax > 1 || cas) ? partition_tokens : 0;
  a.pmax = pmax;
  a.grid_parts = grid_parts;
  a.qscale = scale * pa::kLog2e;
  a.new_key = new_key;
  a.new_value = new_value;
  if (cas) {
    a.seq_start = cas->plan;
    a.slot_base = cas->plan + S;
    a.items = cas->plan + 2 * static_cast<size_t>(S);
    a.n_items = cas->n_items;
  }
  if (pmax > 1) {
    const size_t need = cas ? pa_cascade_workspace_bytes(S, Hq, D, pmax)
                            : pa_decode_workspace_bytes(S, Hq, D, eff_ctx, partition_tokens);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return PA_ERR_WORKSPACE;
    const size_t n = static_cast<size_t>(S) * Hq * pmax;
    char* base = static_cast<char*>(workspace);
    a.ws_m = reinterpret_cast<float*>(base);
    a.ws_l = reinterpret_cast<float*>(base + pa::align256(n * sizeof(float)));
    a.ws_o = reinterpret_cast<float*>(base + 2 * pa::align256(n * sizeof(float)));
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Grouped heads that fill a matrix-core tile go to the MFMA kernel; every
  // other shape runs the vector-ALU kernel.
  const bool mfma = (dtype == PA_BF16 || dtype == PA_F16) && D == 128 && G == 8;
  int rc;
  if (cas) {
    rc = pa::launch_items_mfma(a, dtype, bs, st);
  } else if (mfma) {
    rc = pa::launch_decode_gqa_mfma(a, dtype, bs, st);
  } else {
    switch (dtype) {
      case PA_F32: rc = pa::dispatch_d<PA_F32>(a, D, bs, G, st); break;
      case PA_F16: rc = pa::dispatch_d<PA_F16>(a, D, bs, G, st); break;
      default: rc = pa::dispatch_d<PA_BF16>(a, D, bs, G, st); break;
    }
  }
  if (rc != PA_OK || pmax <= 1) return rc;
  switch (dtype) {
    case PA_F32: return pa::dispatch_reduce_d<PA_F32>(a, D, bs, st);
    case PA_F16: return pa::dispatch_reduce_d<PA_F16>(a, D, bs, st);
    default: return pa::dispatch_reduce_d<PA_BF16>(a, D, bs, st);
  }
}

}  // namespace
}  // namespace pa

extern "C" int pa_decode_attention(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t S, int32_t Hq,
                                   int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t MB,
                                   int32_t max_context_len, float scale,
                                   int32_t partition_tokens, void* workspace,
                                   size_t workspace_bytes, int32_t dtype, void* stream) {
  return pa::decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                         context_lens, S, Hq, Hkv, D, bs, NB, MB, max_context_len, scale,
                         partition_tokens, workspace, workspace_bytes, dtype, stream);
}

extern "C" int pa_decode_step(void* out, const void* query, const void* key, const void* value,
                              void* key_cache, void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t bs, int32_t NB, int32_t MB,
                              int32_t max_context_len, float scale, int32_t partition_tokens,
                              void* workspace, size_t workspace_bytes, int32_t dtype,
                              void* stream) {
  if (S > 0 && (!key || !value || !pa::aligned16(key) || !pa::aligned16(value)))
    return PA_ERR_INVALID;
  return pa::decode_impl(out, query, key, value, key_cache, value_cache, block_tables,
                         context_lens, S, Hq, Hkv, D, bs, NB, MB, max_context_len, scale,
                         partition_tokens, workspace, workspace_bytes, dtype, stream);
}

extern "C" int pa_decode_cascade(void* out, const void* query, const void* key,
                                 const void* value, void* key_cache, void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* plan, int32_t n_items, int32_t slots_max,
                                 int32_t S, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t bs, int32_t NB, int32_t MB,
                                 int32_t max_context_len, float scale, int32_t partition_tokens,
                                 void* workspace, size_t workspace_bytes, int32_t dtype,
                                 void* stream) {
  if ((key == nullptr) != (value == nullptr)) return PA_ERR_INVALID;
  if (key && (!pa::aligned16(key) || !pa::aligned16(value))) return PA_ERR_INVALID;
  const pa::Cascade cas{plan, n_items, slots_max};
  return pa::decode_impl(out, query, key, value, key_cache, value_cache, block_tables,
                         context_lens, S, Hq, Hkv, D, bs, NB, MB, max_context_len, scale,
                         partition_tokens, workspace, workspace_bytes, dtype, stream, &cas);
}

// ---------------------------------------------------------------------------
// The fused step for callers that cannot allocate: the split-context partials
// live in this file-scope array (one copy per GPU, held until the process
// ends).  Host code never passes the array's name to a kernel: it is a host
// stand-in, not a device address.  The address on each device comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

extern "C" int pa_decode_step_noalloc(void* out, const void* query, const void* key,
                                      const void* value, void* key_cache, void* value_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                                      int32_t NB, int32_t MB, int32_t max_context_len,
                                      float scale, int32_t partition_tokens, int32_t dtype,
                                      void* stream) {
  if (bs < 1 || MB < 1 || max_context_len < 1) return PA_ERR_INVALID;
  const int32_t eff_ctx = static_cast<int32_t>(
      std::min<int64_t>(max_context_len, static_cast<int64_t>(MB) * bs));
  const size_t need = pa_decode_workspace_bytes(S, Hq, D, eff_ctx, partition_tokens);
  if (need > PA_STATIC_SCRATCH_BYTES) return PA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    const int rc = pa::scratch_on_current_device(&ws);
    if (rc != PA_OK) return rc;
  }
  return pa_decode_step(out, query, key, value, key_cache, value_cache, block_tables,
                        context_lens, S, Hq, Hkv, D, bs, NB, MB, max_context_len, scale,
                        partition_tokens, ws, need > 0 ? PA_STATIC_SCRATCH_BYTES : 0, dtype,
                        stream);
}
