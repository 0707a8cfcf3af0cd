// Paged prefill attention on the gfx950 matrix cores.
//
// "PagedAttention: the KV cache was the bottleneck all along", section
// "Virtual memory for attention": a prompt's tokens go into blocks acquired
// as the sequence grows, and attention gathers keys and values through the
// sequence's block table.  Prefill attends a chunk of new tokens causally:
// token i of sequence s's n-token chunk sits at position p = ctx - n + i and
// attends positions 0..p.  The chunk's own keys and values are already in
// the pool (written by pa_reshape_and_cache), so earlier chunks and blocks
// shared with other sequences are read the same way.
//
// One workgroup of 8 wavefronts per (KV head g, sequence s, query tile),
// ordered so each XCD runs whole (s, g) pairs (see the kernel's prologue).  A
// wavefront owns 16 MFMA columns: 16/G query tokens x the G query heads of
// KV head g, each column with its own causal limit.  Keys go through LDS in
// 64-key stages of two 32-key product tiles:
//   * a stage's K and V rows are copied from the pool straight into LDS by
//     the buffer unit (buffer_load_dwordx4 ... lds: each lane's 16 bytes land
//     at the lane's own slot of a 1 KB run), without passing through
//     registers.  Two stage buffers alternate, so the next stage's copies
//     are in flight while one is used; each stage costs one workgroup
//     barrier.  Rows are stored unpadded with their 16-byte chunks permuted
//     (XOR of the chunk index with a function of the row), which keeps both
//     LDS read patterns below free of bank conflicts;
//   * S^T = K . Q^T per tile (2 x 4 v_mfma_f32_16x16x32): A = K rows from
//     LDS, B = the wavefront's queries in registers; lane l then holds 8
//     scores of column l%16.  Both tiles' scores are issued first, so the
//     second tile's products run while the first tile's softmax does;
//   * causal and validity masks, online softmax per column (lazy rescale as
//     in the decode kernel; the column max across lane groups by two
//     permlane swaps);
//   * O^T += V^T . P^T: P^T is where the scores left it, V^T comes from
//     the row-major tile through the transposing LDS read; for bf16, P goes
//     in as its top 16 bits plus the top 16 bits of the remainder (two
//     products), so the probabilities keep about 15 bits.
// Each wavefront writes its own columns' outputs: no cross-wavefront merge.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

namespace {

using namespace mfma;

constexpr int kPWaves = 8;                 // wavefronts per workgroup
constexpr int kPTile = 32;                 // keys per product tile
constexpr int kPTPS = 2;                   // product tiles per stage
constexpr int kPStage = kPTile * kPTPS;    // keys per stage
constexpr int kPD = 128;                   // head dim
constexpr int kPRowB = kPD * 2;            // bytes of one K or V row
constexpr int kPHalf = kPStage * kPRowB;   // a stage's K (or V) rows
constexpr int kPRowsW = kPStage / kPWaves; // stage rows each wavefront copies
constexpr int kPRuns = kPRowsW / 4;        // 1 KB runs (4 rows) per matrix per wavefront
// V operands read ahead of their product (more spills registers for bf16)
constexpr int kPVAhead = 1;
constexpr float kPLazy = 8.f;              // lazy-rescale threshold (log2 units)

struct PrefillArgs {
  void* out;
  const void* q;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;
  int32_t S, T, Hq, Hkv, NB, MB;
  int32_t tiles;                           // query tiles per (sequence, KV head)
  int32_t per_xcd;                         // workgroups per XCD
  float qscale;                            // scale * log2(e)
};

// Row r of a stage holds its 16-byte chunk c at position c ^ kswz(r) (K) or
// c ^ vswz(r) (V).  The score product reads 16 rows at one chunk index
// (lanes n = 0..15): positions c ^ n are all distinct.  The transposing read
// takes 32 bytes (chunks 2d, 2d + 1) of rows 4q .. 4q+3 per 16 lanes, rows
// 0..7 per 32: XOR with 2(r & 7) sends the eight rows to eight disjoint
// 32-byte spans.
__device__ __forceinline__ uint32_t kswz(uint32_t r) { return r & 15u; }
__device__ __forceinline__ uint32_t vswz(uint32_t r) { return 2u * (r & 7u); }

// Copy 16 bytes per lane from the buffer resource into LDS: lane l's bytes
// land at lds + 16 l (lds is wavefront-uniform); an offset past the
// resource's end writes zeros.
__device__ __forceinline__ void dma16(rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, static_cast<int>(voff), 0, 0, 0);
}

// Wait until at most N of this wavefront's vector-memory operations are
// outstanding (expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses for the compiler without
// waiting for the copies still landing in other stage buffers (a memory
// fence would wait for every outstanding vector-memory operation).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int DT, int BS, int G>
__global__ __launch_bounds__(kPWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void prefill_kernel(PrefillArgs a) {
  using T = typename KV<DT>::T;
  constexpr float kNegInf = -INFINITY;
  constexpr int TPW = 16 / G;              // query tokens per wavefront
  constexpr int QT = kPWaves * TPW;        // query tokens per workgroup
  static_assert(BS >= 8 && (BS % 8 == 0), "block size");

  // The two stage buffers: one array each, so the compiler can tell a read
  // of one stage from the copies still landing in the other.  K rows first,
  // V rows kPHalf bytes on.
  __shared__ __attribute__((aligned(16))) char sb0[2 * kPHalf];
  __shared__ __attribute__((aligned(16))) char sb1[2 * kPHalf];

  // XCD-aware order.  The hardware hands consecutive workgroups to the 8
  // XCDs in turn, each with its own L2.  Pair p = (sequence, KV head) goes to
  // XCD p % 8, where its query tiles, which re-read the same keys and
  // values, run back to back on one L2; interleaving the pairs keeps the
  // XCDs' shares of the (quadratic) causal work even.
  const int wid = static_cast<int>(blockIdx.x);
  const int k = wid >> 3;                  // k-th workgroup on this XCD
  const int pair = (wid & 7) + 8 * (k / a.tiles);
  if (pair >= a.S * a.Hkv) return;
  const int zt = k % a.tiles;              // 0 = the pair's last (longest) tile
  const int s = pair / a.Hkv;
  const int g = pair - s * a.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 15;                 // column
  const int q4 = lane >> 4;                // lane group

  const int r0 = min(max(a.query_start[s], 0), a.T);
  const int r1 = min(max(a.query_start[s + 1], r0), a.T);
  const int nq = r1 - r0;
  const int ctx = max(0, min(a.context_lens[s], a.MB * BS));
  const int ntiles = (nq + QT - 1) / QT;
  if (zt >= ntiles) return;
  const int qbase = (ntiles - 1 - zt) * QT;   // last tiles first

  // this lane's column: query token qi of the chunk, query head h
  const int qi = qbase + w * TPW + n / G;
  const int h = g * G + n % G;
  const int pos = ctx - nq + qi;           // its position (negative: no keys)
  const bool col_valid = qi < nq && pos >= 0;
  // keys the workgroup needs: up to its last query's position
  const int last = min(qbase + QT, nq) - 1;
  const int kend = min(ctx, ctx - nq + last + 1);
  // the last position this wavefront's columns attend: key tiles past it
  // are masked out for all its columns and are skipped (they would add
  // zero probability and leave the running max alone)
  const int wlast = qbase + w * TPW < nq ? ctx - nq + min(qbase + w * TPW + TPW, nq) - 1 : -1;
  const int wend = __builtin_amdgcn_readfirstlane(wlast);
  // the first position of the wavefront's columns when all of them hold a
  // query (else -1: every tile takes the mask)
  const int wfirst = __builtin_amdgcn_readfirstlane(
      qbase + w * TPW + TPW <= nq ? ctx - nq + qbase + w * TPW : -1);

  // B operand of S^T = K Q^T: lane (n, q4) holds q[column n][32kk + 8q4 .. +8]
  // (loaded without a branch from a row that always exists, nq >= 1 here;
  // columns without a query then take zeros)
  u16x8_t qt[4];
  {
    const T* qb = static_cast<const T*>(a.q) +
                  (static_cast<size_t>(r0 + min(qi, nq - 1)) * a.Hq + h) * kPD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint4 v = *reinterpret_cast<const uint4*>(qb + 32 * kk + 8 * q4);
      qt[kk] = as_u16x8(col_valid ? v : make_uint4(0, 0, 0, 0));
    }
  }
  // The scale enters through the exponent's fma, so the running max is
  // taken over unscaled scores; a negative scale flips the query's signs
  // (exact) and its magnitude is used, which keeps that max the max of the
  // scaled scores.
  const float qs = fabsf(a.qscale);
  if (a.qscale < 0.f) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qt[kk] = __builtin_bit_cast(u16x8_t, __builtin_bit_cast(u32x4_t, qt[kk]) ^ 0x80008000u);
  }

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.MB;
  const size_t bstride = static_cast<size_t>(a.Hkv) * BS * kPD * 2;
  const char* kb = static_cast<const char*>(a.key_cache) + static_cast<size_t>(g) * BS * kPD * 2;
  const char* vb = static_cast<const char*>(a.value_cache) + static_cast<size_t>(g) * BS * kPD * 2;

  // Stage copy: wavefront w carries rows 4w .. 4w+3 of the stage (one 1 KB
  // run of K and one of V); lane l fills slot l of the run, i.e. row
  // 4w + l/16 at chunk position l%16, and so reads the row's chunk
  // (l%16) ^ swz(row).  The four rows sit in one block (bs >= 8, stages start
  // at multiples of 32), so one table entry and one resource per pool serve
  // the wavefront.  Rows past kend load zeros without touching memory.
  const int wv = __builtin_amdgcn_readfirstlane(w);
  const uint32_t lpos = static_cast<uint32_t>(lane & 15);
  auto issue = [&](int t0, char* sb) {
#pragma unroll
    for (int j = 0; j < kPRuns; ++j) {
      // rows 4 (kPRuns wv + j) .. +3 of the stage: one block (bs >= 8)
      const int run = kPRuns * wv + j;
      const uint32_t lrow = static_cast<uint32_t>(4 * run + (lane >> 4));
      const int lb = min(t0 + 4 * run, max(kend - 1, 0)) / BS;   // wave-uniform
      // a scalar load: a vector load here would make the compiler wait for
      // every copy in flight before its value could be used
      const int blk = table_entry(trow, lb);
      const bool bok = static_cast<unsigned>(blk) < static_cast<unsigned>(a.NB);
      const size_t off = bok ? static_cast<size_t>(blk) * bstride : 0;
      const uint32_t bytes = bok ? static_cast<uint32_t>(BS * kPD * 2) : 0u;
      const rsrc_t kres = make_rsrc(kb + off, bytes);
      const rsrc_t vres = make_rsrc(vb + off, bytes);
      // row within its block: t0 is a multiple of the stage, so for bs <=
      // the stage it is the stage row mod bs, else the stage's offset plus
      // that row
      const uint32_t rib =
          BS > kPStage ? (static_cast<uint32_t>(t0) & (BS - 1)) + lrow : lrow & (BS - 1);
      const bool in = t0 + static_cast<int>(lrow) < kend;
      dma16(kres, sb + 1024 * run, in ? rib * kPRowB + 16u * (lpos ^ kswz(lrow)) : kOutOfRange);
      dma16(vres, sb + kPHalf + 1024 * run,
            in ? rib * kPRowB + 16u * (lpos ^ vswz(lrow)) : kOutOfRange);
    }
  };

  // LDS read offsets of this lane.  Scores: row 16u + n at chunk
  // (4kk + q4) ^ n.  Transposing read: row vr = 4 q4 + n/4 (and vr + 16),
  // bytes 32 dt + 8 (n%4) of the row, i.e. chunk 2 dt + (n/2)%2, which sits
  // at chunk position 2 (dt ^ (vr & 7)) + (n/2)%2.
  const uint32_t vr = static_cast<uint32_t>(4 * q4 + (n >> 2));
  const uint32_t vbase = vr * kPRowB + 16u * ((n >> 1) & 1) + 8u * (n & 1);
  auto v_operand = [&](const char* vs, int dt) {
    const char* p0 = vs + vbase + 32u * (static_cast<uint32_t>(dt) ^ (vr & 7u));
    const v4s_t lo = ds_read_tr16(p0);
    const v4s_t hi = ds_read_tr16(p0 + 16 * kPRowB);
    return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T of the 32-key tile whose K rows start at ks: lane (n, q4) gets keys
  // 16u + 4q4 + i of column n
  auto scores = [&](const char* ks, f32x4_t (&sc)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t c = static_cast<uint32_t>(4 * kk + q4) ^ static_cast<uint32_t>(n);
        const uint4 ka = *reinterpret_cast<const uint4*>(ks + (16 * u + n) * kPRowB + 16 * c);
        sc[u] = mma<DT>(as_u16x8(ka), qt[kk], sc[u]);
      }
    }
  };

  // The tile's masked scores (raw) into sv and its column max, scaled.
  // Causal mask; rows of blocks outside the pool were loaded as zeros and
  // count as zero keys and values.  A tile that ends before the wavefront's
  // first position (all its columns valid) needs no mask.
  auto tile_max = [&](int t0, const f32x4_t (&sc)[2], float (&sv)[8], bool masked) {
    float mt = kNegInf;
    if (!masked) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[4 * u + i] = sc[u][i];
          mt = fmaxf(mt, sc[u][i]);
        }
    } else {
      const int lim = col_valid ? pos - t0 : -1;   // rows r <= lim take part
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * u + 4 * q4 + i;
          const float x = r <= lim ? sc[u][i] : kNegInf;
          sv[4 * u + i] = x;
          mt = fmaxf(mt, x);
        }
    }
    // column max over the four lane groups
    return max_lane_groups(mt) * qs;
  };

  // Lazy rescale: the reference max moves only when a tile's max exceeds it
  // by more than kPLazy (log2 units).  Returns the finite reference the
  // tile's probabilities are taken against: while no key has taken part
  // (reference -inf) every score is -inf and exp2(-inf) = 0.
  auto rescale = [&](float mt) {
    const bool bump = mt > m_run + kPLazy;
    const float mn = bump ? mt : m_run;
    if (__any(bump)) {
      const float alpha = bump ? (m_run == kNegInf ? 0.f : fast_exp2(m_run - mn)) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    m_run = mn;
    return mn == kNegInf ? 0.f : mn;
  };

  // P enters the MFMA in the KV type.  f16 keeps 11 significant bits and is
  // rounded to nearest.  bf16 keeps 8, so each probability goes in as two
  // bf16 parts: its top 16 bits (truncation) and the top 16 bits of the
  // exact remainder; both are multiplied in, carrying P to about 15 bits;
  // the sum adds pv itself (the parts differ from it by under 2^-14
  // relative).  Truncation makes each part a bit mask and a byte permute.
  auto probs = [&](const float (&sv)[8], float mref, u16x8_t& pb, u16x8_t& pl) {
    float psum = 0.f;
    if constexpr (DT == PA_BF16) {
      uint32_t hb[8], lb[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float pv = fast_exp2(__builtin_fmaf(sv[jj], qs, -mref));
        const uint32_t b = __builtin_bit_cast(uint32_t, pv);
        const float hf = __builtin_bit_cast(float, b & 0xffff0000u);
        hb[jj] = b;
        lb[jj] = __builtin_bit_cast(uint32_t, pv - hf);   // exact remainder
        psum += pv;   // the two parts carry pv to within 2^-14 of itself
      }
      // upper halves of two words into one: byte selector 0x07060302
      uint32_t ph[4], pq[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        ph[kq] = __builtin_amdgcn_perm(hb[2 * kq + 1], hb[2 * kq], 0x07060302u);
        pq[kq] = __builtin_amdgcn_perm(lb[2 * kq + 1], lb[2 * kq], 0x07060302u);
      }
      pb = __builtin_bit_cast(u16x8_t, ph);
      pl = __builtin_bit_cast(u16x8_t, pq);
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float pv = fast_exp2(__builtin_fmaf(sv[jj], qs, -mref));
        const uint16_t hi = to_bits<DT>(pv);
        pb[jj] = hi;
        psum += from_bits<DT>(hi);
      }
      pl = pb;
    }
    l_run += psum;
  };

  // O^T += V^T P^T.  V^T comes from the V rows through the transposing LDS
  // read (ds_read_b64_tr_b16): within a group of 16 lanes, lane i receives
  // element i%4 of the 8-byte pieces that lanes 4e + i/4 (e = 0..3) point
  // at.  Lane j of group q4 points at key row 4*q4 + j/4, dims
  // 16*dt + 4*(j%4), so lane i receives V[4*q4 + e][16*dt + i]: the A
  // operand's first four entries; the same read 16 rows down gives the
  // other four.
  auto pv_product = [&](const char* vs, const u16x8_t& pb, const u16x8_t& pl) {
    u16x8_t va[8];
#pragma unroll
    for (int dt = 0; dt < kPVAhead; ++dt) va[dt] = v_operand(vs, dt);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (dt + kPVAhead < 8) va[dt + kPVAhead] = v_operand(vs, dt + kPVAhead);
      o[dt] = mma<DT>(va[dt], pb, o[dt]);
      if constexpr (DT == PA_BF16) o[dt] = mma<DT>(va[dt], pl, o[dt]);
    }
  };

  // one tile: softmax and V product after its scores
  auto soft_pv = [&](int t0, const f32x4_t (&sc)[2], const char* vs) {
    float sv[8];
    const float mref = rescale(tile_max(t0, sc, sv, t0 + kPTile - 1 > wfirst));
    u16x8_t pb, pl;
    probs(sv, mref, pb, pl);
    pv_product(vs, pb, pl);
  };

  // the stage at t0 held in sb: the scores of all its tiles first, so the
  // products of one tile overlap the softmax of the one before
  auto compute = [&](int t0, const char* sb) {
    f32x4_t sc[kPTPS][2];
#pragma unroll
    for (int i = 0; i < kPTPS; ++i)
      if (i == 0 || t0 + kPTile * i <= wend) scores(sb + kPTile * i * kPRowB, sc[i]);
#pragma unroll
    for (int i = 0; i < kPTPS; ++i)
      if (i == 0 || t0 + kPTile * i <= wend)
        soft_pv(t0 + kPTile * i, sc[i], sb + kPHalf + kPTile * i * kPRowB);
  };

  // One stage: this wavefront's copies of stage t0 have landed (nothing
  // else is outstanding); after the barrier every wavefront's have, and
  // every wavefront is done with the previous stage, whose buffer takes the
  // copy of the next one.  Stages past the wavefront's last position are
  // not computed (their copies still run, to keep the counts uniform).
  auto step = [&](int t0, const char* cur, char* refill) {
    wait_vm<0>();
    stage_barrier();
    issue(t0 + kPStage, refill);
    if (t0 <= wend) compute(t0, cur);
  };

  // The query loads, older than every copy, have returned once the first
  // stage's copies have.
  issue(0, sb0);
  for (int t0 = 0; t0 < kend; t0 += 2 * kPStage) {
    step(t0, sb0, sb1);
    if (t0 + kPStage >= kend) break;
    step(t0 + kPStage, sb1, sb0);
  }
  // No copy may land in LDS after the workgroup has ended.
  wait_vm<0>();

  // column n's sum over the four lane groups, then this lane's four dims of
  // each 16-dim slice
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qi < nq) {
    const float inv = (col_valid && l_run > 0.f) ? 1.f / l_run : 0.f;
    T* ob = static_cast<T*>(a.out) + (static_cast<size_t>(r0 + qi) * a.Hq + h) * kPD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint2 pk;
      pk.x = static_cast<uint32_t>(to_bits<DT>(o[dt][0] * inv)) |
             (static_cast<uint32_t>(to_bits<DT>(o[dt][1] * inv)) << 16);
      pk.y = static_cast<uint32_t>(to_bits<DT>(o[dt][2] * inv)) |
             (static_cast<uint32_t>(to_bits<DT>(o[dt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(ob + 16 * dt + 4 * q4) = pk;
    }
  }
}

template <int DT, int BS>
int launch_g(const PrefillArgs& a, int G, hipStream_t st) {
  const dim3 grid(static_cast<uint32_t>(8 * a.per_xcd));
  const dim3 block(kPWaves * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<DT, BS, 1>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<DT, BS, 2>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<DT, BS, 4>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<DT, BS, 8>), grid, block, 0, st, a); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return launch_status();
}

template <int DT>
int launch_bs(const PrefillArgs& a, int bs, int G, hipStream_t st) {
  switch (bs) {
    case 8: return launch_g<DT, 8>(a, G, st);
    case 16: return launch_g<DT, 16>(a, G, st);
    case 32: return launch_g<DT, 32>(a, G, st);
    case 64: return launch_g<DT, 64>(a, G, st);
    case 128: return launch_g<DT, 128>(a, G, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace
}  // namespace pa

extern "C" int pa_prefill_attention(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_start,
                                    int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t bs, int32_t NB, int32_t MB, int32_t max_query_len,
                                    float scale, int32_t dtype, void* stream) {
  if (pa::elem_bytes(dtype) == 0) return PA_ERR_INVALID;
  if (S < 0 || T < 0 || Hq < 1 || Hkv < 1 || D < 1 || bs < 1 || NB < 1 || MB < 1)
    return PA_ERR_INVALID;
  if (max_query_len < 0 || Hq % Hkv || !std::isfinite(scale)) return PA_ERR_INVALID;
  if (dtype != PA_BF16 && dtype != PA_F16) return PA_ERR_UNSUPPORTED;
  if (D != 128) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  if (bs != 8 && bs != 16 && bs != 32 && bs != 64 && bs != 128) return PA_ERR_UNSUPPORTED;
  if (S == 0 || T == 0 || max_query_len == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start)
    return PA_ERR_INVALID;
  if (!pa::aligned16(out) || !pa::aligned16(query) || !pa::aligned16(key_cache) ||
      !pa::aligned16(value_cache))
    return PA_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(block_tables) | reinterpret_cast<uintptr_t>(context_lens) |
       reinterpret_cast<uintptr_t>(query_start)) & 3u)
    return PA_ERR_INVALID;
  const int qt = pa::kPWaves * (16 / G);
  const int64_t tiles = (static_cast<int64_t>(max_query_len) + qt - 1) / qt;
  const int64_t units = tiles * S * Hkv;
  if (tiles > 65535 || units > (int64_t(1) << 30)) return PA_ERR_UNSUPPORTED;
  pa::PrefillArgs a{};
  a.out = out;
  a.q = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.S = S;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.NB = NB;
  a.MB = MB;
  a.tiles = static_cast<int32_t>(tiles);
  a.per_xcd = static_cast<int32_t>((static_cast<int64_t>(S) * Hkv + 7) / 8 * tiles);
  a.qscale = scale * pa::kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == PA_BF16 ? pa::launch_bs<PA_BF16>(a, bs, G, st)
                          : pa::launch_bs<PA_F16>(a, bs, G, st);
}
