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
// KV head g, each column with its own causal limit.  Per 32-token key tile:
//   * all 512 lanes load 64 keys' K and V rows once (16 bytes each, raw
//     buffer loads that return zero past a block or the range) into LDS,
//     where the eight wavefronts share them as two 32-key tiles; the next
//     64 keys' loads are issued before the current ones are used;
//   * S^T = K . Q^T (2 x 4 v_mfma_f32_16x16x32): A = K rows from LDS, B = the
//     wavefront's queries in registers; lane l then holds 8 scores of
//     column l%16;
//   * causal and validity masks, online softmax per column (lazy rescale as
//     in the decode kernel);
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
constexpr int kPStage = 64;                // keys staged in LDS per barrier pair
constexpr int kPRowsW = kPStage / kPWaves; // staged rows each wavefront loads
constexpr int kPD = 128;                   // head dim
// Padded LDS rows.  K rows (68 dwords) let the 16 lanes of an operand read
// (rows n = 0..15, 16 bytes each) hit 16 distinct bank groups; V rows (72
// dwords) let the transposing read's four rows of 8 dwords per 16-lane
// group fall on disjoint banks.  No single stride does both.
constexpr int kPRow = kPD * 2 + 16;        // K
constexpr int kPRowV = kPD * 2 + 32;       // V
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

template <int DT, int BS, int G>
__global__ __launch_bounds__(kPWaves * 64) void prefill_kernel(PrefillArgs a) {
  using T = typename KV<DT>::T;
  constexpr float kNegInf = -INFINITY;
  constexpr int TPW = 16 / G;              // query tokens per wavefront
  constexpr int QT = kPWaves * TPW;        // query tokens per workgroup
  static_assert(BS >= 8 && (BS % 8 == 0), "block size");

  __shared__ __attribute__((aligned(16))) char ks[kPStage * kPRow];
  __shared__ __attribute__((aligned(16))) char vs[kPStage * kPRowV];

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

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.MB;
  const size_t bstride = static_cast<size_t>(a.Hkv) * BS * kPD * 2;
  const char* kb = static_cast<const char*>(a.key_cache) + static_cast<size_t>(g) * BS * kPD * 2;
  const char* vb = static_cast<const char*>(a.value_cache) + static_cast<size_t>(g) * BS * kPD * 2;

  // Cooperative stage load: wavefront w carries staged rows 8w .. 8w+7 (lane
  // l: rows 8w + l/16 and 8w + 4 + l/16, 16-byte column l%16).  The eight
  // rows sit in one block (bs >= 8, stages start at multiples of 64), so one
  // table entry and one buffer resource per pool serve the wavefront.  The
  // next stage's loads are issued as soon as the current one is in LDS.
  const int wv = __builtin_amdgcn_readfirstlane(w);
  constexpr int NJ = kPRowsW / 4;          // 16-lane row groups per wavefront
  const int lrow = kPRowsW * wv + (lane >> 4);
  const int lcol = lane & 15;
  struct Stage {
    uint4 kr[NJ], vr[NJ];
  };
  auto issue = [&](int t0, Stage& st) {
    const int lb = min(t0 + kPRowsW * wv, max(kend - 1, 0)) / BS;   // wave-uniform
    const int blk = table_entry(trow, lb);
    const bool bok = static_cast<unsigned>(blk) < static_cast<unsigned>(a.NB);
    const size_t off = bok ? static_cast<size_t>(blk) * bstride : 0;
    const uint32_t bytes = bok ? static_cast<uint32_t>(BS * kPD * 2) : 0u;
    const rsrc_t kres = make_rsrc(kb + off, bytes);
    const rsrc_t vres = make_rsrc(vb + off, bytes);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // row within its block: t0 is a multiple of 64, so for bs <= 64 it is
      // the lane's staged row mod bs, else the stage's offset plus that row
      const uint32_t r = static_cast<uint32_t>(lrow + 4 * j);
      const uint32_t rib = BS > kPStage ? (static_cast<uint32_t>(t0) & (BS - 1)) + r : r & (BS - 1);
      const uint32_t in = rib * (kPD * 2) + 16u * static_cast<uint32_t>(lcol);
      const uint32_t voff = t0 + static_cast<int>(r) < kend ? in : kOutOfRange;
      st.kr[j] = buffer_load16(kres, voff);
      st.vr[j] = buffer_load16(vres, voff);
    }
  };

  // products of the 32-key tile at t0, staged at LDS row rb
  auto compute = [&](int t0, int rb) {
      // scores: lane (n, q4) gets keys t0 + 16u + 4q4 + i of column n
      f32x4_t sc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint4 ka =
              *reinterpret_cast<const uint4*>(ks + (rb + 16 * u + n) * kPRow + 64 * kk + 16 * q4);
          sc[u] = mma<DT>(as_u16x8(ka), qt[kk], sc[u]);
        }
      }
      // Causal mask; rows of blocks outside the pool were loaded as zeros
      // and count as zero keys and values.  A tile that ends before the
      // wavefront's first position (all its columns valid) needs no mask.
      float sv[8];
      float mt = kNegInf;
      if (t0 + kPTile - 1 <= wfirst) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sc[u][i] * a.qscale;
            sv[4 * u + i] = x;
            mt = fmaxf(mt, x);
          }
      } else {
        const int lim = col_valid ? pos - t0 : -1;   // rows r <= lim take part
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * u + 4 * q4 + i;
            const float x = r <= lim ? sc[u][i] * a.qscale : kNegInf;
            sv[4 * u + i] = x;
            mt = fmaxf(mt, x);
          }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const bool bump = mt > m_run + kPLazy;
      const float mn = bump ? mt : m_run;
      if (__any(bump)) {
        const float alpha = bump ? (m_run == kNegInf ? 0.f : fast_exp2(m_run - mn)) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      }
      m_run = mn;
      // P enters the MFMA in the KV type.  f16 keeps 11 significant bits
      // and is rounded to nearest.  bf16 keeps 8, so each probability goes
      // in as two bf16 parts: its top 16 bits (truncation) and the top 16
      // bits of the exact remainder; both are multiplied in, carrying P to
      // about 15 bits; the sum adds pv itself (the parts differ from it by
      // under 2^-14 relative).  Truncation makes each part a bit mask and a
      // byte permute.
      // a finite reference: while no key has taken part (mn = -inf) every
      // score is -inf and exp2(-inf - 0) = 0
      const float mref = mn == kNegInf ? 0.f : mn;
      u16x8_t pb, pl;
      float psum = 0.f;
      if constexpr (DT == PA_BF16) {
        uint32_t hb[8], lb[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float pv = fast_exp2(sv[jj] - mref);        // exp2(-inf) = 0
          const uint32_t b = __builtin_bit_cast(uint32_t, pv);
          const float hf = __builtin_bit_cast(float, b & 0xffff0000u);
          hb[jj] = b;
          lb[jj] = __builtin_bit_cast(uint32_t, pv - hf);   // exact remainder
          psum += pv;   // the two parts carry pv to within 2^-14 of itself
        }
        // upper halves of two words into one: byte selector 0x07060302
        uint32_t ph[4], pq[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          ph[k] = __builtin_amdgcn_perm(hb[2 * k + 1], hb[2 * k], 0x07060302u);
          pq[k] = __builtin_amdgcn_perm(lb[2 * k + 1], lb[2 * k], 0x07060302u);
        }
        pb = __builtin_bit_cast(u16x8_t, ph);
        pl = __builtin_bit_cast(u16x8_t, pq);
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float pv = fast_exp2(sv[jj] - mref);
          const uint16_t hi = to_bits<DT>(pv);
          pb[jj] = hi;
          psum += from_bits<DT>(hi);
        }
      }
      l_run += psum;

      // O^T += V^T P^T.  V^T comes from the row-major V tile through the
      // transposing LDS read (ds_read_b64_tr_b16): within a group of 16
      // lanes, lane i receives element i%4 of the 8-byte chunks that lanes
      // 4e + i/4 (e = 0..3) point at.  Lane j of group q4 points at key row
      // 4*q4 + j/4, dims 16*dt + 4*(j%4), so lane i receives
      // V[4*q4 + e][16*dt + i]: the A operand's first four entries; the same
      // read 16 rows down gives the other four.
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u16x8_t va = vt_operand(vs + rb * kPRowV, kPRowV, dt, n, q4);
        o[dt] = mma<DT>(va, pb, o[dt]);
        if constexpr (DT == PA_BF16) o[dt] = mma<DT>(va, pl, o[dt]);
      }
  };

  // one stage: publish the 64 staged keys in LDS, refill the registers with
  // the next 64 (past kend: zero loads, no traffic), then the two 32-key
  // product tiles (skipped past the wavefront's last position)
  Stage st;
  auto step = [&](int t0) {
    __syncthreads();                       // every wavefront is done with the last stage
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = lrow + 4 * j;
      *reinterpret_cast<uint4*>(ks + r * kPRow + 16 * lcol) = st.kr[j];
      *reinterpret_cast<uint4*>(vs + r * kPRowV + 16 * lcol) = st.vr[j];
    }
    __syncthreads();
    issue(t0 + kPStage, st);
    if (t0 <= wend) compute(t0, 0);
    if (t0 + kPTile <= wend) compute(t0 + kPTile, kPTile);
  };

  // The query loads (older than the stage's) are waited for before the loop,
  // where the stage's loads stay in flight.
  issue(0, st);
  asm volatile("" ::"v"(qt[0]), "v"(qt[1]), "v"(qt[2]), "v"(qt[3]));
  for (int t0 = 0; t0 < kend; t0 += kPStage) step(t0);

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
