// Paged decode attention for grouped-query heads on the gfx950 matrix cores.
//
// "PagedAttention: the KV cache was the bottleneck all along", section
// "Virtual memory for attention": keys and values are gathered from scattered
// fixed-size blocks through the sequence's block table.  When G = Hq/Hkv
// query heads share one KV head, the two products of a decode step are dense
// contractions over a tile of T tokens: S = Q_g K^T ([G x D] . [D x T]) and
// O = P V ([G x T] . [T x D]).  This kernel runs both on
// v_mfma_f32_16x16x32_{bf16,f16} (G = 8 padded to the 16-wide tile, D = 128);
// the step stays bound by HBM, the matrix cores only take the arithmetic off
// the vector ALUs.
//
// Per wavefront and 16-token tile (t0 a multiple of 16, so the tile starts on
// a block boundary for bs in {8, 16}, and sits inside one block for larger
// bs):
//   * K and V rows are loaded coalesced (16 lanes x 16 B per 256-byte row)
//     with raw buffer loads, one resource per block; rows past the context
//     load zero without touching memory, so no load sits behind a branch.
//     A tile's K and V rows go to the wavefront's LDS rows as soon as they
//     arrive.  In plain grouped-query decode the next tile's loads then go
//     into the same registers, in flight while the tile is used (one
//     register stage, about 125 VGPRs, four wavefronts per SIMD); work items,
//     often only a few tiles long, keep two register stages (about 150,
//     three wavefronts per SIMD).  Workgroups of two wavefronts keep short
//     ranges from leaving wavefronts idle.
//   * S^T = K . Q^T, one 16-token MFMA tile x 4 k-steps of 32 dims
//     (v_mfma_f32_16x16x32): A = K through the wavefront's LDS tile (lane l:
//     token l%16, dims 8*(l/16) + 32kk .. +8, one 16-byte read), B = Q^T kept
//     in registers (lane l: head l%16, zero for the padding heads).  Lane l
//     then holds the scores of tokens 4(l/16) + i (i = 0..3) for head l%16.
//   * online softmax per head (max across the 4 lane groups of a head with
//     two permlane swaps; the running sum stays per lane and is added up at the
//     end); the reference max moves only when it grows by more than 2^8, so
//     the accumulators are rarely rescaled.
//   * O^T += V^T . P^T on v_mfma_f32_16x16x16 (K = the tile's 16 tokens):
//     B = P^T is already where the scores left it (lane l: head l%16, tokens
//     4(l/16) + i), A = V^T comes from the tile's V rows in LDS (rows padded
//     to 272 bytes) through one transposing LDS read (ds_read_b64_tr_b16)
//     per 16 dims.  The output rows of O^T are dims and
//     its columns heads, so lane l holds head l%16: the per-head rescale
//     factor never leaves the lane.
// Probabilities enter the second product rounded to the KV type; the running
// sum adds the same rounded values, so numerator and denominator agree.
#include <hip/hip_runtime.h>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

namespace {

// Wavefronts per workgroup and register stages: plain grouped-query decode
// runs 2 and 1, work items 2 and 2.  (One wavefront with two stages per
// 512-token partition, 149 VGPRs, fits the long-context grid into the
// resident slots in one round and runs as fast as two with one stage.)
constexpr int kPlainWaves = 2, kPlainStages = 1;
constexpr int kItemWaves = 2, kItemStages = 2;
constexpr int kMTile = 16;                 // tokens per wavefront per tile
constexpr int kMD = 128;                   // head dim
constexpr int kMG = 8;                     // query heads per KV head
constexpr int kVRow = kMD * 2 + 16;        // padded LDS row of one V token (bytes)

using namespace mfma;

constexpr float kLazy = 8.f;               // lazy-rescale threshold (log2 units)

// Registers of one tile in flight: K and V rows (token t0 + 4j + q, 16-byte
// column n), block flags.
constexpr int kMRowGroups = kMTile / 4;    // 4-row load groups per tile
template <int NBK>
struct TileRegs {
  uint4 kr[kMRowGroups];
  uint4 vr[kMRowGroups];
  bool bok[NBK];
};

// GROUP = false: grouped-query decode, the 8 query heads of KV head g of
// sequence s are the tile's columns; grid (Hkv, partitions, S).
// GROUP = true: work items, one per grid row.  A shared-prefix item's
// columns are (member sequence, query head) pairs of sequences whose block
// tables share the item's token range, which is read once for all of them;
// a suffix item has one member, the sequence itself.  Each column writes a
// partial to its member's workspace slot, or, for slot -1, the final output.
template <int DT, int BS, bool GROUP, int kMWaves, int kStages>
__global__ __launch_bounds__(kMWaves * 64) __attribute__((amdgpu_waves_per_eu(kStages == 2 ? 3 : 4)))
void decode_gqa_mfma_kernel(DecodeArgs a) {
  using T = typename KV<DT>::T;
  constexpr float kNegInf = -INFINITY;
  constexpr int NC = GROUP ? 16 : kMG;     // columns that produce output
  // A tile spans 16/bs blocks when bs divides 16 (t0 is then a multiple of
  // bs: partitions are multiples of bs), else it sits inside one block at
  // offset t0 % bs (a multiple of 16).
  constexpr int NBK = BS >= kMTile ? 1 : kMTile / BS;
  static_assert((kMTile % BS == 0 || BS % kMTile == 0) && BS >= 4, "block size");
  using Tile = TileRegs<NBK>;

  // Per-wavefront K/V tiles during the loop; the same bytes hold the
  // cross-wavefront merge afterwards.
  struct Merge {
    float o[kMWaves][NC][kMD];
    float m[kMWaves][NC];
    float l[kMWaves][NC];
  };
  constexpr int kTileBytes = kMWaves * 2 * kMTile * kVRow;   // K and V rows per wavefront
  constexpr int kSmem = kTileBytes > static_cast<int>(sizeof(Merge)) ? kTileBytes : sizeof(Merge);
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  Merge& red = *reinterpret_cast<Merge*>(smem);

  const int g = blockIdx.x;
  const int p = GROUP ? 0 : blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 15;                 // column (scores, output) / token row (K) / d col
  const int q = lane >> 4;                 // lane group

  // Which (sequence, query head) each column n stands for, the token range,
  // and where the results go.
  const int Gh = a.Hq / a.Hkv;            // query heads per KV head
  int s, start, end, ctx;
  PartRange pr{};
  int col_seq = -1, col_head = -1;         // this lane's column
  int slot = 0;
  bool owns_last = false;                  // the item ends at its sequence's last token
  if constexpr (GROUP) {
    const int32_t* it = a.items + static_cast<size_t>(blockIdx.y) * kItemInts;
    s = it[0];
    if (static_cast<unsigned>(s) >= static_cast<unsigned>(a.S)) return;
    ctx = clamp_ctx(a, s, BS);
    // Rounded down to where tiles may start: anywhere on a block boundary
    // when bs <= 32, at a 32-row offset inside a block otherwise.
    constexpr int kAlign = BS < kMTile ? BS : kMTile;
    start = min(max(it[1], 0) / kAlign * kAlign, ctx);
    end = min(max(it[2], start), ctx);
    slot = it[3];
    const int nmem = min(max(it[4], 0), kItemMembers);
    owns_last = nmem == 1 && it[5] == s && end == ctx;
    const int mi = n / Gh;
    if (mi < nmem) {
      const int m = it[5 + mi];
      if (static_cast<unsigned>(m) < static_cast<unsigned>(a.S)) {
        col_seq = m;
        col_head = g * Gh + n % Gh;
      }
    }
  } else {
    s = blockIdx.z;
    ctx = clamp_ctx(a, s, BS);
    pr = part_range(a, s, p, ctx, BS > kMTile ? BS : kMTile);
    if (p >= pr.nparts) return;
    start = pr.start;
    end = pr.end;
    if (n < kMG) {
      col_seq = s;
      col_head = g * kMG + n;
    }
  }
  const int nparts = pr.nparts;

  // B operand of S^T = K Q^T: lane (n, q) holds q[column n][32kk + 8q .. +8].
  u16x8_t qt[4];
  {
    const T* qb = static_cast<const T*>(a.q) +
                  (static_cast<size_t>(max(col_seq, 0)) * a.Hq + max(col_head, 0)) * kMD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (col_seq >= 0) v = *reinterpret_cast<const uint4*>(qb + 32 * kk + 8 * q);
      qt[kk] = as_u16x8(v);
    }
  }

  float m_run = kNegInf;                   // reference max of head n (log2 domain)
  float l_run = 0.f;                       // this lane's share of head n's sum
  f32x4_t o[8];                            // O^T tile dt: dims 16dt + 4q + i, head n
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = a.block_tables + static_cast<size_t>(s) * a.MB;
  const size_t bstride = static_cast<size_t>(a.Hkv) * BS * kMD * 2;
  const char* kb = static_cast<const char*>(a.key_cache) + static_cast<size_t>(g) * BS * kMD * 2;
  const char* vb = static_cast<const char*>(a.value_cache) + static_cast<size_t>(g) * BS * kMD * 2;
  const int last_lb = end > 0 ? (end - 1) / BS : 0;
  const int wv = __builtin_amdgcn_readfirstlane(w);
  char* kt = smem + w * (2 * kMTile * kVRow);   // the tile's K rows
  char* vt = kt + kMTile * kVRow;               // and its V rows

  // Fused step: the last partition owns the new token at position c-1,
  // c = context_lens[s].  Its K/V rows of head g come from the inputs
  // (loaded here with the query; lane (n, q) holds bytes 16n .. 16n+15) and
  // are stored into the slot after the loop; when c is the attended length
  // (not clamped) they also replace that row of the tile in LDS.  A plain
  // decode with a clamped length stores the row without attending it, as a
  // separate cache write would; a work item stores it only when c is not
  // clamped.  Without a new token the loads go through an empty resource and
  // return zeros.
  const int raw_ctx = a.context_lens[s];
  const bool owns_new = a.new_key != nullptr && raw_ctx > 0 &&
                        (GROUP ? owns_last && raw_ctx == ctx : p == nparts - 1);
  const bool append = owns_new && raw_ctx == ctx;
  uint4 nk, nv;
  {
    const size_t src = (static_cast<size_t>(s) * a.Hkv + g) * kMD * 2;
    const uint32_t nbytes = owns_new ? static_cast<uint32_t>(kMD * 2) : 0u;
    nk = buffer_load16(make_rsrc(owns_new ? static_cast<const char*>(a.new_key) + src : kb, nbytes),
                       16u * n);
    nv = buffer_load16(make_rsrc(owns_new ? static_cast<const char*>(a.new_value) + src : vb, nbytes),
                       16u * n);
  }

  // Issue every load of the tile at t0.  Each block's head tile is one buffer
  // resource; a row past the context, or in a block outside the pool, gets
  // an offset past the resource's end and loads zero without touching
  // memory, so no load sits behind a branch.
  auto issue = [&](int t0, Tile& tl) {
    const int boff = BS > kMTile ? t0 % BS : 0;   // tile's row offset in its first block
    int blk[NBK];
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      blk[b] = table_entry(trow, min(t0 / BS + b, last_lb));
      tl.bok[b] = static_cast<unsigned>(blk[b]) < static_cast<unsigned>(a.NB);
    }
    rsrc_t kres[NBK], vres[NBK];
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const size_t off = tl.bok[b] ? static_cast<size_t>(blk[b]) * bstride : 0;
      const uint32_t bytes = tl.bok[b] ? static_cast<uint32_t>(BS * kMD * 2) : 0u;
      kres[b] = make_rsrc(kb + off, bytes);
      vres[b] = make_rsrc(vb + off, bytes);
    }
    // K and V rows, coalesced: 16 lanes x 16 B per 256-byte row, four rows
    // (tokens t0 + 4j + q) per instruction.
#pragma unroll
    for (int j = 0; j < kMRowGroups; ++j) {
      const int rel = 4 * j + q;
      const uint32_t voff =
          t0 + rel < end ? static_cast<uint32_t>(((boff + rel) % BS) * (kMD * 2) + 16 * n)
                         : kOutOfRange;
      tl.kr[j] = buffer_load16(kres[NBK == 1 ? 0 : (boff + 4 * j) / BS], voff);
    }
#pragma unroll
    for (int j = 0; j < kMRowGroups; ++j) {
      const int rel = 4 * j + q;
      const uint32_t voff =
          t0 + rel < end ? static_cast<uint32_t>(((boff + rel) % BS) * (kMD * 2) + 16 * n)
                         : kOutOfRange;
      tl.vr[j] = buffer_load16(vres[NBK == 1 ? 0 : (boff + 4 * j) / BS], voff);
    }
  };

  // The tile's K and V rows go to the wavefront's LDS rows as soon as they
  // arrive (the new token's row, if the tile holds it, over its row), which
  // frees the load registers for the next tile's loads.
  auto stage = [&](int t0, const Tile& tl) {
#pragma unroll
    for (int j = 0; j < kMRowGroups; ++j) {
      *reinterpret_cast<uint4*>(kt + (4 * j + q) * kVRow + 16 * n) = tl.kr[j];
      *reinterpret_cast<uint4*>(vt + (4 * j + q) * kVRow + 16 * n) = tl.vr[j];
    }
    if (append && t0 <= ctx - 1 && ctx - 1 < t0 + kMTile && q == 0) {
      *reinterpret_cast<uint4*>(kt + (ctx - 1 - t0) * kVRow + 16 * n) = nk;
      *reinterpret_cast<uint4*>(vt + (ctx - 1 - t0) * kVRow + 16 * n) = nv;
    }
  };

  // Scores, online softmax and the V product for the staged tile at t0
  // (< end); bok are its blocks' pool flags.
  constexpr int NU = kMTile / 16;          // 16-token score sub-tiles
  auto consume = [&](int t0, const bool (&bok)[NBK]) {
    // A operand: lane (n, q) of sub-tile u takes 16 bytes of token 16u + n
    // at dims 32kk + 8q.
    f32x4_t sc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      sc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 ka =
            *reinterpret_cast<const uint4*>(kt + (16 * u + n) * kVRow + 64 * kk + 16 * q);
        sc[u] = mma<DT>(as_u16x8(ka), qt[kk], sc[u]);
      }
    }
    float sv[4 * NU];
    float mt = kNegInf;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rel = 16 * u + 4 * q + i;
        const bool ok = t0 + rel < end &&
                        pick_ok(bok, (BS > kMTile ? t0 % BS + rel : rel) / BS);
        const float x = ok ? sc[u][i] * a.qscale : kNegInf;
        sv[4 * u + i] = x;
        mt = fmaxf(mt, x);
      }
    mt = max_lane_groups(mt);
    // Lazy rescale: the reference max moves only when the tile's max exceeds
    // it by more than kLazy (log2 units), so weights stay <= 2^kLazy and the
    // accumulators are rarely touched.
    const bool bump = mt > m_run + kLazy;
    const float mn = bump ? mt : m_run;
    if (__any(bump)) {
      const float alpha = bump ? (m_run == kNegInf ? 0.f : fast_exp2(m_run - mn)) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
    m_run = mn;
    uint16_t pbits[4 * NU];
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4 * NU; ++jj) {
      const float pv = (sv[jj] == kNegInf) ? 0.f : fast_exp2(sv[jj] - mn);
      const uint16_t bits = to_bits<DT>(pv);
      pbits[jj] = bits;
      psum += from_bits<DT>(bits);
    }
    l_run += psum;

    // V^T read back transposed from the V rows
    if constexpr (NU == 2) {
      u16x8_t pb;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pb[jj] = pbits[jj];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] = mma<DT>(vt_operand(vt, kVRow, dt, n, q), pb, o[dt]);
    } else {
      // 16 tokens: the 16x16x16 product, B = this lane's 4 probabilities
      u16x4_t pb;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pb[jj] = pbits[jj];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = mma16<DT>(vt_operand16(vt, kVRow, dt, n, q), pb, o[dt]);
    }
  };

  constexpr int kStride = kMWaves * kMTile;
  const int first = start + wv * kMTile;
  // The query and new-row loads, issued before the tiles', are waited for
  // after the first tile loads are issued, so those stay in flight.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  auto wait_query = [&]() {
    asm volatile("" ::"v"(qt[0]), "v"(qt[1]), "v"(qt[2]), "v"(qt[3]),
                 "v"(__builtin_bit_cast(u32x4_t, nk)), "v"(__builtin_bit_cast(u32x4_t, nv)));
  };
  // The loads are issued without conditions (a tile past the end loads zeros
  // without touching memory), so the compiler can count the loads in flight
  // on every path and wait only for the ones each use needs.
  if constexpr (kStages == 1) {
    // One register stage: the next tile's loads go into the registers the
    // current tile has just left for LDS, and are in flight while it is
    // used.  About 125 VGPRs: 4 wavefronts per SIMD.
    Tile ta;
    issue(first, ta);
    wait_query();
    for (int t0 = first; t0 < end; t0 += kStride) {
      stage(t0, ta);
      bool bok[NBK];
#pragma unroll
      for (int b = 0; b < NBK; ++b) bok[b] = ta.bok[b];
      issue(t0 + kStride, ta);
      lds_order();
      consume(t0, bok);
      lds_order();                         // the next tile rewrites these rows
    }
  } else {
    // Two register stages: work items are often a few tiles long, and the
    // tile after next is already in flight when a wavefront starts a tile.
    // About 150 VGPRs: 3 wavefronts per SIMD.
    Tile ta, tb;
    issue(first, ta);
    issue(first + kStride, tb);
    wait_query();
    for (int t0 = first; t0 < end; t0 += 2 * kStride) {
      stage(t0, ta);
      lds_order();
      consume(t0, ta.bok);
      lds_order();
      issue(t0 + 2 * kStride, ta);
      if (t0 + kStride >= end) break;
      stage(t0 + kStride, tb);
      lds_order();
      consume(t0 + kStride, tb.bok);
      lds_order();
      issue(t0 + 3 * kStride, tb);
    }
  }
  // The new token's rows go into its slot after the loop: with no store
  // before them, the block-table reads above stay scalar loads (a store
  // through the pool pointers could alias the table as far as the compiler
  // knows, and a vector load of a table entry would have to wait for every
  // tile load issued before it).  Only this workgroup reads that slot.
  if (owns_new && (!append || (ctx - 1 >= start && ctx - 1 < end)) && wv == 0 && q == 0 &&
      (raw_ctx - 1) / BS < a.MB) {
    const int pos = raw_ctx - 1;
    const int blk = table_entry(trow, pos / BS);
    if (static_cast<unsigned>(blk) < static_cast<unsigned>(a.NB)) {
      const size_t dst = static_cast<size_t>(blk) * bstride +
                         static_cast<size_t>(pos % BS) * (kMD * 2) + 16 * n;
      *reinterpret_cast<uint4*>(const_cast<char*>(kb) + dst) = nk;
      *reinterpret_cast<uint4*>(const_cast<char*>(vb) + dst) = nv;
    }
  }
  lds_barrier();                           // every wavefront is done with its tile

  // column n's sum over the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (n < NC) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red.o[w][n][16 * dt + 4 * q + i] = o[dt][i];
    if (q == 0) {
      red.m[w][n] = m_run;
      red.l[w][n] = l_run;
    }
  }
  lds_barrier();

  for (int i = tid; i < NC * kMD; i += kMWaves * 64) {
    const int gi = i / kMD;
    const int d = i - gi * kMD;
    // the column's sequence and query head (as the lanes of column gi had it)
    int cs, ch;
    if constexpr (GROUP) {
      const int32_t* it = a.items + static_cast<size_t>(blockIdx.y) * kItemInts;
      const int nmem = min(max(it[4], 0), kItemMembers);
      const int mi = gi / Gh;
      cs = mi < nmem ? it[5 + mi] : -1;
      ch = g * Gh + gi % Gh;
      if (static_cast<unsigned>(cs) >= static_cast<unsigned>(a.S)) continue;
    } else {
      cs = s;
      ch = g * kMG + gi;
    }
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < kMWaves; ++v) M = fmaxf(M, red.m[v][gi]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int v = 0; v < kMWaves; ++v) {
      const float mv = red.m[v][gi];
      const float sw = (mv == kNegInf) ? 0.f : fast_exp2(mv - M);
      num = fmaf(red.o[v][gi][d], sw, num);
      den = fmaf(red.l[v][gi], sw, den);
    }
    if (GROUP ? slot < 0 : pr.total == 1) {
      static_cast<T*>(a.out)[(static_cast<size_t>(cs) * a.Hq + ch) * kMD + d] =
          narrow<DT>(den > 0.f ? num / den : 0.f);
    } else {
      const int sl = GROUP ? slot : pr.slot;
      // no workspace exists when pmax < 2
      if (a.pmax < 2 || static_cast<unsigned>(sl) >= static_cast<unsigned>(a.pmax)) continue;
      const size_t idx = (static_cast<size_t>(cs) * a.Hq + ch) * a.pmax + sl;
      a.ws_o[idx * kMD + d] = num;
      if (d == 0) {
        a.ws_m[idx] = M;
        a.ws_l[idx] = den;
      }
    }
  }
}

template <int DT, bool GROUP, int NW = GROUP ? kItemWaves : kPlainWaves,
          int NST = GROUP ? kItemStages : kPlainStages>
int launch_bs(const DecodeArgs& a, int32_t bs, hipStream_t st) {
  // Plain decode: grid (KV head, partition, sequence), so a sequence's
  // partitions are dispatched together (3-4% faster on the long-context
  // batch than partition-major order).  Work items: (KV head, item).
  const dim3 grid(static_cast<uint32_t>(a.Hkv),
                  static_cast<uint32_t>(GROUP ? a.n_items : a.grid_parts),
                  static_cast<uint32_t>(GROUP ? 1 : a.S));
  const dim3 block(NW * 64);
  switch (bs) {
    case 8: hipLaunchKernelGGL((decode_gqa_mfma_kernel<DT, 8, GROUP, NW, NST>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((decode_gqa_mfma_kernel<DT, 16, GROUP, NW, NST>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((decode_gqa_mfma_kernel<DT, 32, GROUP, NW, NST>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((decode_gqa_mfma_kernel<DT, 64, GROUP, NW, NST>), grid, block, 0, st, a); break;
    case 128: hipLaunchKernelGGL((decode_gqa_mfma_kernel<DT, 128, GROUP, NW, NST>), grid, block, 0, st, a); break;
    default: return PA_ERR_UNSUPPORTED;
  }
  return launch_status();
}

}  // namespace

int launch_decode_gqa_mfma(const DecodeArgs& a, int32_t dtype, int32_t bs, hipStream_t st) {
  switch (dtype) {
    case PA_BF16: return launch_bs<PA_BF16, false>(a, bs, st);
    case PA_F16: return launch_bs<PA_F16, false>(a, bs, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

int launch_items_mfma(const DecodeArgs& a, int32_t dtype, int32_t bs, hipStream_t st) {
  if (a.n_items <= 0) return PA_OK;
  switch (dtype) {
    case PA_BF16: return launch_bs<PA_BF16, true>(a, bs, st);
    case PA_F16: return launch_bs<PA_F16, true>(a, bs, st);
    default: return PA_ERR_UNSUPPORTED;
  }
}

}  // namespace pa
