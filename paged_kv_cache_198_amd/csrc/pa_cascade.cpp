// Host planner for shared-prefix (cascade) decode.
//
// "PagedAttention: the KV cache was the bottleneck all along", section
// "Virtual memory for attention" (parallel sampling and beam search): after a
// fork, sequences point at the same physical blocks for their common prompt.
// Attention over those blocks reads the same bytes once per sequence in a
// plain decode.  The planner finds, in a batch's block tables, groups of
// sequences whose tables start with the same full blocks, and splits each
// sequence's context into
//   * a shared prefix [0, T_sh), attended once per group by the matrix-core
//     kernel with the members' queries as the tile's columns, and
//   * its own suffix [T_sh, ctx), attended per sequence as in a plain decode.
// Both kinds of piece are work items of one launch: a prefix item lists the
// group's members, a suffix item its one sequence.  Each piece leaves a
// partial softmax state (max, sum, unnormalised output) in the workspace; the
// partition reduce combines them, which is exact because softmax over a
// union of disjoint token sets is the weighted merge of the per-set results.
// A sequence that is a single piece writes its output directly.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr int kMembers = 16;                 // member slots per work item
constexpr int kItemInts = 5 + kMembers;      // [table seq, start, end, slot, n, members...]

}  // namespace

extern "C" int pa_cascade_plan(const int32_t* block_tables, const int32_t* context_lens,
                               int32_t S, int32_t MB, int32_t bs, int32_t Hq, int32_t Hkv,
                               int32_t partition_tokens, int32_t prefix_tokens, int32_t* plan,
                               size_t plan_ints, int32_t* info) {
  if (!info) return PA_ERR_INVALID;
  std::memset(info, 0, sizeof(int32_t) * PA_CASCADE_INFO_INTS);
  if (S < 0 || MB < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return PA_ERR_INVALID;
  if (bs != 8 && bs != 16 && bs != 32 && bs != 64 && bs != 128) return PA_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PA_ERR_UNSUPPORTED;
  const int align = std::max(bs, 32);
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % bs)) return PA_ERR_INVALID;
  if (prefix_tokens < 0 || (prefix_tokens > 0 && prefix_tokens % align)) return PA_ERR_INVALID;
  if (S > 0 && (!block_tables || !context_lens)) return PA_ERR_INVALID;

  const int per_item = kMembers / G;         // sequences whose heads fill one tile
  std::vector<int32_t> start(S, 0), base(S, 0), items;
  int64_t prefix_rows = 0, saved_rows = 0;

  // Full blocks strictly before each sequence's last position: the block
  // that holds the newest token is never treated as shared.
  auto full_blocks = [&](int s) -> int {
    const int64_t ctx = std::min<int64_t>(std::max(context_lens[s], 0), int64_t(MB) * bs);
    return ctx > 0 ? static_cast<int>((ctx - 1) / bs) : 0;
  };

  // Groups by first physical block, in order of first appearance.
  std::vector<std::vector<int>> groups;
  std::unordered_map<int32_t, int> by_first;
  for (int s = 0; s < S; ++s) {
    if (full_blocks(s) < 1) continue;
    const int32_t b0 = block_tables[static_cast<size_t>(s) * MB];
    if (b0 < 0) continue;
    auto ins = by_first.emplace(b0, static_cast<int>(groups.size()));
    if (ins.second) groups.emplace_back();
    groups[ins.first->second].push_back(s);
  }

  for (auto& grp : groups) {
    if (grp.size() < 2) continue;
    // Sorted by table row (stable), so sequences that share more blocks end
    // up in the same chunk.
    std::stable_sort(grp.begin(), grp.end(), [&](int x, int y) {
      const int32_t* rx = block_tables + static_cast<size_t>(x) * MB;
      const int32_t* ry = block_tables + static_cast<size_t>(y) * MB;
      const int n = std::min(full_blocks(x), full_blocks(y));
      for (int j = 0; j < n; ++j)
        if (rx[j] != ry[j]) return rx[j] < ry[j];
      return full_blocks(x) > full_blocks(y);
    });
    // Members are taken in tile-sized chunks; each chunk's shared prefix is
    // the run of leading blocks all its members hold, within every member's
    // full blocks, rounded down to the tile alignment.
    for (size_t c0 = 0; c0 < grp.size(); c0 += per_item) {
      const size_t c1 = std::min(grp.size(), c0 + per_item);
      if (c1 - c0 < 2) continue;
      int nb = full_blocks(grp[c0]);
      for (size_t i = c0 + 1; i < c1; ++i) nb = std::min(nb, full_blocks(grp[i]));
      const int32_t* r0 = block_tables + static_cast<size_t>(grp[c0]) * MB;
      int common = 0;
      while (common < nb) {
        bool same = true;
        for (size_t i = c0 + 1; i < c1 && same; ++i)
          same = block_tables[static_cast<size_t>(grp[i]) * MB + common] == r0[common];
        if (!same) break;
        ++common;
      }
      const int T_sh = common * bs / align * align;
      if (T_sh == 0) continue;
      const int piece = prefix_tokens > 0 ? prefix_tokens : T_sh;
      const int k = (T_sh + piece - 1) / piece;
      for (int j = 0; j < k; ++j) {
        const int t0 = j * piece, t1 = std::min(T_sh, t0 + piece);
        const size_t at = items.size();
        items.resize(at + kItemInts, -1);
        items[at + 0] = grp[c0];
        items[at + 1] = t0;
        items[at + 2] = t1;
        items[at + 3] = j;
        items[at + 4] = static_cast<int32_t>(c1 - c0);
        for (size_t i = c0; i < c1; ++i) items[at + 5 + (i - c0)] = grp[i];
        prefix_rows += t1 - t0;
        saved_rows += static_cast<int64_t>(t1 - t0) * static_cast<int64_t>(c1 - c0 - 1);
      }
      for (size_t i = c0; i < c1; ++i) {
        start[grp[i]] = T_sh;
        base[grp[i]] = k;
      }
    }
  }

  // Suffix partitions: one single-member item each, in slots base..; a
  // sequence with one piece in all writes its output directly (slot -1).
  struct Suffix {
    int32_t s, t0, t1, slot;
  };
  std::vector<Suffix> suffix;
  int32_t suffix_parts = 1, slots_max = 1;
  for (int s = 0; s < S; ++s) {
    const int32_t ctx = static_cast<int32_t>(
        std::min<int64_t>(std::max(context_lens[s], 0), int64_t(MB) * bs));
    const int32_t len = ctx - start[s];
    int32_t np = partition_tokens > 0 ? (len + partition_tokens - 1) / partition_tokens
                                      : (len > 0 ? 1 : 0);
    if (base[s] == 0) np = std::max(np, 1);
    suffix_parts = std::max(suffix_parts, np);
    slots_max = std::max(slots_max, base[s] + np);
    const int32_t PT = partition_tokens > 0 ? partition_tokens : std::max(len, 1);
    const bool direct = base[s] + np == 1;
    for (int32_t p = 0; p < np; ++p) {
      const int32_t t0 = start[s] + p * PT;
      suffix.push_back({s, t0, std::min(ctx, t0 + PT), direct ? -1 : base[s] + p});
    }
  }
  for (const Suffix& x : suffix) {
    const size_t at = items.size();
    items.resize(at + kItemInts, -1);
    items[at + 0] = x.s;
    items[at + 1] = x.t0;
    items[at + 2] = x.t1;
    items[at + 3] = x.slot;
    items[at + 4] = 1;
    items[at + 5] = x.s;
  }
  // Longest first: the hardware hands out workgroups roughly in grid order,
  // so long items start first and short ones fill the tail.
  const size_t n_all = items.size() / kItemInts;
  std::vector<size_t> order(n_all);
  for (size_t i = 0; i < n_all; ++i) order[i] = i;
  auto rows = [&](size_t i) { return items[i * kItemInts + 2] - items[i * kItemInts + 1]; };
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return rows(x) > rows(y); });
  std::vector<int32_t> sorted(items.size());
  for (size_t i = 0; i < n_all; ++i)
    std::copy_n(items.begin() + order[i] * kItemInts, kItemInts, sorted.begin() + i * kItemInts);
  items.swap(sorted);
  const int32_t n_items = static_cast<int32_t>(n_all);
  const size_t need = 2 * static_cast<size_t>(S) + items.size();
  info[0] = n_items;
  info[1] = slots_max;
  info[2] = suffix_parts;
  info[3] = static_cast<int32_t>(need);
  info[4] = static_cast<int32_t>(std::min<int64_t>(prefix_rows, INT32_MAX));
  info[5] = static_cast<int32_t>(std::min<int64_t>(saved_rows, INT32_MAX));
  if (!plan || plan_ints < need) return PA_ERR_WORKSPACE;
  std::copy(start.begin(), start.end(), plan);
  std::copy(base.begin(), base.end(), plan + S);
  std::copy(items.begin(), items.end(), plan + 2 * static_cast<size_t>(S));
  return PA_OK;
}
