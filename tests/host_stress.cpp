// Host-side stress of the allocator, the prefix registry and the cascade
// planner through their C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py (CPU only).
// Random operations are checked after every step against invariants that
// hold for any sequence of operations:
//   * every block's reference count equals the number of table entries and
//     registry entries that point at it;
//   * the free stack holds exactly the blocks with no reference, once each;
//   * every planned work item lies inside its sequence's context and the
//     plan's own bounds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pa.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                   \
    }                                                                 \
  } while (0)

static void check_allocator(pa_allocator* a, const std::set<int64_t>& live,
                            const std::map<uint64_t, int32_t>& registry) {
  const int32_t nb = pa_alloc_num_blocks(a);
  std::vector<int32_t> ref(nb), stack(nb);
  int32_t n_free = 0;
  CHECK(pa_alloc_export(a, ref.data(), stack.data(), &n_free) == PA_OK);
  std::vector<int32_t> expect(nb, 0);
  for (int64_t sid : live) {
    const int32_t n = pa_seq_num_blocks(a, sid);
    CHECK(n >= 0);
    std::vector<int32_t> blocks(n > 0 ? n : 1);
    CHECK(pa_seq_blocks(a, sid, blocks.data(), n) == PA_OK);
    const int32_t len = pa_seq_len(a, sid);
    CHECK(len >= 0 && static_cast<int64_t>(n) * pa_alloc_block_size(a) >= len);
    CHECK(static_cast<int64_t>(n - 1) * pa_alloc_block_size(a) < (len > 0 ? len : 1));
    for (int32_t j = 0; j < n; ++j) {
      CHECK(blocks[j] >= 0 && blocks[j] < nb);
      expect[blocks[j]] += 1;
    }
  }
  for (const auto& kv : registry) expect[kv.second] += 1;
  CHECK(n_free == pa_alloc_num_free(a));
  std::vector<int> seen(nb, 0);
  for (int32_t i = 0; i < n_free; ++i) {
    CHECK(stack[i] >= 0 && stack[i] < nb);
    CHECK(seen[stack[i]]++ == 0);
  }
  for (int32_t b = 0; b < nb; ++b) {
    CHECK(ref[b] == expect[b]);
    CHECK((ref[b] == 0) == (seen[b] == 1));
  }
}

static void stress_allocator(uint32_t seed) {
  std::mt19937 rng(seed);
  const int32_t nb = 64 + static_cast<int32_t>(rng() % 128);
  const int32_t bs_choices[] = {1, 8, 16, 32};
  const int32_t bs = bs_choices[rng() % 4];
  pa_allocator* a = pa_alloc_create(nb, bs, nullptr);
  CHECK(a);
  std::set<int64_t> live;
  std::map<uint64_t, int32_t> registry;   // key -> block, mirrored from the calls
  int64_t next = 0;
  for (int step = 0; step < 3000; ++step) {
    const int op = static_cast<int>(rng() % 100);
    if (op < 10 || live.empty()) {
      const int rc = pa_seq_create(a, next);
      CHECK(rc == PA_OK);
      live.insert(next++);
    } else if (op < 55) {
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      const int32_t n = 1 + static_cast<int32_t>(rng() % 40);
      std::vector<int64_t> slots(n);
      int64_t src = -2, dst = -2;
      const int32_t len0 = pa_seq_len(a, *it);
      const int rc = pa_seq_append_n(a, *it, n, slots.data(), &src, &dst);
      CHECK(rc == PA_OK || rc == PA_ERR_OOM);
      if (rc == PA_OK) {
        CHECK((src == -1) == (dst == -1));
        CHECK(src == -1 || (src >= 0 && src < nb && dst >= 0 && dst < nb && src != dst));
        CHECK(pa_seq_len(a, *it) == len0 + n);
        for (int32_t i = 0; i < n; ++i)
          CHECK(slots[i] >= 0 && slots[i] < static_cast<int64_t>(nb) * bs);
      } else {
        CHECK(pa_seq_len(a, *it) == len0);  // all or nothing
      }
    } else if (op < 70) {
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      CHECK(pa_seq_fork(a, *it, next) == PA_OK);
      live.insert(next++);
    } else if (op < 85) {
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      CHECK(pa_seq_free(a, *it) == PA_OK);
      live.erase(it);
    } else if (op < 92) {
      // publish a sequence's full blocks under keys of its own
      auto it = live.begin();
      std::advance(it, rng() % live.size());
      const int32_t full = pa_seq_len(a, *it) / bs;
      const int32_t n = full > 0 ? 1 + static_cast<int32_t>(rng() % full) : 0;
      std::vector<int32_t> blocks(pa_seq_num_blocks(a, *it) + 1);
      CHECK(pa_seq_blocks(a, *it, blocks.data(), pa_seq_num_blocks(a, *it)) == PA_OK);
      std::vector<uint64_t> keys(n > 0 ? n : 1);
      for (int32_t j = 0; j < n; ++j) keys[j] = (static_cast<uint64_t>(*it % 7) << 32) | j;
      int32_t added = -1;
      CHECK(pa_prefix_publish(a, *it, keys.data(), n, &added) == PA_OK);
      int32_t expect_added = 0;
      for (int32_t j = 0; j < n; ++j)
        if (registry.emplace(keys[j], blocks[j]).second) ++expect_added;
      CHECK(added == expect_added);
    } else if (op < 97) {
      // a new request on a registered prefix
      const uint64_t fam = rng() % 7;
      const int32_t n = static_cast<int32_t>(rng() % 6);
      std::vector<uint64_t> keys(n > 0 ? n : 1);
      for (int32_t j = 0; j < n; ++j) keys[j] = (fam << 32) | j;
      int32_t matched = -1;
      CHECK(pa_seq_create_prefixed(a, next, keys.data(), n, &matched) == PA_OK);
      int32_t expect_matched = 0;
      while (expect_matched < n && registry.count(keys[expect_matched])) ++expect_matched;
      CHECK(matched == expect_matched);
      live.insert(next++);
    } else {
      const uint64_t fam = rng() % 7;
      std::vector<uint64_t> keys(8);
      for (int32_t j = 0; j < 8; ++j) keys[j] = (fam << 32) | j;
      int32_t removed = -1;
      CHECK(pa_prefix_evict(a, keys.data(), 8, &removed) == PA_OK);
      int32_t expect_removed = 0;
      for (uint64_t k : keys) expect_removed += static_cast<int32_t>(registry.erase(k));
      CHECK(removed == expect_removed);
    }
    check_allocator(a, live, registry);
    CHECK(pa_prefix_size(a) == static_cast<int32_t>(registry.size()));
  }
  // argument errors leave the state alone
  CHECK(pa_seq_create(a, *live.begin()) == PA_ERR_INVALID);
  CHECK(pa_seq_fork(a, -12345, next) == PA_ERR_INVALID);
  CHECK(pa_seq_free(a, -12345) == PA_ERR_INVALID);
  check_allocator(a, live, registry);
  pa_alloc_destroy(a);
}

static void stress_planner(uint32_t seed) {
  std::mt19937 rng(seed);
  const int32_t bs_choices[] = {8, 16, 32, 64, 128};
  const int32_t g_choices[] = {1, 2, 4, 8};
  for (int round = 0; round < 200; ++round) {
    const int32_t bs = bs_choices[rng() % 5];
    const int32_t G = g_choices[rng() % 4];
    const int32_t Hkv = 1 + static_cast<int32_t>(rng() % 4);
    const int32_t S = static_cast<int32_t>(rng() % 40);
    const int32_t MB = 1 + static_cast<int32_t>(rng() % 12);
    const int32_t nb = 4 * S * MB + 8;
    // tables: a few families sharing leading blocks, the rest random;
    // lengths may exceed MB * bs or be zero or negative
    std::vector<int32_t> tables(static_cast<size_t>(S) * MB, -1), lens(S);
    std::vector<std::vector<int32_t>> fams(3);
    for (auto& f : fams)
      for (int32_t j = 0; j < MB; ++j) f.push_back(static_cast<int32_t>(rng() % nb));
    for (int32_t s = 0; s < S; ++s) {
      lens[s] = static_cast<int32_t>(rng() % (MB * bs + 20)) - 2;
      const int32_t fam = static_cast<int32_t>(rng() % 4);
      const int32_t shared = fam < 3 ? static_cast<int32_t>(rng() % (MB + 1)) : 0;
      for (int32_t j = 0; j < MB; ++j)
        tables[static_cast<size_t>(s) * MB + j] =
            j < shared ? fams[fam][j] : static_cast<int32_t>(rng() % nb) - (rng() % 9 == 0);
    }
    const int32_t align = bs > 32 ? bs : 32;
    const int32_t part = rng() % 3 == 0 ? 0 : bs * (1 + static_cast<int32_t>(rng() % 8));
    const int32_t piece = rng() % 3 == 0 ? align * (1 + static_cast<int32_t>(rng() % 4)) : 0;
    int32_t info[PA_CASCADE_INFO_INTS];
    const int rc0 = pa_cascade_plan(tables.data(), lens.data(), S, MB, bs, G * Hkv, Hkv, part,
                                    piece, nullptr, 0, info);
    CHECK(rc0 == PA_ERR_WORKSPACE);
    const size_t need = static_cast<size_t>(info[3]);
    CHECK(need == 2 * static_cast<size_t>(S) +
                      static_cast<size_t>(info[0]) * PA_CASCADE_ITEM_INTS);
    std::vector<int32_t> plan(need + 1, 0x7eadbeef);
    CHECK(pa_cascade_plan(tables.data(), lens.data(), S, MB, bs, G * Hkv, Hkv, part, piece,
                          plan.data(), need, info) == PA_OK);
    CHECK(plan[need] == 0x7eadbeef);       // nothing written past the plan
    const int32_t n_items = info[0], slots_max = info[1];
    CHECK(n_items >= 0 && slots_max >= 1);
    for (int32_t s = 0; s < S; ++s) {
      CHECK(plan[s] >= 0);                  // own tokens start
      CHECK(plan[S + s] >= 0 && plan[S + s] <= slots_max);
    }
    int32_t prev_rows = 1 << 30;
    for (int32_t i = 0; i < n_items; ++i) {
      const int32_t* it = plan.data() + 2 * S + static_cast<size_t>(i) * PA_CASCADE_ITEM_INTS;
      CHECK(it[0] >= 0 && it[0] < S);
      const int32_t ctx = lens[it[0]] < 0 ? 0 : (lens[it[0]] > MB * bs ? MB * bs : lens[it[0]]);
      CHECK(0 <= it[1] && it[1] <= it[2] && it[2] <= ctx);
      CHECK(it[3] >= -1 && it[3] < slots_max);
      CHECK(it[4] >= 1 && it[4] <= 16 / G);
      for (int32_t m = 0; m < 16; ++m)
        CHECK(m < it[4] ? (it[5 + m] >= 0 && it[5 + m] < S) : it[5 + m] == -1);
      CHECK(it[2] - it[1] <= prev_rows);    // longest first
      prev_rows = it[2] - it[1];
    }
    // a plan buffer one int short is refused and left alone
    if (need > 0) {
      std::vector<int32_t> small(need, 0x5a5a5a5a);
      CHECK(pa_cascade_plan(tables.data(), lens.data(), S, MB, bs, G * Hkv, Hkv, part, piece,
                            small.data(), need - 1, info) == PA_ERR_WORKSPACE);
      for (int32_t v : small) CHECK(v == 0x5a5a5a5a);
    }
  }
}

int main(int argc, char** argv) {
  const uint32_t seeds = argc > 1 ? static_cast<uint32_t>(std::atoi(argv[1])) : 4;
  for (uint32_t seed = 0; seed < seeds; ++seed) {
    stress_allocator(seed);
    stress_planner(seed);
  }
  std::printf("host stress ok\n");
  return 0;
}
