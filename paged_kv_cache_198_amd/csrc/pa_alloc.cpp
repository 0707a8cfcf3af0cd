// Host block allocator for the paged KV cache.
//
// "PagedAttention: the KV cache was the bottleneck all along", section
// "Virtual memory for attention": fixed-size blocks acquired as a sequence
// grows, a block table per sequence, sharing between completions of one
// prompt with a copy only on divergence, beams forked and discarded.  The
// tie-break rules (LIFO free stack, lazy copy-on-write, release order, OOM
// leaving the state unchanged) are stated in include/pa.h.
//
// Sharing across requests ("From the abstract": sharing within and across
// requests; "What is left": common system prompts shared across users): a
// prefix registry maps caller keys to full blocks and holds one reference
// to each, so a later request whose prompt starts the same way takes those
// blocks instead of writing its own.
//
// Plain C++17 with no HIP dependency: it runs on the scheduler's host thread.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;  // logical -> physical
  int64_t len = 0;              // tokens stored
};

}  // namespace

struct pa_allocator {
  int32_t nb = 0;
  int32_t bs = 1;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  std::unordered_map<uint64_t, int32_t> prefix;  // key -> full block (one reference each)

  int32_t pop() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

extern "C" {

pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t bs, const int32_t* init_order) {
  if (num_blocks < 0 || bs < 1) return nullptr;
  auto* a = new pa_allocator;
  a->nb = num_blocks;
  a->bs = bs;
  a->ref.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (init_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = init_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return nullptr;
      }
      seen[b] = 1;
    }
  }
  // init_order[0] must end on top of the stack.
  for (int32_t i = 0; i < num_blocks; ++i)
    a->free_stack[num_blocks - 1 - i] = init_order ? init_order[i] : i;
  return a;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_num_free(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->free_stack.size()) : -1;
}
int32_t pa_alloc_num_blocks(const pa_allocator* a) { return a ? a->nb : -1; }
int32_t pa_alloc_block_size(const pa_allocator* a) { return a ? a->bs : -1; }

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->nb) return -1;
  return a->ref[block];
}

int pa_seq_create(pa_allocator* a, int64_t seq_id) {
  if (!a || a->find(seq_id)) return PA_ERR_INVALID;
  a->seqs.emplace(seq_id, Seq{});
  return PA_OK;
}

int pa_seq_append_n(pa_allocator* a, int64_t seq_id, int32_t n, int64_t* slots,
                    int64_t* cow_src, int64_t* cow_dst) {
  if (!a || n < 0 || (n > 0 && !slots)) return PA_ERR_INVALID;
  Seq* s = a->find(seq_id);
  if (!s) return PA_ERR_INVALID;
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  if (n == 0) return PA_OK;
  const int64_t bs = a->bs;
  const int64_t off0 = s->len % bs;
  const bool cow = off0 != 0 && a->ref[s->blocks.back()] > 1;
  // Blocks this call takes: one per block boundary crossed, plus the copy.
  const int64_t have = (s->len + bs - 1) / bs;
  const int64_t want = (s->len + n + bs - 1) / bs;
  const int64_t need = (want - have) + (cow ? 1 : 0);
  if (need > static_cast<int64_t>(a->free_stack.size())) return PA_ERR_OOM;
  if (cow) {
    int32_t old = s->blocks.back();
    int32_t fresh = a->pop();
    a->ref[old] -= 1;
    s->blocks.back() = fresh;
    if (cow_src) *cow_src = old;
    if (cow_dst) *cow_dst = fresh;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t off = s->len % bs;
    if (off == 0) s->blocks.push_back(a->pop());
    slots[i] = static_cast<int64_t>(s->blocks.back()) * bs + off;
    s->len += 1;
  }
  return PA_OK;
}

int pa_seq_append(pa_allocator* a, int64_t seq_id, int64_t* slot, int64_t* cow_src,
                  int64_t* cow_dst) {
  if (!slot) return PA_ERR_INVALID;
  return pa_seq_append_n(a, seq_id, 1, slot, cow_src, cow_dst);
}

int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
  if (!a || parent == child) return PA_ERR_INVALID;
  const Seq* p = a->find(parent);
  if (!p || a->find(child)) return PA_ERR_INVALID;
  Seq c = *p;
  for (int32_t b : c.blocks) a->ref[b] += 1;
  a->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_seq_free(pa_allocator* a, int64_t seq_id) {
  if (!a) return PA_ERR_INVALID;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PA_ERR_INVALID;
  const std::vector<int32_t>& bl = it->second.blocks;
  for (auto r = bl.rbegin(); r != bl.rend(); ++r) {
    if (--a->ref[*r] == 0) a->free_stack.push_back(*r);
  }
  a->seqs.erase(it);
  return PA_OK;
}

int32_t pa_seq_len(const pa_allocator* a, int64_t seq_id) {
  const Seq* s = a ? a->find(seq_id) : nullptr;
  return s ? static_cast<int32_t>(s->len) : -1;
}

int32_t pa_seq_num_blocks(const pa_allocator* a, int64_t seq_id) {
  const Seq* s = a ? a->find(seq_id) : nullptr;
  return s ? static_cast<int32_t>(s->blocks.size()) : -1;
}

int pa_seq_blocks(const pa_allocator* a, int64_t seq_id, int32_t* blocks, int32_t cap) {
  const Seq* s = a ? a->find(seq_id) : nullptr;
  if (!s || (!blocks && !s->blocks.empty())) return PA_ERR_INVALID;
  if (static_cast<int64_t>(s->blocks.size()) > cap) return PA_ERR_INVALID;
  if (!s->blocks.empty())
    std::memcpy(blocks, s->blocks.data(), s->blocks.size() * sizeof(int32_t));
  return PA_OK;
}

int pa_build_batch(const pa_allocator* a, const int64_t* seq_ids, int32_t S, int32_t MB,
                   int32_t* block_tables, int32_t* context_lens) {
  if (!a || S < 0 || MB < 0) return PA_ERR_INVALID;
  if (S > 0 && (!seq_ids || !context_lens || (MB > 0 && !block_tables))) return PA_ERR_INVALID;
  for (int32_t i = 0; i < S; ++i) {
    const Seq* s = a->find(seq_ids[i]);
    if (!s || static_cast<int64_t>(s->blocks.size()) > MB) return PA_ERR_INVALID;
  }
  for (int32_t i = 0; i < S; ++i) {
    const Seq* s = a->find(seq_ids[i]);
    int32_t* row = block_tables + static_cast<int64_t>(i) * MB;
    const int32_t nbk = static_cast<int32_t>(s->blocks.size());
    for (int32_t j = 0; j < MB; ++j) row[j] = j < nbk ? s->blocks[j] : -1;
    context_lens[i] = static_cast<int32_t>(s->len);
  }
  return PA_OK;
}

int pa_prefix_publish(pa_allocator* a, int64_t seq_id, const uint64_t* keys, int32_t n,
                      int32_t* added) {
  if (added) *added = 0;
  if (!a || n < 0 || (n > 0 && !keys)) return PA_ERR_INVALID;
  const Seq* s = a->find(seq_id);
  if (!s || static_cast<int64_t>(n) * a->bs > s->len) return PA_ERR_INVALID;
  int32_t count = 0;
  for (int32_t j = 0; j < n; ++j) {
    // a key that is already present keeps its block (first publisher wins)
    if (a->prefix.emplace(keys[j], s->blocks[j]).second) {
      a->ref[s->blocks[j]] += 1;
      ++count;
    }
  }
  if (added) *added = count;
  return PA_OK;
}

int pa_seq_create_prefixed(pa_allocator* a, int64_t seq_id, const uint64_t* keys, int32_t n,
                           int32_t* matched) {
  if (matched) *matched = 0;
  if (!a || n < 0 || (n > 0 && !keys) || a->find(seq_id)) return PA_ERR_INVALID;
  Seq s;
  for (int32_t j = 0; j < n; ++j) {
    auto it = a->prefix.find(keys[j]);
    if (it == a->prefix.end()) break;      // the run of hits ends at the first miss
    s.blocks.push_back(it->second);
  }
  for (int32_t b : s.blocks) a->ref[b] += 1;
  s.len = static_cast<int64_t>(s.blocks.size()) * a->bs;
  if (matched) *matched = static_cast<int32_t>(s.blocks.size());
  a->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_prefix_evict(pa_allocator* a, const uint64_t* keys, int32_t n, int32_t* removed) {
  if (removed) *removed = 0;
  if (!a || n < 0 || (n > 0 && !keys)) return PA_ERR_INVALID;
  int32_t count = 0;
  for (int32_t j = n - 1; j >= 0; --j) {  // last to first, as a table is released
    auto it = a->prefix.find(keys[j]);
    if (it == a->prefix.end()) continue;
    const int32_t b = it->second;
    a->prefix.erase(it);
    if (--a->ref[b] == 0) a->free_stack.push_back(b);
    ++count;
  }
  if (removed) *removed = count;
  return PA_OK;
}

int32_t pa_prefix_size(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->prefix.size()) : -1;
}

int pa_alloc_export(const pa_allocator* a, int32_t* refcounts, int32_t* free_stack,
                    int32_t* n_free) {
  if (!a) return PA_ERR_INVALID;
  if (refcounts && a->nb) std::memcpy(refcounts, a->ref.data(), a->ref.size() * sizeof(int32_t));
  if (free_stack) {
    const size_t n = a->free_stack.size();
    for (size_t i = 0; i < n; ++i) free_stack[i] = a->free_stack[n - 1 - i];
  }
  if (n_free) *n_free = static_cast<int32_t>(a->free_stack.size());
  return PA_OK;
}

}  // extern "C"
