// Host-side block manager of libpagedattn: which physical pool blocks every sequence owns,
// with reference-counted sharing, copy on write and a prefix tree of full blocks.  The rules
// are stated with the declarations in include/pagedattn.h.
//
// Pages: Colossal-Inference release post, "分块式KV缓存 (BlockedKeyValueCache)" (blocks taken
// from the pool as tokens arrive); LLM inference optimisation overview, 2.1.2 "Paged Attention"
// (reserved pool, logical -> physical table, several logical blocks on one physical block,
// reference counts, freed at zero); Taco-LLM article, "使用 Prefix Cache 技术降低 TTFT" (earlier
// prompts' cache kept as a prefix tree, the matching part of a new prompt read from it).
#include <cstdint>
#include <map>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa_status.hpp"
#include "pagedattn.h"

struct pa_block_manager {
  struct Block {
    int32_t ref = 0;
    bool registered = false;
    int32_t parent = -1;          // registered parent block, -1 for a first block
    int32_t depth = 0;            // index of the block in the sequence that registered it
    int32_t children = 0;         // registered blocks whose parent this is
    int64_t released = 0;         // logical time at which the count last dropped to zero
    std::vector<int32_t> tokens;  // the token ids of a registered block
  };
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t num_tokens = 0;
    bool tracked = false;        // token ids were given
    bool chain = true;           // every full block so far is registered (the next may be)
    std::vector<int32_t> tail;   // token ids in the partly filled last block
  };
  using Key = std::pair<int32_t, std::vector<int32_t>>;

  int32_t num_blocks = 0, block_size = 0;
  std::vector<Block> blocks;
  std::set<int32_t> free_set;                                 // unregistered, count 0
  std::set<std::tuple<int64_t, int32_t, int32_t>> evictable;  // (released, -depth, id): registered leaves, count 0
  std::map<Key, int32_t> tree;                                // prefix tree of full blocks
  std::unordered_map<int64_t, Seq> seqs;
  int64_t clock = 0;
  int32_t registered = 0;       // registered blocks
  int32_t registered_idle = 0;  // registered blocks with count 0 (evictable now or once their children go)

  int32_t available() const { return static_cast<int32_t>(free_set.size()) + registered_idle; }

  int32_t evict() {
    const auto it = evictable.begin();
    const int32_t id = std::get<2>(*it);
    evictable.erase(it);
    Block& b = blocks[id];
    tree.erase(Key(b.parent, b.tokens));
    if (b.parent >= 0) {
      Block& p = blocks[b.parent];
      if (--p.children == 0 && p.ref == 0) evictable.emplace(p.released, -p.depth, b.parent);
    }
    b.registered = false;
    b.parent = -1;
    b.tokens.clear();
    --registered;
    --registered_idle;
    return id;
  }

  int32_t take() {  // the caller has checked available() > 0
    int32_t id;
    if (!free_set.empty()) {
      id = *free_set.begin();
      free_set.erase(free_set.begin());
    } else {
      id = evict();
    }
    blocks[id].ref = 1;
    return id;
  }

  void hold(int32_t id) {  // one more reference to a registered block found in the tree
    Block& b = blocks[id];
    if (b.ref == 0) {
      --registered_idle;
      if (b.children == 0) evictable.erase(std::make_tuple(b.released, -b.depth, id));
    }
    ++b.ref;
  }

  // Block `index` of `s` has just been filled with `tokens`: register it if the chain allows.
  void filled(Seq& s, size_t index, const std::vector<int32_t>& tokens) {
    if (!s.tracked || !s.chain) return;
    const int32_t parent = index == 0 ? -1 : s.blocks[index - 1];
    Key key(parent, tokens);
    if (tree.count(key)) {  // the same content is registered already: this block stays private
      s.chain = false;
      return;
    }
    const int32_t id = s.blocks[index];
    Block& b = blocks[id];
    b.registered = true;
    b.parent = parent;
    b.depth = static_cast<int32_t>(index);
    b.tokens = tokens;
    if (parent >= 0) ++blocks[parent].children;
    tree.emplace(std::move(key), id);
    ++registered;
  }

  // Add n tokens (ids may be null) at the end of s; the blocks they need are available.
  void extend(Seq& s, const int32_t* ids, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
      if (s.num_tokens % block_size == 0) s.blocks.push_back(take());
      if (s.tracked) s.tail.push_back(ids[i]);
      ++s.num_tokens;
      if (s.num_tokens % block_size == 0) {
        filled(s, s.blocks.size() - 1, s.tail);
        s.tail.clear();
      }
    }
  }

  void release(int32_t id) {
    Block& b = blocks[id];
    if (--b.ref > 0) return;
    b.released = clock;
    if (b.registered) {
      ++registered_idle;
      if (b.children == 0) evictable.emplace(b.released, -b.depth, id);
    } else {
      free_set.insert(id);
    }
  }
};

using pa::fail;
using pa::ok;

extern "C" {

pa_status_t pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** manager) {
  const char* fn = "pa_bm_create";
  if (manager == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  *manager = nullptr;
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_blocks %d <= 0", fn, num_blocks);
  if (block_size <= 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: block_size %d <= 0", fn, block_size);
  auto* m = new (std::nothrow) pa_block_manager;
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: out of host memory", fn);
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->blocks.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) m->free_set.insert(m->free_set.end(), i);
  *manager = m;
  return ok();
}

void pa_bm_destroy(pa_block_manager* manager) { delete manager; }

pa_status_t pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                               int32_t* cached_tokens) {
  const char* fn = "pa_bm_add_sequence";
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens %d < 0", fn, num_tokens);
  if (m->seqs.count(seq_id)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: sequence %lld exists", fn, (long long)seq_id);
  const int32_t B = m->block_size;
  // the longest registered chain matching the prompt, leaving at least one token to compute
  std::vector<int32_t> matched;
  if (token_ids != nullptr && num_tokens > 0) {
    int32_t parent = -1;
    const int32_t max_match = (num_tokens - 1) / B;
    for (int32_t i = 0; i < max_match; ++i) {
      const auto it = m->tree.find(pa_block_manager::Key(
          parent, std::vector<int32_t>(token_ids + static_cast<size_t>(i) * B, token_ids + static_cast<size_t>(i + 1) * B)));
      if (it == m->tree.end()) break;
      matched.push_back(it->second);
      parent = it->second;
    }
  }
  const int64_t total_blocks = (static_cast<int64_t>(num_tokens) + B - 1) / B;
  const int64_t needed = total_blocks - static_cast<int64_t>(matched.size());
  int64_t held_idle = 0;  // matched blocks that would stop being evictable
  for (int32_t id : matched) held_idle += m->blocks[id].ref == 0;
  if (needed > m->available() - held_idle)
    return fail(PA_ERR_OUT_OF_BLOCKS, "%s: %lld blocks needed, %lld available", fn, (long long)needed,
                (long long)(m->available() - held_idle));
  pa_block_manager::Seq s;
  s.tracked = token_ids != nullptr;
  for (int32_t id : matched) {
    m->hold(id);
    s.blocks.push_back(id);
  }
  s.num_tokens = static_cast<int64_t>(matched.size()) * B;
  const int64_t first = s.num_tokens;
  m->extend(s, token_ids != nullptr ? token_ids + first : nullptr, num_tokens - first);
  m->seqs.emplace(seq_id, std::move(s));
  if (cached_tokens != nullptr) *cached_tokens = static_cast<int32_t>(first);
  return ok();
}

pa_status_t pa_bm_append(pa_block_manager* m, int64_t seq_id, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* copies, int32_t max_copies, int32_t* num_copies) {
  const char* fn = "pa_bm_append";
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARGUMENT, "%s: num_tokens %d < 0", fn, num_tokens);
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return fail(PA_ERR_INVALID_ARGUMENT, "%s: no sequence %lld", fn, (long long)seq_id);
  pa_block_manager::Seq& s = it->second;
  if (s.tracked != (token_ids != nullptr) && num_tokens > 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: token ids must be given exactly for sequences added with them", fn);
  if (num_copies != nullptr) *num_copies = 0;
  if (num_tokens == 0) return ok();
  const int32_t B = m->block_size;
  const bool partial = s.num_tokens % B != 0;
  const bool cow = partial && m->blocks[s.blocks.back()].ref > 1;
  if (cow && (copies == nullptr || max_copies < 1 || num_copies == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: the last block is shared and no room for the copy was given", fn);
  const int64_t total_blocks = (s.num_tokens + num_tokens + B - 1) / B;
  const int64_t needed = total_blocks - static_cast<int64_t>(s.blocks.size()) + (cow ? 1 : 0);
  if (needed > m->available())
    return fail(PA_ERR_OUT_OF_BLOCKS, "%s: %lld blocks needed, %d available", fn, (long long)needed, m->available());
  if (cow) {
    const int32_t old = s.blocks.back();
    const int32_t fresh = m->take();
    --m->blocks[old].ref;  // still held by the other sequences sharing it
    s.blocks.back() = fresh;
    copies[0] = old;
    copies[1] = fresh;
    *num_copies = 1;
  }
  m->extend(s, token_ids, num_tokens);
  return ok();
}

pa_status_t pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id) {
  const char* fn = "pa_bm_fork";
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  const auto it = m->seqs.find(parent_id);
  if (it == m->seqs.end()) return fail(PA_ERR_INVALID_ARGUMENT, "%s: no sequence %lld", fn, (long long)parent_id);
  if (m->seqs.count(child_id)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: sequence %lld exists", fn, (long long)child_id);
  pa_block_manager::Seq child = it->second;
  for (int32_t id : child.blocks) ++m->blocks[id].ref;
  m->seqs.emplace(child_id, std::move(child));
  return ok();
}

pa_status_t pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
  const char* fn = "pa_bm_free_sequence";
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return fail(PA_ERR_INVALID_ARGUMENT, "%s: no sequence %lld", fn, (long long)seq_id);
  ++m->clock;
  for (int32_t id : it->second.blocks) m->release(id);
  m->seqs.erase(it);
  return ok();
}

pa_status_t pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* table, int32_t max_blocks,
                              int32_t* num_blocks, int32_t* num_tokens) {
  const char* fn = "pa_bm_block_table";
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: manager is null", fn);
  const auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return fail(PA_ERR_INVALID_ARGUMENT, "%s: no sequence %lld", fn, (long long)seq_id);
  const auto& s = it->second;
  const int64_t nb = static_cast<int64_t>(s.blocks.size());
  if (nb > max_blocks || (nb > 0 && table == nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: %lld blocks do not fit in %d", fn, (long long)nb, max_blocks);
  for (int64_t i = 0; i < nb; ++i) table[i] = s.blocks[i];
  if (num_blocks != nullptr) *num_blocks = static_cast<int32_t>(nb);
  if (num_tokens != nullptr) *num_tokens = static_cast<int32_t>(s.num_tokens);
  return ok();
}

pa_status_t pa_bm_stats(const pa_block_manager* m, int32_t* free_blocks, int32_t* registered_blocks,
                        int32_t* used_blocks) {
  if (m == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "pa_bm_stats: manager is null");
  int32_t used = 0;
  for (const auto& b : m->blocks) used += b.ref > 0;
  if (free_blocks != nullptr) *free_blocks = static_cast<int32_t>(m->free_set.size());
  if (registered_blocks != nullptr) *registered_blocks = m->registered;
  if (used_blocks != nullptr) *used_blocks = used;
  return ok();
}

}  // extern "C"

namespace pa {
int32_t bm_block_size(const pa_block_manager* m) { return m->block_size; }
int32_t bm_num_blocks(const pa_block_manager* m) { return m->num_blocks; }
}  // namespace pa
