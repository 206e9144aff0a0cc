// Host step scheduler for continuous batching: Running / Waiting queues, the prefill-ratio
// trigger and block-budget admission over a block manager.  The rules are stated with the
// declarations in include/pagedattn.h ("Step scheduler"); this file follows them in order.
//
// Colossal-Inference release post, "连续批量化算法 (Continuous Batching)": prefill and decode
// run as separate steps over unpadded input, a prefill step when the inputs needing prefill
// reach a ratio.  LLM inference optimisation overview, 2.4 "服务": step-level scheduling with
// a Running and a Waiting queue (a finished sequence leaves, a waiting one enters) and dynamic
// batching by the memory left; 2.1.2 "Paged Attention": block-granular accounting of what
// still fits, and a bound on the tokens of one batch.
#include <algorithm>
#include <cmath>
#include <deque>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa_status.hpp"

using pa::fail;
using pa::ok;

struct pa_scheduler {
  struct Request {
    std::vector<int32_t> tokens;  // prompt, then every token produced so far
    int32_t max_new = 0;
    int32_t generated = 0;
    int32_t cached = 0;  // tokens reused from the prefix tree at the last admission
  };
  pa_sched_config cfg{};
  pa_block_manager* bm = nullptr;
  int32_t block_size = 0;
  int32_t num_blocks = 0;
  std::unordered_map<int64_t, Request> requests;  // every waiting or running request
  std::deque<int64_t> waiting;                    // FIFO; preempted requests go to the head
  std::vector<int64_t> running;                   // admission order
  std::vector<int64_t> pending;                   // the last step's sequences, until commit
  int64_t finished = 0;
  int64_t preemptions = 0;
};

namespace {

// Block table row of `id` into `row` (max_blocks entries, -1 past its blocks).
pa_status_t table_row(pa_scheduler* s, int64_t id, int32_t* row) {
  int32_t nb = 0, nt = 0;
  const pa_status_t st = pa_bm_block_table(s->bm, id, row, s->cfg.max_blocks_per_seq, &nb, &nt);
  if (st != PA_OK) return st;
  std::fill(row + nb, row + s->cfg.max_blocks_per_seq, -1);
  return PA_OK;
}

void clear_batch(pa_sched_batch* b) {
  b->kind = PA_STEP_IDLE;
  b->num_seqs = b->total_q = b->max_q_len = b->max_context_len = 0;
  b->num_copies = b->num_preempted = 0;
  b->cu_seqlens_q[0] = 0;
}

// Release the most recently admitted running sequence and put its request back at the head of
// Waiting, with every token it knows (prompt and produced), to be prefilled again.
int64_t preempt_last(pa_scheduler* s, pa_sched_batch* b) {
  const int64_t victim = s->running.back();
  s->running.pop_back();
  pa_bm_free_sequence(s->bm, victim);
  s->waiting.push_front(victim);
  b->preempted[b->num_preempted++] = victim;
  ++s->preemptions;
  return victim;
}

}  // namespace

extern "C" {

pa_status_t pa_sched_create(const pa_sched_config* config, pa_block_manager* manager, pa_scheduler** scheduler) {
  const char* fn = "pa_sched_create";
  if (config == nullptr || manager == nullptr || scheduler == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  const pa_sched_config& c = *config;
  if (c.max_running <= 0 || c.max_batch_tokens <= 0 || c.max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_running, max_batch_tokens and max_blocks_per_seq must be > 0", fn);
  if (!(c.prefill_ratio > 0.f) || !std::isfinite(c.prefill_ratio))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: prefill_ratio must be finite and > 0", fn);
  auto* s = new pa_scheduler;
  s->cfg = c;
  s->bm = manager;
  s->block_size = pa::bm_block_size(manager);
  s->num_blocks = pa::bm_num_blocks(manager);
  *scheduler = s;
  return ok();
}

void pa_sched_destroy(pa_scheduler* scheduler) { delete scheduler; }

pa_status_t pa_sched_add_request(pa_scheduler* s, int64_t request_id, const int32_t* prompt, int32_t prompt_len,
                                 int32_t max_new_tokens) {
  const char* fn = "pa_sched_add_request";
  if (s == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: scheduler is null", fn);
  if (prompt == nullptr || prompt_len < 1) return fail(PA_ERR_INVALID_ARGUMENT, "%s: empty prompt", fn);
  if (max_new_tokens < 1) return fail(PA_ERR_INVALID_ARGUMENT, "%s: max_new_tokens %d < 1", fn, max_new_tokens);
  if (s->requests.count(request_id)) return fail(PA_ERR_INVALID_ARGUMENT, "%s: request %lld in use", fn, (long long)request_id);
  const int64_t most = static_cast<int64_t>(prompt_len) + max_new_tokens - 1;
  const int64_t blocks = (most + s->block_size - 1) / s->block_size;
  if (most > s->cfg.max_batch_tokens)
    return fail(PA_ERR_UNSUPPORTED, "%s: %lld tokens exceed max_batch_tokens %d", fn, (long long)most,
                s->cfg.max_batch_tokens);
  if (blocks > s->cfg.max_blocks_per_seq || blocks > s->num_blocks)
    return fail(PA_ERR_UNSUPPORTED, "%s: %lld blocks exceed the table width or the pool", fn, (long long)blocks);
  pa_scheduler::Request r;
  r.tokens.assign(prompt, prompt + prompt_len);
  r.max_new = max_new_tokens;
  s->requests.emplace(request_id, std::move(r));
  s->waiting.push_back(request_id);
  return ok();
}

pa_status_t pa_sched_step(pa_scheduler* s, pa_sched_batch* b) {
  const char* fn = "pa_sched_step";
  if (s == nullptr || b == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: null pointer", fn);
  if (!s->pending.empty()) return fail(PA_ERR_INVALID_ARGUMENT, "%s: the previous step is not committed", fn);
  if (!b->seq_ids || !b->cu_seqlens_q || !b->context_lens || !b->block_tables || !b->input_tokens || !b->copies ||
      !b->preempted)
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: null batch array", fn);
  clear_batch(b);
  const pa_sched_config& c = s->cfg;
  const size_t cap = static_cast<size_t>(c.max_running);

  // ---- prefill step: admit from the head of Waiting --------------------------------------
  const bool room = s->running.size() < cap;
  const bool ratio = s->running.empty() ||
                     static_cast<double>(s->waiting.size()) >= static_cast<double>(c.prefill_ratio) * s->running.size();
  if (!s->waiting.empty() && room && ratio) {
    int64_t known = 0;
    while (!s->waiting.empty() && s->running.size() < cap) {
      const int64_t id = s->waiting.front();
      pa_scheduler::Request& r = s->requests.at(id);
      const int64_t n = static_cast<int64_t>(r.tokens.size());
      if (b->num_seqs > 0 && known + n > c.max_batch_tokens) break;
      int32_t cached = 0;
      const pa_status_t st = pa_bm_add_sequence(s->bm, id, r.tokens.data(), static_cast<int32_t>(n), &cached);
      if (st == PA_ERR_OUT_OF_BLOCKS) break;
      if (st != PA_OK) return st;
      s->waiting.pop_front();
      s->running.push_back(id);
      r.cached = cached;
      known += n;
      const int32_t rows = static_cast<int32_t>(n) - cached;
      const int32_t i = b->num_seqs++;
      b->seq_ids[i] = id;
      b->context_lens[i] = static_cast<int32_t>(n);
      std::copy(r.tokens.begin() + cached, r.tokens.end(), b->input_tokens + b->total_q);
      b->total_q += rows;
      b->cu_seqlens_q[i + 1] = b->total_q;
      b->max_q_len = std::max(b->max_q_len, rows);
      b->max_context_len = std::max(b->max_context_len, static_cast<int32_t>(n));
      const pa_status_t tt = table_row(s, id, b->block_tables + static_cast<size_t>(i) * c.max_blocks_per_seq);
      if (tt != PA_OK) return tt;
      s->pending.push_back(id);
    }
    if (b->num_seqs > 0) {
      b->kind = PA_STEP_PREFILL;
      return ok();
    }
  }

  // ---- decode step: every running sequence appends its newest token ----------------------
  size_t i = 0;
  while (i < s->running.size()) {
    const int64_t id = s->running[i];
    pa_scheduler::Request& r = s->requests.at(id);
    const int32_t tok = r.tokens.back();
    int32_t pair[2], ncopies = 0;
    const pa_status_t st = pa_bm_append(s->bm, id, &tok, 1, pair, 1, &ncopies);
    if (st == PA_ERR_OUT_OF_BLOCKS) {
      preempt_last(s, b);  // the sequence itself when it is the most recent: the loop then ends
      continue;
    }
    if (st != PA_OK) return st;
    if (ncopies > 0) {
      b->copies[2 * b->num_copies] = pair[0];
      b->copies[2 * b->num_copies + 1] = pair[1];
      ++b->num_copies;
    }
    ++i;
  }
  for (size_t k = 0; k < s->running.size(); ++k) {
    const int64_t id = s->running[k];
    const pa_scheduler::Request& r = s->requests.at(id);
    const int32_t n = static_cast<int32_t>(r.tokens.size());
    b->seq_ids[k] = id;
    b->context_lens[k] = n;
    b->input_tokens[k] = r.tokens.back();
    b->cu_seqlens_q[k + 1] = static_cast<int32_t>(k + 1);
    b->max_context_len = std::max(b->max_context_len, n);
    const pa_status_t tt = table_row(s, id, b->block_tables + k * c.max_blocks_per_seq);
    if (tt != PA_OK) return tt;
    s->pending.push_back(id);
  }
  b->num_seqs = static_cast<int32_t>(s->running.size());
  b->total_q = b->num_seqs;
  b->max_q_len = b->num_seqs > 0 ? 1 : 0;
  b->kind = b->num_seqs > 0 ? PA_STEP_DECODE : PA_STEP_IDLE;
  return ok();
}

pa_status_t pa_sched_commit(pa_scheduler* s, const int32_t* next_tokens, const uint8_t* finished, int32_t num_seqs) {
  const char* fn = "pa_sched_commit";
  if (s == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: scheduler is null", fn);
  if (num_seqs != static_cast<int32_t>(s->pending.size()))
    return fail(PA_ERR_INVALID_ARGUMENT, "%s: %d results for a step of %zu sequences", fn, num_seqs, s->pending.size());
  if (num_seqs == 0) return ok();
  if (next_tokens == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "%s: next_tokens is null", fn);
  std::unordered_set<int64_t> done;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t id = s->pending[i];
    pa_scheduler::Request& r = s->requests.at(id);
    r.tokens.push_back(next_tokens[i]);
    ++r.generated;
    if ((finished != nullptr && finished[i]) || r.generated >= r.max_new) {
      pa_bm_free_sequence(s->bm, id);
      s->requests.erase(id);
      done.insert(id);
      ++s->finished;
    }
  }
  if (!done.empty())
    s->running.erase(std::remove_if(s->running.begin(), s->running.end(), [&](int64_t id) { return done.count(id) > 0; }),
                     s->running.end());
  s->pending.clear();
  return ok();
}

pa_status_t pa_sched_stats(const pa_scheduler* s, int32_t* waiting, int32_t* running, int64_t* finished,
                           int64_t* preemptions) {
  if (s == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "pa_sched_stats: scheduler is null");
  if (waiting != nullptr) *waiting = static_cast<int32_t>(s->waiting.size());
  if (running != nullptr) *running = static_cast<int32_t>(s->running.size());
  if (finished != nullptr) *finished = s->finished;
  if (preemptions != nullptr) *preemptions = s->preemptions;
  return ok();
}

}  // extern "C"
