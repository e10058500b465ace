// Token-budget step generator (declared in include/ha_scheduler.h).  Host
// code only.  The rules, as the wangyu.me chunked-prefill page states them in
// its section on the vLLM implementation (token budget, running-first
// scheduling, metadata assembly):
//   * a step carries at most max_num_batched_tokens tokens;
//   * requests already running are served before new ones, in the order they
//     were admitted; waiting requests are admitted in arrival order while
//     budget is left;
//   * a request is granted the tokens it still has to put through the model
//     (its prompt, or the rest of it, or one token while decoding), cut to
//     the long-prefill threshold and to the budget left -- a long prompt thus
//     runs as several chunks.
// Added here: a grant is also cut to the KV pages the pool can still hand out
// (no preemption), and a per-step segment cap.
#include "ha_scheduler.h"

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

namespace {

constexpr int kPageTokens = 16;

struct Request {
  int64_t id;
  int32_t prompt;
  int32_t max_new;
  int32_t generated = 0;  // tokens sampled so far
  int32_t computed = 0;   // tokens already through the model
  std::vector<int32_t> pages;
  int32_t known() const { return prompt + generated; }  // tokens that exist so far
};

struct Planned {
  Request* req;
  int32_t first;  // first position of this step's tokens
  int32_t n;      // tokens this step
};

int32_t pages_for(int64_t tokens) {
  return static_cast<int32_t>((tokens + kPageTokens - 1) / kPageTokens);
}

}  // namespace

struct ha_sched {
  int32_t budget, threshold, max_blocks;
  std::vector<int32_t> free_pages;  // stack; lowest ids handed out first
  std::deque<Request*> waiting;
  std::vector<Request*> running;    // admission order
  std::unordered_set<int64_t> live_ids;
  std::vector<Planned> planned;
  bool step_open = false;

  ~ha_sched() {
    for (Request* r : waiting) delete r;
    for (Request* r : running) delete r;
  }

  // Tokens request r is granted this step (0: none): what it still has to
  // compute -- its known tokens (prompt plus samples) not yet through the
  // model -- cut to the long-prefill threshold, to the budget left and to
  // the room its pages plus the free pages leave.
  int32_t grant(const Request& r, int32_t left) const {
    int64_t n = r.known() - r.computed;
    if (threshold > 0) n = std::min<int64_t>(n, threshold);
    n = std::min<int64_t>(n, left);
    const int64_t room = static_cast<int64_t>(r.pages.size() + free_pages.size()) * kPageTokens - r.computed;
    return static_cast<int32_t>(std::max<int64_t>(std::min(n, room), 0));
  }

  // Plans request r's grant for this step; false when it gets nothing.
  bool take(Request& r, int32_t& left) {
    const int32_t n = grant(r, left);
    if (n <= 0) return false;
    grow(r, r.computed + n);
    planned.push_back({&r, r.computed, n});
    left -= n;
    return true;
  }

  void grow(Request& r, int32_t upto_tokens) {
    const int32_t need = pages_for(upto_tokens);
    while (static_cast<int32_t>(r.pages.size()) < need) {
      r.pages.push_back(free_pages.back());
      free_pages.pop_back();
    }
  }

  void release(Request& r) {
    for (auto it = r.pages.rbegin(); it != r.pages.rend(); ++it) free_pages.push_back(*it);
    r.pages.clear();
  }
};

extern "C" {

ha_sched* ha_sched_create(int32_t max_num_batched_tokens, int32_t long_prefill_token_threshold,
                          int32_t num_blocks, int32_t max_blocks_per_seq) {
  if (max_num_batched_tokens < 1 || long_prefill_token_threshold < 0 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return nullptr;
  ha_sched* s = new (std::nothrow) ha_sched;
  if (!s) return nullptr;
  s->budget = max_num_batched_tokens;
  s->threshold = long_prefill_token_threshold;
  s->max_blocks = max_blocks_per_seq;
  s->free_pages.reserve(num_blocks);
  for (int32_t p = num_blocks - 1; p >= 0; --p) s->free_pages.push_back(p);
  return s;
}

void ha_sched_destroy(ha_sched* s) { delete s; }

ha_status ha_sched_add_request(ha_sched* s, int64_t request_id, int32_t prompt_len,
                               int32_t max_new_tokens) {
  if (!s || s->step_open || prompt_len < 1 || max_new_tokens < 1) return HA_ERR_INVALID_ARGUMENT;
  if (pages_for(static_cast<int64_t>(prompt_len) + max_new_tokens - 1) > s->max_blocks)
    return HA_ERR_INVALID_ARGUMENT;
  if (s->live_ids.count(request_id)) return HA_ERR_INVALID_ARGUMENT;
  Request* r = new (std::nothrow) Request;
  if (!r) return HA_ERR_INVALID_ARGUMENT;
  r->id = request_id;
  r->prompt = prompt_len;
  r->max_new = max_new_tokens;
  s->live_ids.insert(request_id);
  s->waiting.push_back(r);
  return HA_OK;
}

ha_status ha_sched_next_step(ha_sched* s, ha_step_shape* shape, int32_t* cu_seqlens_q,
                             int32_t* seqlens_k, int32_t* block_table, int32_t* slot_mapping,
                             int64_t* request_ids, int32_t* first_pos, int32_t max_seqs,
                             int32_t max_tokens) {
  if (!s || !shape || !cu_seqlens_q || !seqlens_k || !block_table || !slot_mapping ||
      !request_ids || !first_pos || max_seqs < 1 || max_tokens < s->budget || s->step_open)
    return HA_ERR_INVALID_ARGUMENT;
  s->planned.clear();
  int32_t left = s->budget;
  const size_t seg_cap = static_cast<size_t>(max_seqs);
  auto open = [&] { return left > 0 && s->planned.size() < seg_cap; };
  // the running requests, in admission order; one the pool cannot serve now
  // (no page left) skips this step
  for (size_t i = 0; i < s->running.size() && open(); ++i) s->take(*s->running[i], left);
  // then admissions from the waiting queue, in arrival order; when the head of
  // the queue cannot be served the queue waits
  while (open() && !s->waiting.empty() && s->take(*s->waiting.front(), left)) {
    s->running.push_back(s->waiting.front());
    s->waiting.pop_front();
  }
  ha_step_shape sh{};
  if (s->planned.empty()) {
    *shape = sh;
    cu_seqlens_q[0] = 0;
    return (s->waiting.empty() && s->running.empty()) ? HA_OK : HA_ERR_UNSUPPORTED;
  }
  int32_t t = 0;
  cu_seqlens_q[0] = 0;
  for (size_t b = 0; b < s->planned.size(); ++b) {
    const Planned& p = s->planned[b];
    const Request& r = *p.req;
    const int32_t lk = p.first + p.n;
    cu_seqlens_q[b + 1] = t + p.n;
    seqlens_k[b] = lk;
    request_ids[b] = r.id;
    first_pos[b] = p.first;
    int32_t* row = block_table + b * static_cast<size_t>(s->max_blocks);
    for (int32_t j = 0; j < s->max_blocks; ++j)
      row[j] = j < static_cast<int32_t>(r.pages.size()) && j < pages_for(lk) ? r.pages[j] : -1;
    for (int32_t i = 0; i < p.n; ++i) {
      const int32_t pos = p.first + i;
      slot_mapping[t + i] = r.pages[pos / kPageTokens] * kPageTokens + pos % kPageTokens;
    }
    t += p.n;
    sh.max_seqlen_q = std::max(sh.max_seqlen_q, p.n);
    sh.max_seqlen_k = std::max(sh.max_seqlen_k, lk);
    sh.num_decodes += (p.n == 1 && r.computed >= r.prompt) ? 1 : 0;
    sh.num_sampling += (lk == r.known()) ? 1 : 0;
  }
  sh.num_seqs = static_cast<int32_t>(s->planned.size());
  sh.total_q = t;
  *shape = sh;
  s->step_open = true;
  return HA_OK;
}

ha_status ha_sched_complete_step(ha_sched* s, int64_t* finished_ids, int32_t max_finished,
                                 int32_t* num_finished) {
  if (!s || !s->step_open) return HA_ERR_INVALID_ARGUMENT;
  int32_t nf = 0;
  for (const Planned& p : s->planned) {
    Request* r = p.req;
    r->computed += p.n;
    if (r->computed == r->known()) {  // caught up: sample one token
      r->generated += 1;
      if (r->generated >= r->max_new) {
        if (finished_ids && nf < max_finished) finished_ids[nf] = r->id;
        ++nf;
        s->release(*r);
        s->live_ids.erase(r->id);
        s->running.erase(std::find(s->running.begin(), s->running.end(), r));
        delete r;
      }
    }
  }
  s->planned.clear();
  s->step_open = false;
  if (num_finished) *num_finished = nf;
  return HA_OK;
}

int32_t ha_sched_num_unfinished(const ha_sched* s) {
  return s ? static_cast<int32_t>(s->waiting.size() + s->running.size()) : -1;
}

int32_t ha_sched_free_blocks(const ha_sched* s) {
  return s ? static_cast<int32_t>(s->free_pages.size()) : -1;
}

}  // extern "C"
