// Step scheduler over the block allocator: one token budget per step,
// running requests first, then the waiting queue; chunked prefill is what
// happens when the budget runs out inside a prompt; preemption by recompute
// when the pool cannot hold a step ("vLLM: what PagedAttention turned into",
// sections "The scheduler, and what it has to balance now" and "Preemption,
// and the path that got deleted"; "(2) vLLM Internals ...", "2. Continuous
// Batching").
//
// It drives the allocator through its C entry points only: a request's
// allocator sequence has the request's id; at admission the prompt's cached
// full blocks are attached (prefix caching, when the allocator has it on)
// after a side-effect-free lookup has shown that the step's blocks fit.
//
// Points the pages leave open, fixed here: the request preempted is the one
// admitted last (the tail of the running list), and if that is the request
// being placed the running walk stops; the long-prefill threshold caps every
// request's share of a step (0: no cap); max_num_seqs bounds the running
// list (0: no bound); a request finishes when it holds max_new_tokens
// generated tokens; at admission at most all tokens but one count as cached,
// so the step that completes a request's tokens always has a position to
// sample from.
#include <algorithm>
#include <deque>
#include <unordered_map>
#include <vector>

#include "host.h"

namespace {

using pkv::fail;

enum : int32_t { kWaiting = 0, kRunning = 1, kFinished = 2 };

struct Request {
  std::vector<int32_t> tokens;  // prompt, then generated tokens
  int32_t prompt_len = 0;
  int32_t max_new = 0;
  uint64_t extra_key = 0;
  int32_t computed = 0;         // tokens whose K/V are in the pool
  int32_t preemptions = 0;
  int32_t state = kWaiting;
  int32_t num_tokens() const { return (int32_t)tokens.size(); }
  int32_t generated() const { return (int32_t)tokens.size() - prompt_len; }
};

struct Item {
  int64_t id;
  int32_t start;
  int32_t n;
  int32_t samples;
};

}  // namespace

struct pkv_scheduler {
  pkv_allocator* alloc = nullptr;
  int32_t capacity = 0;           // blocks a sequence can ever hold (the pool less the null block)
  int32_t budget = 0;
  int32_t threshold = 0;
  bool chunked = true;
  int32_t max_seqs = 0;
  std::unordered_map<int64_t, Request> reqs;
  std::deque<int64_t> waiting;
  std::vector<int64_t> running;
  // the current plan (between schedule and update)
  bool pending = false;
  std::vector<Item> items;
  std::vector<int64_t> slots;
  std::vector<int64_t> preempted;
  std::vector<int64_t> finished;  // by the last update

  int32_t share(const Request& r, int32_t left) const {
    int32_t n = std::min(r.num_tokens() - r.computed, left);
    if (threshold > 0) n = std::min(n, threshold);
    return n;
  }

  int preempt(int64_t id) {
    Request& r = reqs.at(id);
    if (int e = pkv_seq_free(alloc, id)) return e;
    r.computed = 0;
    r.preemptions += 1;
    r.state = kWaiting;
    waiting.push_front(id);
    return PKV_OK;
  }

  // Appends n positions to request id's sequence, writing their slots at the
  // end of `slots`. PKV_ERR_OUT_OF_BLOCKS leaves everything unchanged.
  int place(int64_t id, int32_t n) {
    const size_t at = slots.size();
    slots.resize(at + n);
    int64_t pairs[2];
    int32_t npairs = 0;
    const int e = pkv_seq_append(alloc, id, n, slots.data() + at, pairs, 1, &npairs);
    if (e != PKV_OK) {
      slots.resize(at);
      return e;
    }
    // The scheduler's sequences never share a partially filled block (only
    // full cached blocks are attached, nothing is forked), so no append copies.
    if (npairs != 0) return fail(PKV_ERR_INVALID_ARG, "request %lld: unexpected copy-on-write",
                                 (long long)id);
    return PKV_OK;
  }

  int schedule() {
    items.clear();
    slots.clear();
    preempted.clear();
    int32_t left = budget;
    size_t i = 0;
    while (i < running.size() && left > 0) {
      const int64_t id = running[i];
      Request& r = reqs.at(id);
      const int32_t n = share(r, left);
      bool placed = false;
      for (;;) {
        const int e = place(id, n);
        if (e == PKV_OK) {
          placed = true;
          break;
        }
        if (e != PKV_ERR_OUT_OF_BLOCKS) return e;
        const int64_t victim = running.back();
        running.pop_back();
        if (int e2 = preempt(victim)) return e2;
        preempted.push_back(victim);
        if (victim == id) break;
      }
      if (!placed) break;
      items.push_back({id, r.computed, n, r.computed + n == r.num_tokens() ? 1 : 0});
      left -= n;
      ++i;
    }
    if (!preempted.empty()) return PKV_OK;  // an over-committed step admits no one
    while (!waiting.empty() && left > 0 &&
           (max_seqs <= 0 || (int32_t)running.size() < max_seqs)) {
      const int64_t id = waiting.front();
      Request& r = reqs.at(id);
      const int32_t limit = r.num_tokens() - 1;
      int32_t cached = 0, revived = 0;
      if (int e = pkv_prefix_lookup(alloc, r.tokens.data(), r.num_tokens(), r.extra_key, limit,
                                    &cached, &revived))
        return e;
      const int32_t need = r.num_tokens() - cached;
      int32_t n = std::min(need, left);
      if (threshold > 0) n = std::min(n, threshold);
      if (!chunked && n < need) break;  // the prompt waits for a step with room for all of it
      const int32_t new_blocks =
          (cached + n + pkv::kBlock - 1) / pkv::kBlock - cached / pkv::kBlock;
      int32_t free_blocks = 0;
      if (int e = pkv_num_free_blocks(alloc, &free_blocks)) return e;
      if (revived + new_blocks > free_blocks) break;
      int32_t got = 0;
      if (int e = pkv_seq_add_cached(alloc, id, r.tokens.data(), r.num_tokens(), r.extra_key, limit,
                                     &got))
        return e;
      if (got != cached) return fail(PKV_ERR_INVALID_ARG, "prefix lookup and attach disagree");
      if (int e = place(id, n)) return e;  // fits: checked above
      r.computed = cached;
      r.state = kRunning;
      waiting.pop_front();
      running.push_back(id);
      items.push_back({id, cached, n, cached + n == r.num_tokens() ? 1 : 0});
      left -= n;
    }
    return PKV_OK;
  }
};

namespace {

int check(pkv_scheduler* s) {
  return s ? PKV_OK : fail(PKV_ERR_INVALID_ARG, "scheduler handle is NULL");
}

}  // namespace

extern "C" {

int pkv_scheduler_create(pkv_allocator* alloc, int32_t token_budget, int32_t long_prefill_threshold,
                         int32_t chunked_prefill, int32_t max_num_seqs, pkv_scheduler** out) {
  pkv::clear_error();
  if (!alloc || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  if (token_budget < 1 || long_prefill_threshold < 0 || max_num_seqs < 0)
    return fail(PKV_ERR_INVALID_ARG, "token_budget must be >= 1, threshold and max_num_seqs >= 0");
  pkv_stats st;
  if (int e = pkv_allocator_stats(alloc, &st)) return e;
  pkv_scheduler* s = new pkv_scheduler();
  s->alloc = alloc;
  s->capacity = st.used_blocks + st.free_blocks;
  s->budget = token_budget;
  s->threshold = long_prefill_threshold;
  s->chunked = chunked_prefill != 0;
  s->max_seqs = max_num_seqs;
  *out = s;
  return PKV_OK;
}

int pkv_scheduler_destroy(pkv_scheduler* s) {
  pkv::clear_error();
  delete s;
  return PKV_OK;
}

int pkv_scheduler_add_request(pkv_scheduler* s, int64_t req_id, const int32_t* prompt,
                              int32_t prompt_len, int32_t max_new_tokens, uint64_t extra_key) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (!prompt || prompt_len < 1 || max_new_tokens < 1)
    return fail(PKV_ERR_INVALID_ARG, "empty prompt or nothing to generate");
  if ((int64_t)prompt_len + max_new_tokens > INT32_MAX / 2)
    return fail(PKV_ERR_INVALID_ARG, "request too long");
  if (s->reqs.count(req_id)) return fail(PKV_ERR_SEQ_EXISTS, "request %lld exists", (long long)req_id);
  // At its end a request holds the K/V of all its tokens but the last
  // sampled one; one that needs more blocks than the pool has could never
  // finish (and would hold up the queue behind it).
  const int32_t need = (prompt_len + max_new_tokens - 1 + pkv::kBlock - 1) / pkv::kBlock;
  if (need > s->capacity)
    return fail(PKV_ERR_OUT_OF_BLOCKS, "request %lld needs %d blocks, the pool holds %d",
                (long long)req_id, need, s->capacity);
  Request r;
  r.tokens.assign(prompt, prompt + prompt_len);
  r.prompt_len = prompt_len;
  r.max_new = max_new_tokens;
  r.extra_key = extra_key;
  s->reqs.emplace(req_id, std::move(r));
  s->waiting.push_back(req_id);
  return PKV_OK;
}

int pkv_scheduler_schedule(pkv_scheduler* s, int32_t* out_num_scheduled, int64_t* out_num_tokens,
                           int32_t* out_num_preempted) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (s->pending) return fail(PKV_ERR_INVALID_ARG, "the previous plan has not been updated");
  if (int e = s->schedule()) return e;
  pkv::clear_error();  // a preemption's out-of-blocks message is not an error of this call
  s->pending = true;
  if (out_num_scheduled) *out_num_scheduled = (int32_t)s->items.size();
  if (out_num_tokens) *out_num_tokens = (int64_t)s->slots.size();
  if (out_num_preempted) *out_num_preempted = (int32_t)s->preempted.size();
  return PKV_OK;
}

int pkv_scheduler_plan(pkv_scheduler* s, int64_t* req_ids, int32_t* start_pos, int32_t* num_new,
                       int32_t* samples, int64_t* slots, int64_t* preempted) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (!s->pending) return fail(PKV_ERR_INVALID_ARG, "no plan: call pkv_scheduler_schedule first");
  for (size_t i = 0; i < s->items.size(); ++i) {
    if (req_ids) req_ids[i] = s->items[i].id;
    if (start_pos) start_pos[i] = s->items[i].start;
    if (num_new) num_new[i] = s->items[i].n;
    if (samples) samples[i] = s->items[i].samples;
  }
  if (slots) std::copy(s->slots.begin(), s->slots.end(), slots);
  if (preempted) std::copy(s->preempted.begin(), s->preempted.end(), preempted);
  return PKV_OK;
}

int pkv_scheduler_update(pkv_scheduler* s, const int32_t* sampled, int32_t n_sampled,
                         int32_t* out_num_finished) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (!s->pending) return fail(PKV_ERR_INVALID_ARG, "no plan to update");
  int32_t want = 0;
  for (const Item& it : s->items) want += it.samples;
  if (n_sampled != want || (want > 0 && !sampled))
    return fail(PKV_ERR_INVALID_ARG, "expected %d sampled tokens, got %d", want, n_sampled);
  // Record the step's token ids first (cannot fail for a consistent plan),
  // then advance.
  for (const Item& it : s->items) {
    const Request& r = s->reqs.at(it.id);
    if (int e = pkv_seq_record_tokens(s->alloc, it.id, r.tokens.data() + it.start, it.n)) return e;
  }
  s->finished.clear();
  int32_t k = 0;
  for (const Item& it : s->items) {
    Request& r = s->reqs.at(it.id);
    r.computed = it.start + it.n;
    if (it.samples) {
      r.tokens.push_back(sampled[k++]);
      if (r.generated() >= r.max_new) s->finished.push_back(it.id);
    }
  }
  for (int64_t id : s->finished) {
    if (int e = pkv_seq_free(s->alloc, id)) return e;
    s->running.erase(std::find(s->running.begin(), s->running.end(), id));
    s->reqs.at(id).state = kFinished;
  }
  s->pending = false;
  if (out_num_finished) *out_num_finished = (int32_t)s->finished.size();
  return PKV_OK;
}

int pkv_scheduler_remove_request(pkv_scheduler* s, int64_t req_id) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (s->pending) return fail(PKV_ERR_INVALID_ARG, "a plan is pending: update it first");
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no request %lld", (long long)req_id);
  if (it->second.state == kRunning) {
    if (int e = pkv_seq_free(s->alloc, req_id)) return e;
    s->running.erase(std::find(s->running.begin(), s->running.end(), req_id));
  } else if (it->second.state == kWaiting) {
    s->waiting.erase(std::find(s->waiting.begin(), s->waiting.end(), req_id));
  }
  s->reqs.erase(it);
  return PKV_OK;
}

int pkv_scheduler_finished(pkv_scheduler* s, int64_t* req_ids) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (!req_ids && !s->finished.empty()) return fail(PKV_ERR_INVALID_ARG, "req_ids is NULL");
  std::copy(s->finished.begin(), s->finished.end(), req_ids);
  return PKV_OK;
}

int pkv_scheduler_counts(pkv_scheduler* s, int32_t* num_waiting, int32_t* num_running) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  if (num_waiting) *num_waiting = (int32_t)s->waiting.size();
  if (num_running) *num_running = (int32_t)s->running.size();
  return PKV_OK;
}

int pkv_scheduler_request(pkv_scheduler* s, int64_t req_id, int32_t* state, int32_t* num_tokens,
                          int32_t* computed, int32_t* preemptions, int32_t* tokens,
                          int32_t max_tokens) {
  pkv::clear_error();
  if (int e = check(s)) return e;
  auto it = s->reqs.find(req_id);
  if (it == s->reqs.end()) return fail(PKV_ERR_NO_SUCH_SEQ, "no request %lld", (long long)req_id);
  const Request& r = it->second;
  if (state) *state = r.state;
  if (num_tokens) *num_tokens = r.num_tokens();
  if (computed) *computed = r.computed;
  if (preemptions) *preemptions = r.preemptions;
  if (tokens) {
    if (max_tokens < r.num_tokens())
      return fail(PKV_ERR_INVALID_ARG, "tokens holds %d, request has %d", max_tokens, r.num_tokens());
    std::copy(r.tokens.begin(), r.tokens.end(), tokens);
  }
  return PKV_OK;
}

}  // extern "C"
