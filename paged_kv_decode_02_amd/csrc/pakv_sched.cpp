// pakv_sched.cpp - host page allocator and request admission for the shared
// K/V page pool (C ABI in include/pakv_sched.h, which states the policy and
// cites the pages it follows). Pure host code.
#include "pakv_sched.h"

#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

namespace {

constexpr int32_t kPageTokens = 16;

enum class State { kQueued, kRunning };

struct Request {
  int32_t prompt = 0;
  int32_t max_new = 0;
  int32_t pages = 0;          // logical pages per layer: ceil((prompt + max_new) / 16)
  int32_t shared_pages = 0;   // leading pages per layer referenced from the parent
  std::vector<int32_t> shared;  // [layer][shared_pages], references held since submit
  int32_t slot = -1;
  int32_t ctx = 0;            // tokens in the cache
  State state = State::kQueued;

  int32_t tokens() const { return prompt + max_new; }
};

int32_t pages_for(int64_t tokens) {
  return static_cast<int32_t>((tokens + kPageTokens - 1) / kPageTokens);
}

}  // namespace

struct pa_sched {
  int32_t num_pages = 0;
  int32_t layers = 0;
  int32_t max_batch = 0;
  int32_t stride = 0;
  int32_t mode = PA_BATCH_CONTINUOUS;
  std::vector<int32_t> refs;        // references per physical page
  std::vector<int32_t> free_pages;  // stack of unreferenced pages
  std::deque<int64_t> queue;        // queued request ids, arrival order
  std::unordered_map<int64_t, Request> reqs;
  std::vector<int64_t> slot_owner;  // request id per batch slot, 0 = empty
  std::vector<int32_t> bt;          // [layers][max_batch][stride]
  std::vector<int32_t> ctx;         // [max_batch]
  int64_t next_id = 1;
  int32_t running = 0;

  int32_t* row(int32_t layer, int32_t slot) {
    return bt.data() + (static_cast<size_t>(layer) * max_batch + slot) * stride;
  }
  // pages the request still needs from the free list
  int64_t need(const Request& r) const {
    return static_cast<int64_t>(layers) * (r.pages - r.shared_pages);
  }
  void release(int32_t page) {
    if (--refs[page] == 0) free_pages.push_back(page);
  }
  int32_t empty_slot() const {
    for (int32_t s = 0; s < max_batch; ++s)
      if (slot_owner[s] == 0) return s;
    return -1;
  }
  bool fits(const Request& r) const {
    return need(r) <= static_cast<int64_t>(free_pages.size()) && running < max_batch;
  }
  void place(int64_t id, Request& r) {
    const int32_t slot = empty_slot();
    r.slot = slot;
    r.state = State::kRunning;
    r.ctx = r.shared_pages * kPageTokens;
    slot_owner[slot] = id;
    for (int32_t l = 0; l < layers; ++l) {
      int32_t* bt_row = row(l, slot);
      for (int32_t j = 0; j < r.shared_pages; ++j)
        bt_row[j] = r.shared[static_cast<size_t>(l) * r.shared_pages + j];
      for (int32_t j = r.shared_pages; j < r.pages; ++j) {
        const int32_t p = free_pages.back();
        free_pages.pop_back();
        refs[p] = 1;
        bt_row[j] = p;
      }
    }
    r.shared.clear();   // the references now live in the block-table rows
    ctx[slot] = r.ctx;
    ++running;
  }
};

extern "C" {

pa_status pa_sched_create(pa_sched** out, int32_t num_pages, int32_t num_layers,
                          int32_t max_batch, int32_t max_pages_per_seq, int32_t mode) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_pages < 1 || num_layers < 1 || max_batch < 1 || max_pages_per_seq < 1)
    return PA_ERR_INVALID;
  if (mode != PA_BATCH_CONTINUOUS && mode != PA_BATCH_STATIC) return PA_ERR_INVALID;
  const size_t bt_size = static_cast<size_t>(num_layers) * max_batch * max_pages_per_seq;
  if (bt_size / num_layers / max_batch != static_cast<size_t>(max_pages_per_seq))
    return PA_ERR_INVALID;
  pa_sched* s = new (std::nothrow) pa_sched;
  if (!s) return PA_ERR_INVALID;
  try {
    s->num_pages = num_pages;
    s->layers = num_layers;
    s->max_batch = max_batch;
    s->stride = max_pages_per_seq;
    s->mode = mode;
    s->refs.assign(num_pages, 0);
    s->free_pages.reserve(num_pages);
    for (int32_t p = num_pages - 1; p >= 0; --p) s->free_pages.push_back(p);  // pops 0, 1, ...
    s->slot_owner.assign(max_batch, 0);
    s->bt.assign(bt_size, -1);
    s->ctx.assign(max_batch, 0);
  } catch (...) {
    delete s;
    return PA_ERR_INVALID;
  }
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* sched) { delete sched; }

static pa_status submit_impl(pa_sched* s, const Request& proto, int64_t* request_id) {
  if (proto.pages > s->stride) return PA_ERR_CAPACITY;
  if (s->need(proto) > s->num_pages) return PA_ERR_CAPACITY;
  const int64_t id = s->next_id++;
  try {
    s->reqs.emplace(id, proto);
    s->queue.push_back(id);
  } catch (...) {
    s->reqs.erase(id);
    return PA_ERR_INVALID;
  }
  *request_id = id;
  return PA_OK;
}

pa_status pa_sched_submit(pa_sched* sched, int32_t prompt_tokens, int32_t max_new_tokens,
                          int64_t* request_id) {
  if (!sched || !request_id) return PA_ERR_NULL;
  if (prompt_tokens < 0 || max_new_tokens < 0) return PA_ERR_INVALID;
  const int64_t tokens = static_cast<int64_t>(prompt_tokens) + max_new_tokens;
  if (tokens < 1) return PA_ERR_INVALID;
  if (tokens > static_cast<int64_t>(sched->stride) * kPageTokens) return PA_ERR_CAPACITY;
  Request r;
  r.prompt = prompt_tokens;
  r.max_new = max_new_tokens;
  r.pages = pages_for(tokens);
  return submit_impl(sched, r, request_id);
}

pa_status pa_sched_submit_shared(pa_sched* sched, int64_t parent_id, int32_t shared_tokens,
                                 int32_t prompt_tokens, int32_t max_new_tokens,
                                 int64_t* request_id) {
  if (!sched || !request_id) return PA_ERR_NULL;
  if (prompt_tokens < 0 || max_new_tokens < 0 || shared_tokens < 0) return PA_ERR_INVALID;
  if (shared_tokens > prompt_tokens) return PA_ERR_INVALID;
  const int64_t tokens = static_cast<int64_t>(prompt_tokens) + max_new_tokens;
  if (tokens < 1) return PA_ERR_INVALID;
  auto it = sched->reqs.find(parent_id);
  if (it == sched->reqs.end()) return PA_ERR_INVALID;
  const Request& parent = it->second;
  if (parent.state != State::kRunning) return PA_ERR_STATE;
  if (shared_tokens > parent.ctx) return PA_ERR_INVALID;
  if (tokens > static_cast<int64_t>(sched->stride) * kPageTokens) return PA_ERR_CAPACITY;
  Request r;
  r.prompt = prompt_tokens;
  r.max_new = max_new_tokens;
  r.pages = pages_for(tokens);
  r.shared_pages = shared_tokens / kPageTokens;
  if (r.pages > sched->stride || sched->need(r) > sched->num_pages) return PA_ERR_CAPACITY;
  try {
    r.shared.resize(static_cast<size_t>(sched->layers) * r.shared_pages);
  } catch (...) {
    return PA_ERR_INVALID;
  }
  for (int32_t l = 0; l < sched->layers; ++l) {
    const int32_t* prow = sched->row(l, parent.slot);
    for (int32_t j = 0; j < r.shared_pages; ++j)
      r.shared[static_cast<size_t>(l) * r.shared_pages + j] = prow[j];
  }
  const pa_status st = submit_impl(sched, r, request_id);
  if (st == PA_OK)
    for (int32_t p : sched->reqs[*request_id].shared) ++sched->refs[p];
  return st;
}

pa_status pa_sched_admit(pa_sched* sched, int64_t* admitted_ids, int32_t capacity,
                         int32_t* num_admitted) {
  if (!sched || !num_admitted) return PA_ERR_NULL;
  *num_admitted = 0;
  if (capacity < 0) return PA_ERR_INVALID;
  if (capacity > 0 && !admitted_ids) return PA_ERR_NULL;
  if (sched->mode == PA_BATCH_STATIC && sched->running > 0) return PA_OK;
  int32_t n = 0;
  while (n < capacity && !sched->queue.empty()) {
    const int64_t id = sched->queue.front();
    Request& r = sched->reqs[id];
    if (!sched->fits(r)) break;   // first in, first out: nothing overtakes the head
    sched->queue.pop_front();
    sched->place(id, r);
    admitted_ids[n++] = id;
  }
  *num_admitted = n;
  return PA_OK;
}

pa_status pa_sched_slot(const pa_sched* sched, int64_t request_id, int32_t* slot) {
  if (!sched || !slot) return PA_ERR_NULL;
  auto it = sched->reqs.find(request_id);
  if (it == sched->reqs.end()) return PA_ERR_INVALID;
  *slot = it->second.state == State::kRunning ? it->second.slot : -1;
  return PA_OK;
}

pa_status pa_sched_advance(pa_sched* sched, int64_t request_id, int32_t tokens) {
  if (!sched) return PA_ERR_NULL;
  auto it = sched->reqs.find(request_id);
  if (it == sched->reqs.end()) return PA_ERR_INVALID;
  Request& r = it->second;
  if (r.state != State::kRunning) return PA_ERR_STATE;
  if (tokens < 0 || static_cast<int64_t>(r.ctx) + tokens > r.tokens()) return PA_ERR_INVALID;
  r.ctx += tokens;
  sched->ctx[r.slot] = r.ctx;
  return PA_OK;
}

pa_status pa_sched_finish(pa_sched* sched, int64_t request_id) {
  if (!sched) return PA_ERR_NULL;
  auto it = sched->reqs.find(request_id);
  if (it == sched->reqs.end()) return PA_ERR_INVALID;
  Request& r = it->second;
  if (r.state == State::kQueued) {
    for (auto q = sched->queue.begin(); q != sched->queue.end(); ++q)
      if (*q == request_id) {
        sched->queue.erase(q);
        break;
      }
    for (int32_t p : r.shared) sched->release(p);
  } else {
    for (int32_t l = 0; l < sched->layers; ++l) {
      int32_t* bt_row = sched->row(l, r.slot);
      for (int32_t j = 0; j < r.pages; ++j) {
        sched->release(bt_row[j]);
        bt_row[j] = -1;
      }
    }
    sched->slot_owner[r.slot] = 0;
    sched->ctx[r.slot] = 0;
    --sched->running;
  }
  sched->reqs.erase(it);
  return PA_OK;
}

const int32_t* pa_sched_block_tables(const pa_sched* sched) {
  return sched ? sched->bt.data() : nullptr;
}

const int32_t* pa_sched_context_lens(const pa_sched* sched) {
  return sched ? sched->ctx.data() : nullptr;
}

pa_status pa_sched_stats(const pa_sched* sched, int32_t* free_pages, int32_t* queued,
                         int32_t* running) {
  if (!sched) return PA_ERR_NULL;
  if (free_pages) *free_pages = static_cast<int32_t>(sched->free_pages.size());
  if (queued) *queued = static_cast<int32_t>(sched->queue.size());
  if (running) *running = sched->running;
  return PA_OK;
}

}  // extern "C"
