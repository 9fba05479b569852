// Request scheduler of libzp: constrained and hybrid scheduling with
// query-cache slots, preemption and shared prefixes.
//
// Zipage (arXiv 2603.08743): Sec. 4.1 (N_max cap, trigger once N >= N_max
// blocks are full, reserved block), Sec. 4.2 (one query-cache slot per
// compressing request, M in all), Sec. 4.3 (constrained scheduling; the four
// rules of hybrid scheduling; Fig. 2 request states), Sec. 4.4 (shared prefix
// blocks, target blocks, preemption of the last uncompressed request).
// The policy is spelled out step by step beside the declarations in zp.h.
//
// Host-only and deterministic: ids are taken lowest first (the block pool is
// a min-heap, slots are scanned from 0), queues are plain FIFO / vectors.
#include <algorithm>
#include <deque>
#include <map>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "zp_internal.h"

using zp::fail;

namespace {

struct Req {
  int32_t rid = 0, prompt = 0, max_new = 0, group = -1, prefix_len = 0;
  int32_t n_max = 0;  // this request's cap (blocks kept + the reserved one)
  int32_t base_n_max = 0;  // the cap it was added with (adaptive N_max grows from it)
  int32_t gen = 0;  // outputs produced
  int32_t n = 0;    // resident tokens
  int32_t slot = -1;
  int32_t state = ZP_REQ_WAITING;
  bool compressed = false, due = false, holds_prefix = false;
  std::vector<int32_t> table;
  std::vector<int32_t> plan_old, plan_new;  // while compressing
};

struct Group {
  std::vector<int32_t> blocks;
  int32_t holders = 0;
  int64_t step = 0;  // step that wrote the blocks
};

}  // namespace

struct zp_sched {
  zp_sched_config cfg{};
  zp_alloc* pool = nullptr;
  std::unordered_map<int32_t, std::unique_ptr<Req>> reqs;
  std::deque<Req*> waiting;
  std::vector<Req*> running;
  std::map<int32_t, Group> groups;
  std::map<int32_t, int32_t> group_len;
  std::vector<uint8_t> slot_used;
  int64_t slot_caps = 0;  // sum of n_max over the slot holders
  int32_t slot_count = 0;
  int64_t t = 0;
  int32_t unfinished = 0;
  zp_sched_stats st{};
  // scratch of one step
  std::vector<int32_t> ids;

  ~zp_sched() { zp_alloc_destroy(pool); }
};

namespace {

int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

bool needs_slot(const zp_sched* s, const Req* r, int32_t p) {
  const int32_t b = s->cfg.block_size;
  return p / b >= r->n_max - 1 && p % b >= b - s->cfg.window;
}

bool is_due(const zp_sched* s, const Req* r) {
  const int32_t b = s->cfg.block_size;
  return r->n > 0 && r->n % b == 0 && r->n / b >= r->n_max;
}

// A slot is free and the holders' caps, r's included, fit the pool: the
// per-request form of M <= N_total / N_max.
bool slot_fits(const zp_sched* s, const Req* r) {
  return s->slot_count < s->cfg.num_slots && s->slot_caps + r->n_max <= s->cfg.num_blocks;
}

int32_t share_count(const zp_sched* s, const Req* r) {
  return (s->cfg.prefix_sharing && r->group >= 0) ? r->prefix_len / s->cfg.block_size : 0;
}

// Gives r the lowest free slot (the caller checked slot_fits).
void take_slot(zp_sched* s, Req* r) {
  for (int32_t i = 0; i < s->cfg.num_slots; ++i) {
    if (!s->slot_used[i]) {
      s->slot_used[i] = 1;
      r->slot = i;
      ++s->slot_count;
      s->slot_caps += r->n_max;
      return;
    }
  }
}

void leave_group(zp_sched* s, Req* r) {
  if (!r->holds_prefix) return;
  auto it = s->groups.find(r->group);
  if (--it->second.holders == 0) s->groups.erase(it);
  r->holds_prefix = false;
}

void release(zp_sched* s, Req* r) {
  if (!r->table.empty())
    zp_block_free(s->pool, r->table.data(), static_cast<int32_t>(r->table.size()));
  leave_group(s, r);
  if (r->slot >= 0) {
    s->slot_used[r->slot] = 0;
    --s->slot_count;
    s->slot_caps -= r->n_max;
  }
  r->table.clear();
  r->slot = -1;
  r->n = 0;
  r->due = false;
  s->running.erase(std::find(s->running.begin(), s->running.end(), r));
}

void preempt(zp_sched* s, Req* v, zp_sched_step_out* out) {
  release(s, v);
  v->state = ZP_REQ_WAITING;
  s->waiting.push_front(v);
  out->preempted[out->n_preempted++] = v->rid;
  ++s->st.preemptions;
}

Req* victim(zp_sched* s) {
  for (auto it = s->running.rbegin(); it != s->running.rend(); ++it) {
    Req* v = *it;
    if (s->cfg.prefix_sharing) {
      if (v->state == ZP_REQ_RUNNING && !v->compressed) return v;
    } else if (s->cfg.policy == ZP_SCHED_HYBRID) {
      if (v->slot < 0) return v;
    }
  }
  return nullptr;
}

void finish(zp_sched* s, Req* r, zp_sched_step_out* out) {
  release(s, r);
  r->state = ZP_REQ_FINISHED;
  --s->unfinished;
  ++s->st.finished;
  out->finished[out->n_finished++] = r->rid;
}

// Adaptive N_max: the cap follows the request's actual sequence length L =
// prompt + outputs, min(cfg n_max, base + L / nmax_growth), never falling; a
// slot holder's raise is cut so the holders' caps still fit the pool.
void grow(zp_sched* s, Req* r) {
  if (s->cfg.nmax_growth <= 0) return;
  const int64_t len = int64_t(r->prompt) + r->gen;
  int64_t want = std::min<int64_t>(s->cfg.n_max, r->base_n_max + len / s->cfg.nmax_growth);
  if (want <= r->n_max) return;
  if (r->slot >= 0) {
    want = std::min<int64_t>(want, r->n_max + int64_t(s->cfg.num_blocks) - s->slot_caps);
    if (want <= r->n_max) return;
    s->slot_caps += want - r->n_max;
  }
  r->n_max = static_cast<int32_t>(want);
}

void advance(zp_sched* s, Req* r, zp_sched_step_out* out) {
  if (r->gen >= r->max_new) {
    finish(s, r, out);
    return;
  }
  grow(s, r);
  if (is_due(s, r)) r->due = true;
}

// Rule (a): plans the compression of a due request; may preempt.
zp_status try_compress(zp_sched* s, Req* r, zp_sched_step_out* out) {
  const int32_t nmax = r->n_max, cap = s->cfg.table_cap, cmax = s->cfg.n_max;
  const int32_t nb = static_cast<int32_t>(r->table.size());
  std::vector<int32_t> dst(nmax - 1), nw(nmax), rel(nb);
  int32_t nrel = 0;
  for (;;) {
    zp_status st = zp_plan_compress(s->pool, r->table.data(), nb, nmax, dst.data(), nw.data(),
                                    rel.data(), &nrel);
    if (st == ZP_OK) break;
    if (st != ZP_ENOBLOCKS) return st;
    Req* v = victim(s);
    if (!v) return ZP_OK;  // waits
    preempt(s, v, out);
    if (v == r) return ZP_OK;
  }
  leave_group(s, r);
  r->plan_old = r->table;
  r->plan_new = nw;
  r->state = ZP_REQ_COMPRESSING;
  r->due = false;
  const int32_t i = out->n_comp++;
  out->c_rid[i] = r->rid;
  out->c_slot[i] = r->slot;
  out->c_first[i] = r->compressed ? 0 : 1;
  out->c_nblocks[i] = nb;
  out->c_nmax[i] = nmax;
  int32_t* src = out->c_src + static_cast<int64_t>(i) * cap;
  for (int32_t j = 0; j < cap; ++j) src[j] = j < nb ? r->table[j] : -1;
  int32_t* d = out->c_dst + static_cast<int64_t>(i) * (cmax - 1);
  for (int32_t j = 0; j < cmax - 1; ++j) d[j] = j < nmax - 1 ? dst[j] : -1;
  int32_t* w = out->c_new + static_cast<int64_t>(i) * cmax;
  for (int32_t j = 0; j < cmax; ++j) w[j] = j < nmax ? nw[j] : -1;
  ++s->st.compressions;
  return ZP_OK;
}

void emit_entry(zp_sched* s, zp_sched_step_out* out, const Req* r, int32_t ctx, int32_t pos,
                int32_t len) {
  const int32_t i = out->n++;
  const int32_t cap = s->cfg.table_cap;
  out->rid[i] = r->rid;
  out->slot[i] = r->slot;
  out->ctx[i] = ctx;
  out->pos[i] = pos;
  out->len[i] = len;
  int32_t* row = out->tables + static_cast<int64_t>(i) * cap;
  const int32_t nt = static_cast<int32_t>(r->table.size());
  for (int32_t j = 0; j < cap; ++j) row[j] = j < nt ? r->table[j] : -1;
}

// Rule (c): admission. Returns the number admitted (entries emitted).
zp_status admit(zp_sched* s, zp_sched_step_out* out, int32_t* admitted,
                std::vector<Req*>* batch) {
  const int32_t b = s->cfg.block_size;
  int64_t tokens = 0;
  *admitted = 0;
  while (!s->waiting.empty() && static_cast<int32_t>(s->running.size()) < s->cfg.max_running) {
    Req* r = s->waiting.front();
    const int32_t L = r->prompt + r->gen;
    Group* g = nullptr;
    if (share_count(s, r) > 0) {
      auto it = s->groups.find(r->group);
      if (it != s->groups.end() && it->second.step < s->t) g = &it->second;
    }
    const int32_t nshare = g ? static_cast<int32_t>(g->blocks.size()) : 0;
    const int32_t chunk = L - nshare * b;
    if (*admitted > 0 && tokens + chunk > s->cfg.max_prefill_tokens) break;
    const int32_t need = cdiv(L, b) - nshare;
    if (nshare + need > s->cfg.table_cap)
      return fail(ZP_ESTATE, "zp_sched_step: request %d needs %d blocks > table_cap %d", r->rid,
                  nshare + need, s->cfg.table_cap);
    if (zp_num_free(s->pool) < need) break;
    const bool with_slot =
        static_cast<int32_t>(s->running.size()) < s->cfg.num_slots && slot_fits(s, r);
    if (!with_slot && (s->cfg.policy == ZP_SCHED_CONSTRAINED || needs_slot(s, r, L - 1))) break;
    s->waiting.pop_front();
    r->table.clear();
    if (g) {
      zp_block_share(s->pool, g->blocks.data(), nshare);
      ++g->holders;
      r->table = g->blocks;
      r->holds_prefix = true;
    }
    s->ids.resize(std::max(need, 1));
    zp_block_alloc(s->pool, need, s->ids.data());
    r->table.insert(r->table.end(), s->ids.begin(), s->ids.begin() + need);
    const int32_t k = share_count(s, r);
    if (!g && k > 0 && s->groups.find(r->group) == s->groups.end()) {
      Group& ng = s->groups[r->group];
      ng.blocks.assign(r->table.begin(), r->table.begin() + k);
      ng.holders = 1;
      ng.step = s->t;
      r->holds_prefix = true;
    }
    r->slot = -1;
    if (with_slot) take_slot(s, r);
    r->state = ZP_REQ_RUNNING;
    s->running.push_back(r);
    emit_entry(s, out, r, nshare * b, nshare * b, chunk);
    batch->push_back(r);
    tokens += chunk;
    ++*admitted;
  }
  return ZP_OK;
}

// Rule (d): decode batch.
zp_status decode(zp_sched* s, zp_sched_step_out* out, std::vector<Req*>* sched) {
  const int32_t b = s->cfg.block_size;
  const std::vector<Req*> order = s->running;
  for (Req* r : order) {
    // a request preempted earlier in this scan is WAITING now
    if (r->state != ZP_REQ_RUNNING || r->due) continue;
    if (r->slot < 0 && needs_slot(s, r, r->n)) {
      ++out->n_blocked;
      continue;
    }
    if (r->n == static_cast<int32_t>(r->table.size()) * b) {
      bool gone = false;
      while (zp_num_free(s->pool) == 0) {
        Req* v = victim(s);
        if (!v) break;
        preempt(s, v, out);
        auto it = std::find(sched->begin(), sched->end(), v);
        if (it != sched->end()) sched->erase(it);
        if (v == r) {
          gone = true;
          break;
        }
      }
      if (gone) continue;
      if (zp_num_free(s->pool) == 0) {
        ++out->n_blocked;
        continue;
      }
      if (static_cast<int32_t>(r->table.size()) >= s->cfg.table_cap)
        return fail(ZP_ESTATE, "zp_sched_step: request %d would exceed table_cap %d", r->rid,
                    s->cfg.table_cap);
      int32_t id = -1;
      zp_block_alloc(s->pool, 1, &id);
      r->table.push_back(id);
    }
    sched->push_back(r);
  }
  for (Req* r : *sched) emit_entry(s, out, r, r->n, r->prompt + r->gen - 1, 1);
  return ZP_OK;
}

}  // namespace

extern "C" zp_sched* zp_sched_create(const zp_sched_config* cfg) {
  if (!cfg) {
    fail(ZP_EINVAL, "zp_sched_create: cfg is NULL");
    return nullptr;
  }
  const zp_sched_config& c = *cfg;
  if (c.num_blocks <= 0 || c.block_size <= 0 || (c.block_size & (c.block_size - 1)) != 0 ||
      c.window < 1 || c.window > c.block_size || c.n_max < 2 || c.num_slots < 1 ||
      c.max_running < 1 || c.max_prefill_tokens < 1 || c.table_cap < c.n_max ||
      c.nmax_growth < 0 ||
      (c.policy != ZP_SCHED_CONSTRAINED && c.policy != ZP_SCHED_HYBRID)) {
    fail(ZP_EINVAL, "zp_sched_create: invalid configuration");
    return nullptr;
  }
  zp_sched* s = new (std::nothrow) zp_sched;
  if (!s) {
    fail(ZP_EINVAL, "zp_sched_create: out of host memory");
    return nullptr;
  }
  s->cfg = c;
  s->pool = zp_alloc_create(c.num_blocks);
  if (!s->pool) {
    delete s;
    return nullptr;
  }
  s->slot_used.assign(c.num_slots, 0);
  return s;
}

extern "C" void zp_sched_destroy(zp_sched* s) { delete s; }

extern "C" zp_status zp_sched_add(zp_sched* s, int32_t rid, int32_t prompt_len, int32_t max_new,
                                  int32_t prefix_group, int32_t prefix_len, int32_t n_max) {
  if (!s) return fail(ZP_EINVAL, "zp_sched_add: NULL scheduler");
  if (s->reqs.count(rid)) return fail(ZP_EINVAL, "zp_sched_add: request %d exists", rid);
  if (prompt_len < 1 || max_new < 1)
    return fail(ZP_EINVAL, "zp_sched_add: prompt_len and max_new must be >= 1");
  if (n_max == 0) n_max = s->cfg.n_max;
  if (n_max < 2 || n_max > s->cfg.n_max)
    return fail(ZP_EINVAL, "zp_sched_add: n_max %d outside [2, %d]", n_max, s->cfg.n_max);
  if (cdiv(prompt_len, s->cfg.block_size) > s->cfg.table_cap)
    return fail(ZP_EINVAL, "zp_sched_add: prompt of %d tokens exceeds table_cap blocks",
                prompt_len);
  if (prefix_group >= 0) {
    if (prefix_len < 0 || prefix_len >= prompt_len)
      return fail(ZP_EINVAL, "zp_sched_add: need 0 <= prefix_len < prompt_len");
    auto it = s->group_len.find(prefix_group);
    if (it != s->group_len.end() && it->second != prefix_len)
      return fail(ZP_EINVAL, "zp_sched_add: group %d has prefix_len %d", prefix_group,
                  it->second);
    s->group_len[prefix_group] = prefix_len;
  }
  auto r = std::make_unique<Req>();
  r->rid = rid;
  r->prompt = prompt_len;
  r->max_new = max_new;
  r->group = prefix_group >= 0 ? prefix_group : -1;
  r->prefix_len = prefix_group >= 0 ? prefix_len : 0;
  r->n_max = n_max;
  r->base_n_max = n_max;
  s->waiting.push_back(r.get());
  s->reqs.emplace(rid, std::move(r));
  ++s->unfinished;
  return ZP_OK;
}

extern "C" zp_status zp_sched_step(zp_sched* s, zp_sched_step_out* out) {
  if (!s || !out || !out->rid || !out->slot || !out->ctx || !out->pos || !out->len ||
      !out->tables ||
      !out->c_rid || !out->c_slot || !out->c_first || !out->c_nblocks || !out->c_src ||
      !out->c_dst || !out->c_new || !out->c_nmax || !out->finished || !out->preempted)
    return fail(ZP_EINVAL, "zp_sched_step: NULL argument");
  ++s->t;
  ++s->st.steps;
  out->kind = ZP_STEP_IDLE;
  out->n = out->n_comp = out->n_finished = out->n_preempted = out->n_blocked = 0;

  // (a) compressions of due requests, in queue order
  {
    const std::vector<Req*> order = s->running;
    for (Req* r : order) {
      if (r->state != ZP_REQ_RUNNING || !r->due) continue;  // preempted ones are WAITING
      zp_status st = try_compress(s, r, out);
      if (st != ZP_OK) return st;
    }
  }
  // (b) slots to the foremost slot-less requests among the first M, in
  // order (no overtaking when the caps do not fit)
  const int32_t m = std::min<int32_t>(s->cfg.num_slots, static_cast<int32_t>(s->running.size()));
  for (int32_t i = 0; i < m; ++i) {
    Req* r = s->running[i];
    if (r->slot >= 0) continue;
    if (!slot_fits(s, r)) break;
    take_slot(s, r);
  }

  // (c) admission, else (d) decode
  std::vector<Req*> batch;
  int32_t admitted = 0;
  zp_status st = admit(s, out, &admitted, &batch);
  if (st != ZP_OK) return st;
  if (admitted > 0) {
    out->kind = ZP_STEP_PREFILL;
    ++s->st.prefill_steps;
    for (int32_t i = 0; i < out->n; ++i) s->st.prefill_tokens += out->len[i];
    for (Req* r : batch) {
      r->n = r->prompt + r->gen;
      ++r->gen;
    }
    for (Req* r : batch) advance(s, r, out);
  } else {
    st = decode(s, out, &batch);
    if (st != ZP_OK) return st;
    if (!batch.empty()) {
      out->kind = ZP_STEP_DECODE;
      ++s->st.decode_steps;
      s->st.decode_tokens += static_cast<int64_t>(batch.size());
      for (Req* r : batch) {
        ++r->n;
        ++r->gen;
      }
      for (Req* r : batch) advance(s, r, out);
    } else {
      ++s->st.idle_steps;
    }
  }
  s->st.blocked += out->n_blocked;
  return ZP_OK;
}

extern "C" zp_status zp_sched_compress_done(zp_sched* s, int32_t rid) {
  if (!s) return fail(ZP_EINVAL, "zp_sched_compress_done: NULL scheduler");
  auto it = s->reqs.find(rid);
  if (it == s->reqs.end() || it->second->state != ZP_REQ_COMPRESSING)
    return fail(ZP_ESTATE, "zp_sched_compress_done: request %d is not compressing", rid);
  Req* r = it->second.get();
  zp_status st = zp_commit_compress(s->pool, r->plan_old.data(),
                                    static_cast<int32_t>(r->plan_old.size()), r->plan_new.data(),
                                    static_cast<int32_t>(r->plan_new.size()));
  if (st != ZP_OK) return st;
  r->table = r->plan_new;
  r->plan_old.clear();
  r->plan_new.clear();
  r->n = (r->n_max - 1) * s->cfg.block_size;
  r->compressed = true;
  r->state = ZP_REQ_RUNNING;
  return ZP_OK;
}

extern "C" zp_status zp_sched_get_stats(const zp_sched* s, zp_sched_stats* out) {
  if (!s || !out) return fail(ZP_EINVAL, "zp_sched_get_stats: NULL argument");
  *out = s->st;
  out->waiting = static_cast<int64_t>(s->waiting.size());
  out->running = static_cast<int64_t>(s->running.size());
  int64_t comp = 0, slots = 0;
  for (const Req* r : s->running) {
    comp += r->state == ZP_REQ_COMPRESSING;
    slots += r->slot >= 0;
  }
  out->compressing = comp;
  out->slots_in_use = slots;
  out->free_blocks = zp_num_free(s->pool);
  return ZP_OK;
}

extern "C" zp_status zp_sched_request(const zp_sched* s, int32_t rid, zp_sched_req_info* info,
                                      int32_t* table) {
  if (!s || !info) return fail(ZP_EINVAL, "zp_sched_request: NULL argument");
  auto it = s->reqs.find(rid);
  if (it == s->reqs.end()) {
    *info = zp_sched_req_info{ZP_REQ_UNKNOWN, 0, 0, -1, 0, 0, 0};
    return ZP_OK;
  }
  const Req* r = it->second.get();
  info->state = r->state;
  info->n = r->n;
  info->gen = r->gen;
  info->slot = r->slot;
  info->compressed = r->compressed ? 1 : 0;
  info->ntable = static_cast<int32_t>(r->table.size());
  info->n_max = r->n_max;
  if (table) std::copy(r->table.begin(), r->table.end(), table);
  return ZP_OK;
}

extern "C" int32_t zp_sched_unfinished(const zp_sched* s) { return s ? s->unfinished : -1; }

extern "C" const zp_alloc* zp_sched_allocator(const zp_sched* s) { return s ? s->pool : nullptr; }
