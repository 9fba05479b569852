// Host-only part of libzp: error reporting, the refcounted block allocator,
// the compression planner and the capacity formula.
//
// Zipage (arXiv 2603.08743): Sec. 3 (block pool and block tables), Sec. 4.1
// (N_max cap, reserved block), Sec. 4.2 eq. (1) (capacity), Sec. 4.4 (shared
// prefix blocks, reference counts, target blocks), App. C.3 eq. (2).
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "zp_internal.h"

namespace zp {

static thread_local char g_err[512] = "";

zp_status fail(zp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace zp

using zp::fail;

extern "C" const char* zp_last_error(void) { return zp::g_err; }
extern "C" const char* zp_version(void) { return "zp 0.1.0 gfx950"; }

// ---------------------------------------------------------------------------
// Block pool. Free blocks sit in a min-heap so allocation is deterministic
// (lowest ids first), which keeps tests and traces reproducible.
// ---------------------------------------------------------------------------
struct zp_alloc {
  std::vector<int32_t> refcount;   // 0 = free
  std::vector<int32_t> free_heap;  // min-heap of free ids
};

namespace {

void heap_push(zp_alloc* a, int32_t id) {
  a->free_heap.push_back(id);
  std::push_heap(a->free_heap.begin(), a->free_heap.end(), std::greater<int32_t>());
}

int32_t heap_pop(zp_alloc* a) {
  std::pop_heap(a->free_heap.begin(), a->free_heap.end(), std::greater<int32_t>());
  int32_t id = a->free_heap.back();
  a->free_heap.pop_back();
  return id;
}

bool valid_id(const zp_alloc* a, int32_t id) {
  return id >= 0 && id < static_cast<int32_t>(a->refcount.size());
}

// Drops one reference of each id; the caller has validated the whole batch.
void decref_all(zp_alloc* a, const int32_t* ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i) {
    if (--a->refcount[ids[i]] == 0) heap_push(a, ids[i]);
  }
}

// Checks that dropping one reference per listed occurrence never takes a
// block below zero (the same id may appear several times).
zp_status check_decref(const zp_alloc* a, const int32_t* ids, int32_t n) {
  std::vector<std::pair<int32_t, int32_t>> cnt;
  cnt.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_id(a, ids[i])) return fail(ZP_EINVAL, "block id %d out of range", ids[i]);
    cnt.emplace_back(ids[i], 1);
  }
  std::sort(cnt.begin(), cnt.end());
  for (size_t i = 0; i < cnt.size();) {
    size_t j = i;
    while (j < cnt.size() && cnt[j].first == cnt[i].first) ++j;
    int32_t times = static_cast<int32_t>(j - i);
    if (a->refcount[cnt[i].first] < times)
      return fail(ZP_ESTATE, "block %d has refcount %d, cannot drop %d reference(s)",
                  cnt[i].first, a->refcount[cnt[i].first], times);
    i = j;
  }
  return ZP_OK;
}

bool contains(const int32_t* v, int32_t n, int32_t x) {
  for (int32_t i = 0; i < n; ++i)
    if (v[i] == x) return true;
  return false;
}

}  // namespace

extern "C" zp_alloc* zp_alloc_create(int32_t num_blocks) {
  if (num_blocks <= 0) {
    fail(ZP_EINVAL, "num_blocks must be positive (got %d)", num_blocks);
    return nullptr;
  }
  zp_alloc* a = new (std::nothrow) zp_alloc;
  if (!a) return nullptr;
  a->refcount.assign(num_blocks, 0);
  a->free_heap.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) a->free_heap[i] = i;  // sorted = valid min-heap
  return a;
}

extern "C" void zp_alloc_destroy(zp_alloc* a) { delete a; }

extern "C" zp_status zp_block_alloc(zp_alloc* a, int32_t n, int32_t* ids) {
  if (!a || n < 0 || (n > 0 && !ids)) return fail(ZP_EINVAL, "zp_block_alloc: bad arguments");
  if (n > static_cast<int32_t>(a->free_heap.size()))
    return fail(ZP_ENOBLOCKS, "need %d blocks, %zu free", n, a->free_heap.size());
  for (int32_t i = 0; i < n; ++i) {
    ids[i] = heap_pop(a);
    a->refcount[ids[i]] = 1;
  }
  return ZP_OK;
}

extern "C" zp_status zp_block_free(zp_alloc* a, const int32_t* ids, int32_t n) {
  if (!a || n < 0 || (n > 0 && !ids)) return fail(ZP_EINVAL, "zp_block_free: bad arguments");
  zp_status st = check_decref(a, ids, n);
  if (st != ZP_OK) return st;
  decref_all(a, ids, n);
  return ZP_OK;
}

extern "C" zp_status zp_block_share(zp_alloc* a, const int32_t* ids, int32_t n) {
  if (!a || n < 0 || (n > 0 && !ids)) return fail(ZP_EINVAL, "zp_block_share: bad arguments");
  for (int32_t i = 0; i < n; ++i) {
    if (!valid_id(a, ids[i])) return fail(ZP_EINVAL, "block id %d out of range", ids[i]);
    if (a->refcount[ids[i]] <= 0) return fail(ZP_ESTATE, "block %d is free", ids[i]);
  }
  for (int32_t i = 0; i < n; ++i) ++a->refcount[ids[i]];
  return ZP_OK;
}

extern "C" int32_t zp_block_refcount(const zp_alloc* a, int32_t id) {
  if (!a || !valid_id(a, id)) return -1;
  return a->refcount[id];
}

extern "C" int32_t zp_num_free(const zp_alloc* a) {
  return a ? static_cast<int32_t>(a->free_heap.size()) : -1;
}

extern "C" int32_t zp_num_blocks(const zp_alloc* a) {
  return a ? static_cast<int32_t>(a->refcount.size()) : -1;
}

// ---------------------------------------------------------------------------
// Compression planner (Zipage Sec. 4.1 and Sec. 4.4)
// ---------------------------------------------------------------------------

extern "C" zp_status zp_plan_compress(zp_alloc* a, const int32_t* table, int32_t n_blocks,
                                      int32_t n_max, int32_t* dst_table, int32_t* new_table,
                                      int32_t* release, int32_t* n_release) {
  if (!a || !table || !dst_table || !new_table || !release || !n_release)
    return fail(ZP_EINVAL, "zp_plan_compress: null pointer");
  if (n_max < 2 || n_blocks < n_max)
    return fail(ZP_EINVAL, "zp_plan_compress: need n_blocks >= n_max >= 2 (got %d, %d)",
                n_blocks, n_max);
  int32_t n_prefix = 0;
  for (int32_t i = 0; i < n_blocks; ++i) {
    if (!valid_id(a, table[i])) return fail(ZP_EINVAL, "block id %d out of range", table[i]);
    if (a->refcount[table[i]] <= 0) return fail(ZP_ESTATE, "table holds free block %d", table[i]);
    for (int32_t j = 0; j < i; ++j)
      if (table[j] == table[i]) return fail(ZP_EINVAL, "block %d repeated in table", table[i]);
    bool shared = a->refcount[table[i]] > 1;
    if (shared && n_prefix != i)
      return fail(ZP_EINVAL, "shared block %d does not belong to the table's prefix", table[i]);
    if (shared) ++n_prefix;
  }
  const int32_t n_targets = n_max - 1;
  // Fresh blocks: one per shared position among the targets, plus the
  // reserved block when no own block is left over.
  const int32_t new_targets = std::min(n_prefix, n_targets);
  const int32_t first_own_unused = std::max(n_prefix, n_targets);  // table index
  const bool reserved_is_new = first_own_unused >= n_blocks;
  const int32_t n_fresh = new_targets + (reserved_is_new ? 1 : 0);
  std::vector<int32_t> fresh(n_fresh);
  if (n_fresh > 0) {
    zp_status st = zp_block_alloc(a, n_fresh, fresh.data());
    if (st != ZP_OK) return st;
  }
  for (int32_t i = 0; i < n_targets; ++i) dst_table[i] = i < n_prefix ? fresh[i] : table[i];
  for (int32_t i = 0; i < n_targets; ++i) new_table[i] = dst_table[i];
  new_table[n_targets] = reserved_is_new ? fresh[new_targets] : table[first_own_unused];
  int32_t nr = 0;
  for (int32_t i = first_own_unused + (reserved_is_new ? 0 : 1); i < n_blocks; ++i)
    release[nr++] = table[i];
  *n_release = nr;
  return ZP_OK;
}

extern "C" zp_status zp_commit_compress(zp_alloc* a, const int32_t* old_table, int32_t n_blocks,
                                        const int32_t* new_table, int32_t n_max) {
  if (!a || !old_table || !new_table || n_blocks < 0 || n_max < 1)
    return fail(ZP_EINVAL, "zp_commit_compress: bad arguments");
  std::vector<int32_t> drop;
  for (int32_t i = 0; i < n_blocks; ++i)
    if (!contains(new_table, n_max, old_table[i])) drop.push_back(old_table[i]);
  for (int32_t i = 0; i < n_max; ++i) {
    if (!valid_id(a, new_table[i]) || a->refcount[new_table[i]] <= 0)
      return fail(ZP_ESTATE, "new table holds unallocated block %d", new_table[i]);
  }
  zp_status st = check_decref(a, drop.data(), static_cast<int32_t>(drop.size()));
  if (st != ZP_OK) return st;
  decref_all(a, drop.data(), static_cast<int32_t>(drop.size()));
  return ZP_OK;
}

extern "C" zp_status zp_abort_compress(zp_alloc* a, const int32_t* old_table, int32_t n_blocks,
                                       const int32_t* new_table, int32_t n_max) {
  if (!a || !old_table || !new_table || n_blocks < 0 || n_max < 1)
    return fail(ZP_EINVAL, "zp_abort_compress: bad arguments");
  std::vector<int32_t> fresh;
  for (int32_t i = 0; i < n_max; ++i)
    if (!contains(old_table, n_blocks, new_table[i])) fresh.push_back(new_table[i]);
  zp_status st = check_decref(a, fresh.data(), static_cast<int32_t>(fresh.size()));
  if (st != ZP_OK) return st;
  decref_all(a, fresh.data(), static_cast<int32_t>(fresh.size()));
  return ZP_OK;
}

// ---------------------------------------------------------------------------
// Capacity (Zipage eq. (1), eq. (2))
// ---------------------------------------------------------------------------

extern "C" zp_status zp_capacity(int64_t m_avail, int64_t m_kv, int64_t m_f, int64_t m_q,
                                 int32_t n_max, int64_t* max_concurrency, int64_t* num_blocks) {
  if (!max_concurrency || !num_blocks || m_avail < 0 || m_kv <= 0 || m_f < 0 || m_q < 0 ||
      n_max < 1)
    return fail(ZP_EINVAL, "zp_capacity: bad arguments");
  const __int128 blk = static_cast<__int128>(m_kv) + m_f;
  const __int128 den = blk * n_max + m_q;
  // M = floor(A / (blk*N_max + m_q));  N_total = floor(A*N_max / (blk*N_max + m_q))
  *max_concurrency = static_cast<int64_t>(static_cast<__int128>(m_avail) / den);
  *num_blocks = static_cast<int64_t>(static_cast<__int128>(m_avail) * n_max / den);
  return ZP_OK;
}

// ---------------------------------------------------------------------------
// Shared validation of the cache geometry
// ---------------------------------------------------------------------------

zp_status zp::validate_geom(const zp_geom* g, const char* who) {
  if (!g) return fail(ZP_EINVAL, "%s: geom is NULL", who);
  if (g->num_layers <= 0 || g->num_blocks <= 0 || g->num_kv_heads <= 0 || g->num_q_heads <= 0 ||
      g->max_slots < 0)
    return fail(ZP_EINVAL, "%s: sizes must be positive", who);
  if (g->dtype != ZP_DTYPE_F32 && g->dtype != ZP_DTYPE_BF16)
    return fail(ZP_EINVAL, "%s: unsupported dtype %d", who, g->dtype);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(ZP_EINVAL, "%s: head_dim must be 64 or 128 (got %d)", who, g->head_dim);
  if (g->block_size < 16 || g->block_size > 256 || (g->block_size & (g->block_size - 1)) != 0)
    return fail(ZP_EINVAL, "%s: block_size must be a power of two in [16, 256] (got %d)", who,
                g->block_size);
  if (g->num_q_heads % g->num_kv_heads != 0)
    return fail(ZP_EINVAL, "%s: num_q_heads must be a multiple of num_kv_heads", who);
  const int32_t grp = g->num_q_heads / g->num_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(ZP_EINVAL, "%s: group size %d not in {1,2,4,8}", who, grp);
  if (g->window < 1 || g->window > g->block_size)
    return fail(ZP_EINVAL, "%s: window must be in [1, block_size]", who);
  if ((grp * g->window) % 16 != 0 || grp * g->window > 128)
    return fail(ZP_EINVAL, "%s: g*window must be a multiple of 16 and at most 128 (got %d)", who,
                grp * g->window);
  if (g->n_max < 2) return fail(ZP_EINVAL, "%s: n_max must be >= 2", who);
  // Element offsets must fit the 64-bit arithmetic used by the kernels.
  const double kv_elems = double(g->num_layers) * g->num_blocks * g->num_kv_heads *
                          g->block_size * g->head_dim;
  if (kv_elems > 9.0e18) return fail(ZP_EINVAL, "%s: cache too large", who);
  return ZP_OK;
}

int32_t zp::decode_launch_shape(const zp_geom* g, int32_t batch, int32_t max_seq_len,
                                int32_t* waves) {
  // Items are (sequence, kv-head) pairs. The GPU holds `slots` resident
  // wavefronts (256 CUs x 4 SIMDs x the kernel's waves per SIMD). Measured
  // on MI355X at the Qwen3-8B decode shape (1793..2048 resident tokens):
  //  - 4 wavefronts per item fill the GPU at least once from 96 sequences
  //    on; one workgroup per item is best there, except when a second round
  //    is started but would be almost empty (between 1 and 1.125 rounds):
  //    then each item is split in two, which evens the rounds out (97 and
  //    104 sequences: +2.6% and +3.2%). From 112 sequences on the unsplit
  //    launch is faster (+2.0..3.7% at 112..144; 256 and 512 sequences:
  //    +4.4% and +4.9%);
  //  - below one round, but above a quarter of one, more splits only add
  //    merge work: one 4-wave workgroup per item (64 sequences: 5.86 TB/s
  //    vs 5.24 with 4-way splits). Splitting in two where the workgroups
  //    per CU sit just above 1 or 2 gained 2..11% on uniform 1793..2048
  //    lengths (66..76 sequences) but cost 3% of the serving run's tokens/s
  //    (ragged lengths), and 6 or 8 wavefronts per workgroup measured
  //    slower than 4 at 24..88 sequences;
  //  - at most a quarter of a round (<= 32 sequences of 8 kv-heads): one
  //    workgroup with a whole CU's waves per item, split only as far as
  //    needed to reach one round (32 sequences: 5.30 vs 4.34 TB/s).
  // A split covers at least 256 tokens and at most ~1000 blocks
  // (kMaxSplitPages = 1024).
  const int64_t mw = decode_waves_per_simd(static_cast<int>(elem_size(g)), g->head_dim,
                                           group_size(g));
  const int64_t slots = int64_t(256) * 4 * mw;
  const int64_t items = std::max<int64_t>(1, int64_t(batch) * g->num_kv_heads);
  const int64_t len = std::max<int32_t>(max_seq_len, 1);
  int64_t w = 4, splits = 1;
  if (4 * items >= slots) {
    if (4 * items > slots && 8 * 4 * items < 9 * slots) splits = 2;
  } else if (4 * mw * items <= slots) {
    w = 4 * mw;
    splits = std::max<int64_t>(1, slots / (w * items));
  }
  int64_t s = std::max<int64_t>(256, (len + splits - 1) / splits);
  s = std::min<int64_t>(s, int64_t(1000) * g->block_size);
  s = (s + 63) / 64 * 64;
  *waves = static_cast<int32_t>(w);
  return static_cast<int32_t>(s);
}
