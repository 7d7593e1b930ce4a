// Host side of the C ABI declared in include/gqa.h: cache state, argument
// checks, the page allocator and the kernel launches.
//
// Sources: page "Prefill：整层状态演化与 KV 建立" (2.1 preconditions fail before
// anything runs; 2.5 LayerCache and invariants; 2.6 write the valid tokens'
// used K/V at their positions, then attend; 2.11 position ids restarting after
// reuse are a failure) and page "KV Cache 与 Prefill/Decode 推理路径"
// (PagedAttention lesson: per-request block table, logical block t/16 at offset
// t%16, any free block when the last one is full; prompt-edit lesson: keep
// [0,m), truncate, re-prefill the suffix).
//
// Rules fixed by this library where the pages leave a choice:
//  * slot = position: the valid tokens of a call must carry positions
//    c, c+1, ... where c is the current length of that (sequence, layer);
//  * the valid tokens of a row may have padding before, after and between
//    them; each run of consecutive valid tokens is one launch entry;
//  * a page serves every layer of its sequence; the first layer that needs a
//    logical page takes it from the front of the free list, in batch order then
//    logical-page order; truncation returns pages to the back in ascending
//    logical order, remap returns source pages in the order given;
//  * a page may be referenced by several sequences' tables (kv_cache_fork); it
//    counts its references and returns to the back of the free list when the
//    last one goes.  A write into a page with more than one reference first
//    copies the page (every layer) to a page from the front of the free list
//    and points the writer's entry at the copy, in batch order, a row's copy
//    before its new pages ([P3] prefix-sharing lesson: shared blocks live until
//    no request references them; a fork inside a block is a question of
//    copy-on-write);
//  * every check runs before any state changes or any launch.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <deque>
#include <string>
#include <utility>
#include <vector>

#include "gqa.h"
#include "common.hpp"

#define GQA_EXPORT extern "C" __attribute__((visibility("default")))

using gqa::kPage;
using gqa::kMaxSeqPerLaunch;

struct gqa_cache {
  gqa_cache_config cfg;
  void* k_pool;
  void* v_pool;
  int32_t* d_table;
  float* d_rope;
  std::deque<int32_t> free_list;
  std::vector<std::vector<int32_t>> pages;  // per sequence: physical page of each logical page
  std::vector<int32_t> len;                 // [seq * num_layers + layer]
  std::vector<float> rope_host;             // [max_position][d/2][2]
  bool rope_uploaded = false;
  std::vector<std::pair<int32_t, int32_t>> pending;  // block-table entries to write on the device
  std::vector<std::pair<int32_t, int32_t>> copies;   // (src, dst) page copies to make before the next write
  std::vector<int32_t> ref;                 // table entries that reference each page (0 = free)
  int elt = 2;
  int64_t layer_elems = 0;                  // elements of one layer of a pool
  int64_t page_elems = 0;                   // elements of one page (all kv heads) of one layer
};

namespace {

thread_local std::string g_err;

gqa_status fail(gqa_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

#ifndef GQA_DECODE_TARGET_BLOCKS
#define GQA_DECODE_TARGET_BLOCKS 4096
#endif
#ifndef GQA_DECODE_MIN_PAGES
#define GQA_DECODE_MIN_PAGES 16
#endif
constexpr int kDecodeTargetBlocks = GQA_DECODE_TARGET_BLOCKS;   // workgroups a decode launch aims for
constexpr int kDecodeMinPages = GQA_DECODE_MIN_PAGES;           // pages per split at least

gqa_status check_config(const gqa_cache_config* c) {
  if (!c) return fail(GQA_ERR_ARG, "config is null");
  if (c->num_layers < 1 || c->num_kv_heads < 1 || c->num_pages < 1 || c->max_seqs < 1 ||
      c->max_pages_per_seq < 1)
    return fail(GQA_ERR_ARG, "layers, kv heads, pages, sequences and table width must be >= 1");
  if (c->page_size != kPage) return fail(GQA_ERR_UNSUPPORTED, "page_size must be 16");
  if (c->dtype != GQA_F32 && c->dtype != GQA_BF16) return fail(GQA_ERR_DTYPE, "unknown dtype");
  if (c->head_dim < 1 || c->head_dim > 128) return fail(GQA_ERR_UNSUPPORTED, "head_dim must be 1..128");
  if (c->dtype == GQA_BF16 && c->head_dim != 64 && c->head_dim != 128)
    return fail(GQA_ERR_UNSUPPORTED, "bf16 caches need head_dim 64 or 128");
  // the bf16 kernels address one layer of a pool with 32-bit byte offsets
  if (c->dtype == GQA_BF16 &&
      static_cast<int64_t>(c->num_pages) * c->num_kv_heads * kPage * c->head_dim * 2 > 0xffffffffLL)
    return fail(GQA_ERR_UNSUPPORTED, "one layer of a bf16 pool must stay below 4 GiB");
  if (c->rope_style != 0 && c->rope_style != 1) return fail(GQA_ERR_UNSUPPORTED, "rope_style must be 0 or 1");
  if (c->rope_style == 1) {
    if (c->head_dim % 2) return fail(GQA_ERR_ARG, "rotation needs an even head_dim");
    if (c->max_position < 1) return fail(GQA_ERR_ARG, "max_position must be >= 1");
    if (!(c->rope_theta > 0.0)) return fail(GQA_ERR_ARG, "rope_theta must be > 0");
  }
  if (c->window < 0) return fail(GQA_ERR_ARG, "window must be >= 0");
  if (c->window > 0 && c->max_pages_per_seq < ceil_div(c->window, kPage) + 1)
    return fail(GQA_ERR_UNSUPPORTED, "a ring must hold a window plus one page");
  return GQA_OK;
}

// Block-table entries a sequence of this length holds: one per logical page,
// at most the table width in a ring (logical page L lives in entry L mod R).
int64_t table_entries(const gqa_cache_config& cf, int64_t length) {
  const int64_t e = ceil_div(length, kPage);
  return cf.window ? std::min<int64_t>(e, cf.max_pages_per_seq) : e;
}

// First position a ring still holds (0 without a window).
int32_t resident_from(const gqa_cache_config& cf, int32_t length) {
  if (!cf.window || length == 0) return 0;
  return std::max(0, ((length - 1) / kPage - cf.max_pages_per_seq + 1) * kPage);
}

// Strided 4-D tensor of the cache dtype with the given logical shape.
gqa_status check_tensor(const gqa_tensor* t, const char* name, int dtype, int64_t s0, int64_t s1, int64_t s2,
                        int64_t s3) {
  if (!t) return fail(GQA_ERR_ARG, std::string(name) + " is null");
  if (t->dtype != dtype) return fail(GQA_ERR_DTYPE, std::string(name) + " dtype differs from the cache dtype");
  const int64_t want[4] = {s0, s1, s2, s3};
  for (int i = 0; i < 4; ++i)
    if (t->shape[i] != want[i]) return fail(GQA_ERR_SHAPE, std::string(name) + " has the wrong shape");
  if (t->stride[3] != 1) return fail(GQA_ERR_SHAPE, std::string(name) + " innermost stride must be 1");
  for (int i = 0; i < 3; ++i)
    if (t->stride[i] < 0) return fail(GQA_ERR_SHAPE, std::string(name) + " has a negative stride");
  const int64_t numel = s0 * s1 * s2 * s3;
  if (numel == 0) return GQA_OK;
  if (!t->data) return fail(GQA_ERR_ARG, std::string(name) + " data is null");
  const uintptr_t p = reinterpret_cast<uintptr_t>(t->data);
  if (dtype == GQA_BF16) {
    if (p % 16) return fail(GQA_ERR_SHAPE, std::string(name) + " must be 16-byte aligned");
    for (int i = 0; i < 3; ++i)
      if (t->stride[i] % 8) return fail(GQA_ERR_SHAPE, std::string(name) + " strides must keep rows 16-byte aligned");
  } else if (p % 4) {
    return fail(GQA_ERR_SHAPE, std::string(name) + " must be 4-byte aligned");
  }
  return GQA_OK;
}

gqa_status check_seqs(const gqa_cache* c, int32_t B, const int32_t* seq_ids) {
  if (B < 0) return fail(GQA_ERR_ARG, "B must be >= 0");
  if (B > 0 && !seq_ids) return fail(GQA_ERR_ARG, "seq_ids is null");
  std::vector<char> seen(c->cfg.max_seqs, 0);
  for (int b = 0; b < B; ++b) {
    const int s = seq_ids[b];
    if (s < 0 || s >= c->cfg.max_seqs) return fail(GQA_ERR_ARG, "sequence id out of range");
    if (seen[s]) return fail(GQA_ERR_ARG, "a sequence appears twice in one call");
    seen[s] = 1;
  }
  return GQA_OK;
}

// One launch entry: a run of consecutive valid rows of batch row b.  A row
// whose valid tokens have holes between them gives one entry per run; a row
// with none gives one empty entry, which only zeroes its output rows.
struct Entry {
  int32_t b;          // batch row: index of Q/K/V/O and of seq_ids
  int32_t start;      // position of the run's first token
  int32_t count;      // tokens in the run
  int32_t row0;       // rectangular row of its first token
  int32_t zlo, zhi;   // rectangular rows [zlo, zhi) whose padding this entry writes as 0
};

// Runs of valid rows of every batch row, positions c[b], c[b]+1, ... in row
// order; count[b] = valid tokens of row b.  GQA_ERR_MASK for entries not 0/1.
gqa_status mask_entries(const uint8_t* mask, int64_t n, int32_t B, const int32_t* c, std::vector<Entry>* out,
                        std::vector<int32_t>* count) {
  out->clear();
  count->assign(B, 0);
  for (int b = 0; b < B; ++b) {
    const uint8_t* m = mask + static_cast<int64_t>(b) * n;
    const size_t first = out->size();
    int32_t pos = c[b];
    for (int64_t i = 0; i < n; ++i) {
      if (m[i] > 1) return fail(GQA_ERR_MASK, "mask entries must be 0 or 1");
      if (!m[i]) continue;
      if (i == 0 || !m[i - 1]) out->push_back(Entry{b, pos, 0, static_cast<int32_t>(i), 0, 0});
      ++out->back().count;
      ++pos;
    }
    (*count)[b] = pos - c[b];
    if (out->size() == first) out->push_back(Entry{b, c[b], 0, 0, 0, 0});
    // padding before run k (after run k-1) belongs to entry k; the last entry also takes the tail
    for (size_t k = first; k < out->size(); ++k) {
      Entry& e = (*out)[k];
      e.zlo = k == first ? 0 : (*out)[k - 1].row0 + (*out)[k - 1].count;
      e.zhi = k + 1 == out->size() ? static_cast<int32_t>(n) : e.row0 + e.count;
    }
  }
  return GQA_OK;
}

// Every entry's positions must be its start, start + 1, ...
gqa_status check_positions(const std::vector<Entry>& es, const int32_t* positions, int64_t n, const char* what) {
  for (const Entry& e : es) {
    const int32_t* p = positions + static_cast<int64_t>(e.b) * n + e.row0;
    for (int i = 0; i < e.count; ++i)
      if (p[i] != e.start + i) return fail(GQA_ERR_POSITION, what);
  }
  return GQA_OK;
}

struct AppendPlan {
  int64_t n = 0;
  std::vector<int32_t> count, start, need;  // per batch row: valid tokens, first position, new pages
  std::vector<uint8_t> cow;                 // the row's first write lands in a shared page: copy it first
  std::vector<Entry> entries;
};

// Every check of an append (mask, positions, capacity, page budget).
gqa_status plan_append(const gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* K,
                       const gqa_tensor* V, const uint8_t* mask, const int32_t* positions, AppendPlan* plan) {
  const gqa_cache_config& cf = c->cfg;
  if (!K || !V) return fail(GQA_ERR_ARG, "K or V is null");
  const int64_t n = K->shape[2];
  if (n < 0) return fail(GQA_ERR_SHAPE, "negative token count");
  gqa_status st = check_tensor(K, "K", cf.dtype, B, cf.num_kv_heads, n, cf.head_dim);
  if (st != GQA_OK) return st;
  st = check_tensor(V, "V", cf.dtype, B, cf.num_kv_heads, n, cf.head_dim);
  if (st != GQA_OK) return st;
  if (B > 0 && n > 0 && (!mask || !positions)) return fail(GQA_ERR_ARG, "mask or positions is null");
  plan->n = n;
  plan->start.assign(B, 0);
  plan->need.assign(B, 0);
  plan->cow.assign(B, 0);
  for (int b = 0; b < B; ++b) plan->start[b] = c->len[static_cast<int64_t>(seq_ids[b]) * cf.num_layers + layer];
  if (n > 0) {
    st = mask_entries(mask, n, B, plan->start.data(), &plan->entries, &plan->count);
    if (st != GQA_OK) return st;
    st = check_positions(plan->entries, positions, n, "positions must continue the cache: c_b, c_b+1, ...");
    if (st != GQA_OK) return st;
  } else {
    plan->count.assign(B, 0);
    plan->entries.clear();
  }
  for (int b = 0; b < B; ++b) {
    const int32_t c0 = plan->start[b];
    const int64_t end = static_cast<int64_t>(c0) + plan->count[b];
    if (cf.rope_style == 1 && end > cf.max_position) return fail(GQA_ERR_POSITION, "position beyond max_position");
    if (cf.window) {
      // every position the call's queries read, and its writes, at once in the ring
      const int64_t first = std::max<int64_t>(0, c0 - cf.window + 1);
      if (plan->count[b] && (end - 1) / kPage - first / kPage + 1 > cf.max_pages_per_seq)
        return fail(GQA_ERR_OUT_OF_PAGES, "the window and the new tokens exceed the ring");
    } else if (ceil_div(end, kPage) > cf.max_pages_per_seq) {
      return fail(GQA_ERR_OUT_OF_PAGES, "sequence exceeds its block-table capacity");
    }
  }
  int64_t total_need = 0;
  std::vector<int32_t> released;            // shared pages that earlier rows of this call copy away from
  for (int b = 0; b < B; ++b) {
    const int s = seq_ids[b];
    const int32_t c0 = plan->start[b];
    if (!cf.window && plan->count[b] > 0 && c0 % kPage != 0) {
      const int32_t page = c->pages[s][c0 / kPage];
      const int32_t refs = c->ref[page] - static_cast<int32_t>(std::count(released.begin(), released.end(), page));
      if (refs > 1) {
        plan->cow[b] = 1;
        released.push_back(page);
        ++total_need;
      }
    }
    const int64_t end = static_cast<int64_t>(c0) + plan->count[b];
    const int64_t have = static_cast<int64_t>(c->pages[s].size());
    plan->need[b] = static_cast<int32_t>(std::max<int64_t>(0, table_entries(cf, end) - have));
    total_need += plan->need[b];
  }
  if (total_need > static_cast<int64_t>(c->free_list.size())) return fail(GQA_ERR_OUT_OF_PAGES, "not enough free pages");
  return GQA_OK;
}

void commit_append(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const AppendPlan& plan) {
  const gqa_cache_config& cf = c->cfg;
  for (int b = 0; b < B; ++b) {
    const int s = seq_ids[b];
    if (plan.cow[b]) {
      const int32_t lp = plan.start[b] / kPage;
      const int32_t old = c->pages[s][lp];
      const int32_t page = c->free_list.front();
      c->free_list.pop_front();
      c->copies.emplace_back(old, page);
      --c->ref[old];
      c->ref[page] = 1;
      c->pages[s][lp] = page;
      c->pending.emplace_back(s * cf.max_pages_per_seq + lp, page);
    }
    for (int k = 0; k < plan.need[b]; ++k) {
      const int32_t page = c->free_list.front();
      c->free_list.pop_front();
      const int32_t lp = static_cast<int32_t>(c->pages[s].size());
      c->pages[s].push_back(page);
      c->ref[page] = 1;
      c->pending.emplace_back(s * cf.max_pages_per_seq + lp, page);
    }
  }
  for (int b = 0; b < B; ++b)
    c->len[static_cast<int64_t>(seq_ids[b]) * cf.num_layers + layer] = plan.start[b] + plan.count[b];
}

gqa_status hip_fail(hipError_t e, const char* what) {
  return fail(GQA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

gqa_status launch_copies(gqa_cache* c, const std::vector<std::pair<int32_t, int32_t>>& copies, hipStream_t s) {
  for (size_t i0 = 0; i0 < copies.size(); i0 += gqa::kMaxCopiesPerLaunch) {
    gqa::CopyArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k_pool = c->k_pool;
    a.v_pool = c->v_pool;
    a.layer_stride = c->layer_elems;
    a.page_elems = c->page_elems;
    a.elt_bytes = c->elt;
    a.n = static_cast<int32_t>(std::min<size_t>(copies.size() - i0, gqa::kMaxCopiesPerLaunch));
    for (int j = 0; j < a.n; ++j) {
      a.src[j] = copies[i0 + j].first;
      a.dst[j] = copies[i0 + j].second;
    }
    hipError_t e = gqa::launch_page_copy(a, c->cfg.num_layers, s);
    if (e != hipSuccess) return hip_fail(e, "page copy launch");
  }
  return GQA_OK;
}

// Upload the rotation table once, make pending copy-on-write page copies and
// write pending block-table entries.
gqa_status sync_metadata(gqa_cache* c, hipStream_t s) {
  if (c->cfg.rope_style == 1 && !c->rope_uploaded) {
    hipError_t e = hipMemcpyAsync(c->d_rope, c->rope_host.data(), c->rope_host.size() * sizeof(float),
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "rotation table upload");
    c->rope_uploaded = true;
  }
  if (!c->copies.empty()) {
    gqa_status st = launch_copies(c, c->copies, s);
    if (st != GQA_OK) return st;
    c->copies.clear();
  }
  // one write per table entry, the last one queued (a fork's entry may be
  // replaced by its copy in the same call, and a patch launch writes its
  // entries in parallel)
  if (c->pending.size() > 1) {
    std::vector<std::pair<int32_t, int32_t>> last;
    last.reserve(c->pending.size());
    std::vector<std::pair<int32_t, int32_t>> sorted(c->pending);
    std::stable_sort(sorted.begin(), sorted.end(),
                     [](const std::pair<int32_t, int32_t>& x, const std::pair<int32_t, int32_t>& y) {
                       return x.first < y.first;
                     });
    for (size_t k = 0; k < sorted.size(); ++k)
      if (k + 1 == sorted.size() || sorted[k + 1].first != sorted[k].first) last.push_back(sorted[k]);
    c->pending.swap(last);
  }
  size_t i = 0;
  while (i < c->pending.size()) {
    gqa::PatchArgs pa;
    pa.table = c->d_table;
    pa.n = 0;
    pa.base = c->pending[i].first;        // entries are in ascending index order
    for (; i < c->pending.size() && pa.n < gqa::kMaxPatchPerLaunch && c->pending[i].first - pa.base < 65536;
         ++i, ++pa.n) {
      pa.offset[pa.n] = static_cast<uint16_t>(c->pending[i].first - pa.base);
      pa.value[pa.n] = c->pending[i].second;
    }
    hipError_t e = gqa::launch_table_patch(pa, s);
    if (e != hipSuccess) return hip_fail(e, "block-table patch");
  }
  c->pending.clear();
  return GQA_OK;
}

template <typename T>
T* layer_base(void* pool, const gqa_cache* c, int layer) {
  return static_cast<T*>(pool) + static_cast<int64_t>(layer) * c->layer_elems;
}

gqa_status launch_append_all(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* K,
                             const gqa_tensor* V, const AppendPlan& plan, hipStream_t s) {
  const gqa_cache_config& cf = c->cfg;
  (void)B;
  std::vector<Entry> es;
  for (const Entry& e : plan.entries)
    if (e.count > 0) es.push_back(e);
  const int E = static_cast<int>(es.size());
  for (int e0 = 0; e0 < E; e0 += kMaxSeqPerLaunch) {
    const int nb = std::min(E - e0, kMaxSeqPerLaunch);
    gqa::AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    a.K = K->data;
    a.V = V->data;
    a.k_s0 = K->stride[0]; a.k_s1 = K->stride[1]; a.k_s2 = K->stride[2];
    a.v_s0 = V->stride[0]; a.v_s1 = V->stride[1]; a.v_s2 = V->stride[2];
    a.k_pool = static_cast<char*>(c->k_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.v_pool = static_cast<char*>(c->v_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.table = c->d_table;
    a.table_w = cf.max_pages_per_seq;
    a.window = cf.window;
    a.Hkv = cf.num_kv_heads;
    a.d = cf.head_dim;
    a.nseq = nb;
    a.rope = cf.rope_style == 1 ? c->d_rope : nullptr;
    int grid_x = 0;
    for (int j = 0; j < nb; ++j) {
      const Entry& e = es[e0 + j];
      a.meta.seq[j] = seq_ids[e.b];
      a.meta.brow[j] = e.b;
      a.meta.start[j] = e.start;
      a.meta.count[j] = e.count;
      a.meta.row0[j] = e.row0;
      a.meta.total[j] = e.start + e.count;
      const int first = e.start / kPage;
      const int last = (e.start + e.count - 1) / kPage;
      grid_x = std::max(grid_x, last - first + 1);
    }
    if (grid_x == 0) continue;
    hipError_t e = gqa::launch_append(a, cf.dtype, grid_x, s);
    if (e != hipSuccess) return hip_fail(e, "cache write launch");
  }
  return GQA_OK;
}


// Short query runs (at most GQA_MAX_CHUNK_TOKENS rectangular rows) of a bf16
// cache go to the split-T kernel when the caller passes a workspace and every
// row's valid tokens are one run (each run would read its whole prefix again).
bool use_split(const gqa_cache* c, int64_t n, const void* workspace, int32_t B, const std::vector<Entry>& es) {
  return c->cfg.dtype == GQA_BF16 && n >= 1 && n <= GQA_MAX_CHUNK_TOKENS && workspace != nullptr &&
         static_cast<int64_t>(es.size()) == B;
}
gqa_status check_split_workspace(const gqa_cache* c, int32_t B, int64_t Hq, int64_t n, const std::vector<Entry>& es,
                                 void* workspace, size_t ws_bytes);
gqa_status attend_split(gqa_cache* c, int32_t layer, const int32_t* seq_ids, const gqa_tensor* Q, const gqa_tensor* O,
                        int64_t n, const std::vector<Entry>& es, void* workspace, size_t ws_bytes, hipStream_t s);

// Causal attention of every entry's queries (positions start.., count of them,
// from rectangular row row0 of batch row b) against slots [0, position] of the
// layer; total[b] = written length of the sequence in that layer.
gqa_status launch_attention(gqa_cache* c, int32_t layer, const int32_t* seq_ids, const gqa_tensor* Q,
                            const gqa_tensor* O, int64_t n, const std::vector<Entry>& es, const int32_t* total,
                            hipStream_t s) {
  const gqa_cache_config& cf = c->cfg;
  const int64_t Hq = Q->shape[1];
  const int E = static_cast<int>(es.size());
  for (int e0 = 0, nb = 0; e0 < E; e0 += nb) {
    // as many entries as fit one launch's entry and batch-row tables
    int rows = 0;
    for (nb = 0; e0 + nb < E && nb < gqa::kMaxRunsPerLaunch; ++nb) {
      const bool new_row = nb == 0 || es[e0 + nb].b != es[e0 + nb - 1].b;
      if (new_row && rows == gqa::kMaxRowsPerLaunch) break;
      rows += new_row;
    }
    gqa::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.Q = Q->data;
    a.q_s0 = Q->stride[0]; a.q_s1 = Q->stride[1]; a.q_s2 = Q->stride[2];
    a.O = O->data;
    a.o_s0 = O->stride[0]; a.o_s1 = O->stride[1]; a.o_s2 = O->stride[2];
    a.k_pool = static_cast<char*>(c->k_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.v_pool = static_cast<char*>(c->v_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.table = c->d_table;
    a.table_w = cf.max_pages_per_seq;
    a.window = cf.window;
    a.Hq = static_cast<int32_t>(Hq);
    a.Hkv = cf.num_kv_heads;
    a.d = cf.head_dim;
    a.n_rect = static_cast<int32_t>(n);
    a.nseq = nb;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(cf.head_dim)));
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(cf.head_dim)));
    a.pool_bytes = static_cast<uint32_t>(c->layer_elems * c->elt);
    a.rope = cf.rope_style == 1 ? c->d_rope : nullptr;
    a.rope_t = cf.rope_style == 1 ? c->d_rope + static_cast<int64_t>(cf.max_position) * cf.head_dim : nullptr;
    a.rope_rows = cf.max_position;
    int rw = -1;
    for (int j = 0; j < nb; ++j) {
      const Entry& e = es[e0 + j];
      if (j == 0 || e.b != es[e0 + j - 1].b) {
        ++rw;
        a.meta.seq[rw] = seq_ids[e.b];
        a.meta.brow[rw] = e.b;
        a.meta.total[rw] = total[e.b];
      }
      a.meta.row[j] = static_cast<uint8_t>(rw);
      a.meta.start[j] = e.start;
      a.meta.count[j] = e.count;
      a.meta.row0[j] = e.row0;
      a.meta.zlo[j] = e.zlo;
      a.meta.zhi[j] = e.zhi;
    }
    hipError_t e = cf.dtype == GQA_BF16 ? gqa::launch_prefill_bf16(a, s) : gqa::launch_attend_f32(a, s);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
  }
  return GQA_OK;
}

}  // namespace

// ------------------------------------------------------------------ lifecycle

GQA_EXPORT gqa_status gqa_cache_buffer_sizes(const gqa_cache_config* cfg, size_t* k_pool_bytes, size_t* v_pool_bytes,
                                             size_t* page_table_bytes, size_t* rope_table_bytes) {
  gqa_status st = check_config(cfg);
  if (st != GQA_OK) return st;
  const size_t elt = cfg->dtype == GQA_BF16 ? 2 : 4;
  const size_t pool = static_cast<size_t>(cfg->num_layers) * cfg->num_pages * cfg->num_kv_heads * kPage *
                      cfg->head_dim * elt;
  if (k_pool_bytes) *k_pool_bytes = pool;
  if (v_pool_bytes) *v_pool_bytes = pool;
  if (page_table_bytes) *page_table_bytes = static_cast<size_t>(cfg->max_seqs) * cfg->max_pages_per_seq * 4;
  if (rope_table_bytes)   // the rows, then the same values grouped by 16-byte chunk
    *rope_table_bytes = cfg->rope_style == 1 ? 2 * static_cast<size_t>(cfg->max_position) * cfg->head_dim * 4 : 0;
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_cache_create(const gqa_cache_config* cfg, void* k_pool, void* v_pool, int32_t* page_table,
                                       void* rope_table, const int32_t* free_list_order, gqa_cache** out) {
  gqa_status st = check_config(cfg);
  if (st != GQA_OK) return st;
  if (!out) return fail(GQA_ERR_ARG, "out is null");
  if (!k_pool || !v_pool || !page_table) return fail(GQA_ERR_ARG, "pool or page-table pointer is null");
  if (cfg->rope_style == 1 && !rope_table) return fail(GQA_ERR_ARG, "rope_table is null");
  if (reinterpret_cast<uintptr_t>(k_pool) % 16 || reinterpret_cast<uintptr_t>(v_pool) % 16)
    return fail(GQA_ERR_ARG, "pools must be 16-byte aligned");
  std::vector<int32_t> order(cfg->num_pages);
  if (free_list_order) {
    std::vector<char> seen(cfg->num_pages, 0);
    for (int i = 0; i < cfg->num_pages; ++i) {
      const int32_t p = free_list_order[i];
      if (p < 0 || p >= cfg->num_pages || seen[p]) return fail(GQA_ERR_ARG, "free_list_order is not a permutation");
      seen[p] = 1;
      order[i] = p;
    }
  } else {
    for (int i = 0; i < cfg->num_pages; ++i) order[i] = i;
  }
  gqa_cache* c = new (std::nothrow) gqa_cache();
  if (!c) return fail(GQA_ERR_ARG, "out of host memory");
  c->cfg = *cfg;
  c->k_pool = k_pool;
  c->v_pool = v_pool;
  c->d_table = page_table;
  c->d_rope = static_cast<float*>(rope_table);
  c->free_list.assign(order.begin(), order.end());
  c->ref.assign(cfg->num_pages, 0);
  c->pages.assign(cfg->max_seqs, {});
  c->len.assign(static_cast<size_t>(cfg->max_seqs) * cfg->num_layers, 0);
  c->elt = cfg->dtype == GQA_BF16 ? 2 : 4;
  c->page_elems = static_cast<int64_t>(cfg->num_kv_heads) * kPage * cfg->head_dim;
  c->layer_elems = static_cast<int64_t>(cfg->num_pages) * c->page_elems;
  if (cfg->rope_style == 1) {
    // pair i turns by p * theta^(-2i/d): frequency and angle in double, cos and
    // sin from the C library, rounded once to float32
    const int half = cfg->head_dim / 2;
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(cfg->rope_theta, -2.0 * i / cfg->head_dim);
    const int64_t rows = cfg->max_position, d = cfg->head_dim;
    c->rope_host.resize(static_cast<size_t>(2 * rows * d));
    for (int64_t p = 0; p < rows; ++p)
      for (int i = 0; i < half; ++i) {
        const double ang = static_cast<double>(p) * inv[i];
        c->rope_host[(p * half + i) * 2] = static_cast<float>(std::cos(ang));
        c->rope_host[(p * half + i) * 2 + 1] = static_cast<float>(std::sin(ang));
      }
    // second copy, chunk-major: 16-byte chunk j of row p at [j][p], so that
    // consecutive positions of one chunk are adjacent in memory (the prefill
    // kernel reads one chunk of 32 consecutive positions per instruction)
    float* tr = c->rope_host.data() + rows * d;
    for (int64_t j = 0; j < d / 4; ++j)
      for (int64_t p = 0; p < rows; ++p)
        for (int e = 0; e < 4; ++e) tr[(j * rows + p) * 4 + e] = c->rope_host[p * d + j * 4 + e];
  }
  *out = c;
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_cache_destroy(gqa_cache* cache) {
  delete cache;
  return GQA_OK;
}

// ------------------------------------------------------------------ append / prefill

GQA_EXPORT gqa_status kv_cache_append(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                      const gqa_tensor* K, const gqa_tensor* V, const uint8_t* valid_mask,
                                      const int32_t* positions, void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  if (layer < 0 || layer >= c->cfg.num_layers) return fail(GQA_ERR_ARG, "layer out of range");
  gqa_status st = check_seqs(c, B, seq_ids);
  if (st != GQA_OK) return st;
  AppendPlan plan;
  st = plan_append(c, layer, B, seq_ids, K, V, valid_mask, positions, &plan);
  if (st != GQA_OK) return st;
  commit_append(c, layer, B, seq_ids, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sync_metadata(c, s);
  if (st != GQA_OK) return st;
  return launch_append_all(c, layer, B, seq_ids, K, V, plan, s);
}

GQA_EXPORT gqa_status gqa_prefill(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                  const gqa_tensor* Q, const gqa_tensor* K, const gqa_tensor* V,
                                  const uint8_t* valid_mask, const int32_t* positions, const gqa_tensor* O,
                                  void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.num_layers) return fail(GQA_ERR_ARG, "layer out of range");
  gqa_status st = check_seqs(c, B, seq_ids);
  if (st != GQA_OK) return st;
  if (!Q || !O || !K) return fail(GQA_ERR_ARG, "Q, K or O is null");
  const int64_t n = K->shape[2];
  const int64_t Hq = Q->shape[1];
  if (Hq < 1 || Hq % cf.num_kv_heads) return fail(GQA_ERR_SHAPE, "Hkv must divide Hq");
  st = check_tensor(Q, "Q", cf.dtype, B, Hq, n, cf.head_dim);
  if (st != GQA_OK) return st;
  st = check_tensor(O, "O", cf.dtype, B, Hq, n, cf.head_dim);
  if (st != GQA_OK) return st;
  AppendPlan plan;
  st = plan_append(c, layer, B, seq_ids, K, V, valid_mask, positions, &plan);
  if (st != GQA_OK) return st;
  const bool split = use_split(c, n, workspace, B, plan.entries);
  if (split) {
    st = check_split_workspace(c, B, Hq, n, plan.entries, workspace, ws_bytes);
    if (st != GQA_OK) return st;
  }
  commit_append(c, layer, B, seq_ids, plan);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sync_metadata(c, s);
  if (st != GQA_OK) return st;
  st = launch_append_all(c, layer, B, seq_ids, K, V, plan, s);
  if (st != GQA_OK) return st;
  if (n == 0) return GQA_OK;
  if (split) return attend_split(c, layer, seq_ids, Q, O, n, plan.entries, workspace, ws_bytes, s);
  std::vector<int32_t> totals(B);
  for (int b = 0; b < B; ++b) totals[b] = plan.start[b] + plan.count[b];
  return launch_attention(c, layer, seq_ids, Q, O, n, plan.entries, totals.data(), s);
}

GQA_EXPORT gqa_status gqa_attention(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                    const gqa_tensor* Q, const uint8_t* valid_mask, const int32_t* positions,
                                    const gqa_tensor* O, void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.num_layers) return fail(GQA_ERR_ARG, "layer out of range");
  gqa_status st = check_seqs(c, B, seq_ids);
  if (st != GQA_OK) return st;
  if (!Q || !O) return fail(GQA_ERR_ARG, "Q or O is null");
  const int64_t n = Q->shape[2];
  const int64_t Hq = Q->shape[1];
  if (n < 0) return fail(GQA_ERR_SHAPE, "negative token count");
  if (Hq < 1 || Hq % cf.num_kv_heads) return fail(GQA_ERR_SHAPE, "Hkv must divide Hq");
  st = check_tensor(Q, "Q", cf.dtype, B, Hq, n, cf.head_dim);
  if (st != GQA_OK) return st;
  st = check_tensor(O, "O", cf.dtype, B, Hq, n, cf.head_dim);
  if (st != GQA_OK) return st;
  if (B > 0 && n > 0 && (!valid_mask || !positions)) return fail(GQA_ERR_ARG, "mask or positions is null");
  // the first valid token of each row fixes the row's positions: start, start + 1, ...
  std::vector<int32_t> start(B, 0), count, totals(B);
  std::vector<Entry> es;
  if (n > 0) {
    for (int b = 0; b < B; ++b) {
      const uint8_t* m = valid_mask + static_cast<int64_t>(b) * n;
      for (int64_t i = 0; i < n; ++i)
        if (m[i] == 1) {
          start[b] = positions[static_cast<int64_t>(b) * n + i];
          break;
        }
    }
    st = mask_entries(valid_mask, n, B, start.data(), &es, &count);
    if (st != GQA_OK) return st;
    st = check_positions(es, positions, n, "query positions must be consecutive");
    if (st != GQA_OK) return st;
  } else {
    count.assign(B, 0);
  }
  for (int b = 0; b < B; ++b) {
    const int32_t have = c->len[static_cast<int64_t>(seq_ids[b]) * cf.num_layers + layer];
    if (count[b] && (start[b] < 0 || static_cast<int64_t>(start[b]) + count[b] > have))
      return fail(GQA_ERR_POSITION, "query positions must lie inside the cached length");
    if (count[b] && std::max(0, start[b] - cf.window + 1) < resident_from(cf, have))
      return fail(GQA_ERR_POSITION, "the window of a query reaches positions the ring no longer holds");
    totals[b] = have;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_split(c, n, workspace, B, es)) {
    st = check_split_workspace(c, B, Hq, n, es, workspace, ws_bytes);
    if (st != GQA_OK) return st;
    return attend_split(c, layer, seq_ids, Q, O, n, es, workspace, ws_bytes, s);
  }
  st = sync_metadata(c, s);
  if (st != GQA_OK) return st;
  if (n == 0) return GQA_OK;
  return launch_attention(c, layer, seq_ids, Q, O, n, es, totals.data(), s);
}

// ------------------------------------------------------------------ decode

namespace {

// Workspace of the split-T kernel: a 256-byte header whose first word is the
// sticky failure status, then slots of one (split, kv head x column chunk)
// each: a ready-flag row of kDecodeMergers int32, 16 split o rows of d float32
// and 16 (m, l) headers.  The cut depends only on the workspace's size and d,
// never on a call's shape, so calls of any B, Hq or chunk length can share one
// workspace: the flags sit first and every call leaves them zero.
constexpr int64_t kWsHeader = 256;

struct WsView {
  int32_t* status = nullptr;
  int32_t* flags = nullptr;
  float* part_o = nullptr;
  float* part_h = nullptr;
  int64_t slots = 0;
  int64_t zero_bytes = 0;    // header + flags: what a reset clears
};

int64_t ws_slot_bytes(int64_t d) { return (16 * d + 16 * 2 + gqa::kDecodeMergers) * 4; }

// count_d: head dimension the slot count is taken for (d itself for a caller's
// workspace; the largest, 128, for the static scratch, whose flags must sit at
// the same place for caches of any d)
int64_t ws_slots(size_t bytes, int64_t count_d) {
  // the header and the 256-byte rounding of the flags fit in 2 * kWsHeader
  return bytes < static_cast<size_t>(2 * kWsHeader)
             ? 0 : static_cast<int64_t>((bytes - 2 * kWsHeader) / ws_slot_bytes(count_d));
}

// bytes of the header and the ready flags of `slots` slots
int64_t ws_zero_bytes(int64_t slots) { return kWsHeader + ceil_div(slots * gqa::kDecodeMergers * 4, 256) * 256; }

WsView ws_view(void* ws, size_t bytes, int64_t d, int64_t count_d = 0) {
  WsView v;
  if (!ws) return v;
  v.slots = ws_slots(bytes, count_d ? count_d : d);
  if (!v.slots) return v;
  v.status = static_cast<int32_t*>(ws);
  v.flags = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kWsHeader);
  v.zero_bytes = ws_zero_bytes(v.slots);
  v.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + v.zero_bytes);
  v.part_h = v.part_o + v.slots * 16 * d;
  return v;
}

// Ready-flag values: every launch takes a fresh nonzero epoch (a flag left by
// a launch whose merge gave up never equals a later launch's).  The merge wait
// and a test control that makes it give up are process-wide.
std::atomic<uint32_t> g_epoch{0};
std::atomic<int32_t> g_spin_limit{1 << 18};
std::atomic<int32_t> g_unreachable{0};

int32_t next_epoch() { return static_cast<int32_t>(g_epoch.fetch_add(1) % 0x3fffffffu) + 1; }

// (kv head x column chunk) rows of the grid for ncol (token, head) columns
int64_t split_ys(const gqa_cache* c, int64_t ncol) { return c->cfg.num_kv_heads * ceil_div(ncol, 16); }

// Workgroups of the split-T kernel the device holds at once: two per compute
// unit (its launch bounds), read once per process from the current device.
int64_t decode_resident_workgroups() {
  static std::atomic<int> cus{0};
  int n = cus.load();
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus.store(n);
  }
  return 2 * static_cast<int64_t>(n);
}

// Pages per split: enough workgroups to fill the chip (about the target count),
// at least kDecodeMinPages pages each, at most kMaxSplitDecode splits per
// sequence (the in-kernel combine stages one weight per split in LDS).  A grid
// a little larger than the workgroups the device holds at once would run a
// short second round, and each sequence's combine waits for its last split:
// when longer splits (under twice as long) fit the grid in one round, take them.
int decode_pages_per_split(const int32_t* T, int B, int64_t ys) {
  int64_t total_pages = 0, max_pages = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t p = ceil_div(T[b], kPage);
    total_pages += p;
    max_pages = std::max(max_pages, p);
  }
  int64_t pps = std::max<int64_t>(kDecodeMinPages, ceil_div(total_pages * ys, kDecodeTargetBlocks));
  pps = std::max<int64_t>(pps, ceil_div(max_pages, gqa::kMaxSplitDecode));
  auto grid = [&](int64_t p) {
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += std::max<int64_t>(1, ceil_div(ceil_div(T[b], kPage), p));
    return n * ys;
  };
  const int64_t resident = decode_resident_workgroups();
  const int64_t n0 = grid(pps);
  if (n0 > resident && n0 <= 2 * resident) {
    for (int64_t p = pps + 1; p < 2 * pps; ++p)
      if (grid(p) <= resident) {
        pps = p;
        break;
      }
  }
  return static_cast<int>(pps);
}

// Keys a split-T entry reads, counted from the first page it reads: with a
// window, the pages wholly before its first query's window are skipped.
int32_t read_length(const gqa_cache* c, int32_t start, int32_t count) {
  if (count == 0) return 0;
  const int32_t T = start + count;
  if (!c->cfg.window) return T;
  return T - (std::max(0, start - c->cfg.window + 1) / kPage) * kPage;
}

// Splits of an entry that reads T keys (one at least, so that a sequence with
// no query still gets the workgroup that zeroes its padding rows).
int64_t split_count(int32_t T, int pps) { return std::max<int64_t>(1, ceil_div(ceil_div(T, kPage), pps)); }

// Workspace bytes that suffice for B sequences at ys grid rows, whatever the
// lengths: pps >= ceil(total_pages * ys / target), so the splits number at
// most ceil(target / ys) + B.
size_t ws_bytes_for(const gqa_cache* c, int64_t B, int64_t ys) {
  const int64_t slots = (ceil_div(kDecodeTargetBlocks, ys) + B) * ys;
  return static_cast<size_t>(2 * kWsHeader + slots * ws_slot_bytes(c->cfg.head_dim));
}

// Split-T attention over the paged cache for short query runs (one launch per
// kMaxSeqPerLaunch sequences): the count[b] queries of sequence b, at positions
// start[b].. in rectangular rows row0[b].., attend to keys 0..position of their
// own; rows of o outside the run are zeroed.  ncol = (longest run) x (Hq/Hkv).
// Decode is the run of one query at T-1; with k_new/v_new the launch also
// writes that token (bf16 only).  Checks (shapes, workspace) are the caller's.
gqa_status launch_split(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* q,
                        const gqa_tensor* o, const int32_t* start, const int32_t* count, const int32_t* row0,
                        int n_rect, int ncol, const gqa_tensor* k_new, const gqa_tensor* v_new, void* workspace,
                        size_t ws_bytes, hipStream_t s, int64_t count_d = 0) {
  const gqa_cache_config& cf = c->cfg;
  const int64_t Hq = q->shape[1];
  const int64_t ys = split_ys(c, ncol);
  std::vector<int32_t> T(B), Tr(B);
  for (int b = 0; b < B; ++b) {
    T[b] = start[b] + count[b];
    Tr[b] = read_length(c, start[b], count[b]);
  }
  const int pps = decode_pages_per_split(Tr.data(), B, ys);
  const WsView wv = ws_view(workspace, ws_bytes, cf.head_dim, count_d);
  // A decode step that opens a page for its new token: when that is all the
  // block table waits for (nothing else pending, one launch), the decode
  // launch takes the page from its arguments and writes the entry itself, so
  // the step needs no block-table patch launch before it.
  std::vector<int32_t> new_page(B, -1);
  std::vector<std::pair<int32_t, int32_t>> fused;   // the entries the launch writes (restored if it fails)
  if (k_new && B <= gqa::kMaxSeqPerLaunch && c->copies.empty() && !c->pending.empty()) {
    bool all = true;
    for (const auto& pe : c->pending) {
      int hit = -1;
      for (int b = 0; b < B && hit < 0; ++b) {
        const int32_t pn = (T[b] - 1) / kPage;
        const int32_t e = cf.window ? pn % cf.max_pages_per_seq : pn;
        if (pe.first == seq_ids[b] * cf.max_pages_per_seq + e) hit = b;
      }
      if (hit < 0) {
        all = false;
        break;
      }
      new_page[hit] = pe.second;
    }
    if (all) fused.swap(c->pending);
    else std::fill(new_page.begin(), new_page.end(), -1);
  }
  gqa_status st = sync_metadata(c, s);
  if (st != GQA_OK) {
    c->pending.insert(c->pending.end(), fused.begin(), fused.end());
    return st;
  }
  int64_t split_base = 0;
  for (int b0 = 0; b0 < B; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(B - b0, kMaxSeqPerLaunch);
    gqa::DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q->data;
    a.q_s0 = q->stride[0]; a.q_s1 = q->stride[1]; a.q_s2 = q->stride[2];
    a.o = o->data;
    a.o_s0 = o->stride[0]; a.o_s1 = o->stride[1]; a.o_s2 = o->stride[2];
    if (k_new) {
      a.k_new = k_new->data;
      a.kn_s0 = k_new->stride[0]; a.kn_s1 = k_new->stride[1];
      a.v_new = v_new->data;
      a.vn_s0 = v_new->stride[0]; a.vn_s1 = v_new->stride[1];
    }
    a.k_pool = static_cast<char*>(c->k_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.v_pool = static_cast<char*>(c->v_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.table = c->d_table;
    a.table_w = cf.max_pages_per_seq;
    a.window = cf.window;
    a.Hq = static_cast<int32_t>(Hq);
    a.Hkv = cf.num_kv_heads;
    a.d = cf.head_dim;
    a.nseq = nb;
    a.ncol = ncol;
    a.n_rect = n_rect;
    a.pages_per_split = pps;
    a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(cf.head_dim)));
    a.rope = cf.rope_style == 1 ? c->d_rope : nullptr;
    if (wv.slots) {
      a.part_o = wv.part_o + split_base * ys * 16 * cf.head_dim;
      a.part_h = wv.part_h + split_base * ys * 16 * 2;
      a.flags = wv.flags + split_base * ys * gqa::kDecodeMergers;
      a.status = wv.status;
    }
    a.epoch = next_epoch();
    a.wait_value = g_unreachable.load() ? (a.epoch ^ 0x40000000) : a.epoch;
    a.spin_limit = g_spin_limit.load();
    int32_t off = 0;
    for (int j = 0; j < nb; ++j) {
      const int b = b0 + j;
      a.meta.seq[j] = seq_ids[b];
      a.meta.brow[j] = b;
      a.meta.start[j] = start[b];
      a.meta.count[j] = count[b];
      a.meta.row0[j] = row0[b];
      a.meta.total[j] = T[b];
      a.meta.zlo[j] = 0;
      a.meta.zhi[j] = n_rect;
      a.split_off[j] = off;
      a.new_page[j] = new_page[b];
      off += static_cast<int>(split_count(Tr[b], pps));
    }
    a.split_off[nb] = off;
    hipError_t e = gqa::launch_decode_bf16(a, off, s);
    if (e != hipSuccess) {
      c->pending.insert(c->pending.end(), fused.begin(), fused.end());
      return hip_fail(e, "split attention launch");
    }
    split_base += off;
  }
  return GQA_OK;
}

gqa_status launch_decode(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* q,
                         const gqa_tensor* o, const int32_t* T, const gqa_tensor* k_new, const gqa_tensor* v_new,
                         void* workspace, size_t ws_bytes, hipStream_t s, int64_t count_d = 0) {
  std::vector<int32_t> start(B), count(B, 1), row0(B, 0);
  for (int b = 0; b < B; ++b) start[b] = T[b] - 1;
  const int G = static_cast<int>(q->shape[1] / c->cfg.num_kv_heads);
  return launch_split(c, layer, B, seq_ids, q, o, start.data(), count.data(), row0.data(), 1, G, k_new, v_new,
                      workspace, ws_bytes, s, count_d);
}

gqa_status launch_decode_f32(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* q,
                             const gqa_tensor* o, const int32_t* T, hipStream_t s) {
  const gqa_cache_config& cf = c->cfg;
  gqa_status st = sync_metadata(c, s);
  if (st != GQA_OK) return st;
  for (int b0 = 0; b0 < B; b0 += gqa::kMaxRowsPerLaunch) {
    const int nb = std::min(B - b0, gqa::kMaxRowsPerLaunch);   // one entry per batch row
    gqa::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.Q = static_cast<const char*>(q->data) + b0 * q->stride[0] * c->elt;
    a.q_s0 = q->stride[0]; a.q_s1 = q->stride[1]; a.q_s2 = q->stride[2];
    a.O = static_cast<char*>(o->data) + b0 * o->stride[0] * c->elt;
    a.o_s0 = o->stride[0]; a.o_s1 = o->stride[1]; a.o_s2 = o->stride[2];
    a.k_pool = static_cast<char*>(c->k_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.v_pool = static_cast<char*>(c->v_pool) + static_cast<int64_t>(layer) * c->layer_elems * c->elt;
    a.table = c->d_table;
    a.table_w = cf.max_pages_per_seq;
    a.window = cf.window;
    a.Hq = static_cast<int32_t>(q->shape[1]);
    a.Hkv = cf.num_kv_heads;
    a.d = cf.head_dim;
    a.n_rect = 1;
    a.nseq = nb;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(cf.head_dim)));
    a.rope = cf.rope_style == 1 ? c->d_rope : nullptr;
    a.rope_t = cf.rope_style == 1 ? c->d_rope + static_cast<int64_t>(cf.max_position) * cf.head_dim : nullptr;
    a.rope_rows = cf.max_position;
    for (int j = 0; j < nb; ++j) {
      a.meta.row[j] = static_cast<uint8_t>(j);
      a.meta.seq[j] = seq_ids[b0 + j];
      a.meta.brow[j] = j;
      a.meta.start[j] = T[b0 + j] - 1;
      a.meta.count[j] = 1;
      a.meta.row0[j] = 0;
      a.meta.total[j] = T[b0 + j];
      a.meta.zlo[j] = 0;
      a.meta.zhi[j] = 1;
    }
    hipError_t e = gqa::launch_attend_f32(a, s);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  return GQA_OK;
}

// q/o checks shared by gqa_decode and gqa_decode_step; the workspace check
// needs the lengths the call will attend over.
gqa_status check_decode_args(const gqa_cache* c, int32_t B, const gqa_tensor* q, const gqa_tensor* o) {
  const gqa_cache_config& cf = c->cfg;
  if (!q || !o) return fail(GQA_ERR_ARG, "q or o is null");
  const int64_t Hq = q->shape[1];
  if (Hq < 1 || Hq % cf.num_kv_heads) return fail(GQA_ERR_SHAPE, "Hkv must divide Hq");
  gqa_status st = check_tensor(q, "q", cf.dtype, B, Hq, 1, cf.head_dim);
  if (st != GQA_OK) return st;
  return check_tensor(o, "o", cf.dtype, B, Hq, 1, cf.head_dim);
}

// The workspace a split-T call needs: none when every sequence fits one split,
// else at least `need` bytes (the documented size), 256-byte aligned, with
// room for the call's split slots.
gqa_status check_workspace(const gqa_cache* c, int32_t B, int64_t ncol, const int32_t* T, void* workspace,
                           size_t ws_bytes, size_t need) {
  if (c->cfg.dtype != GQA_BF16 || B == 0) return GQA_OK;
  const int64_t ys = split_ys(c, ncol);
  const int pps = decode_pages_per_split(T, B, ys);
  int64_t total_splits = 0;
  for (int b = 0; b < B; ++b) total_splits += split_count(T[b], pps);
  if (total_splits <= B) return GQA_OK;
  if (!workspace || ws_bytes < need) return fail(GQA_ERR_ARG, "workspace missing or smaller than its size query");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GQA_ERR_ARG, "workspace must be 256-byte aligned");
  if (ws_view(workspace, ws_bytes, c->cfg.head_dim).slots < total_splits * ys)
    return fail(GQA_ERR_ARG, "workspace smaller than its size query");
  return GQA_OK;
}

// Workspace slots a split-T call over lengths T takes (0 when every sequence
// fits one split and no workspace is needed).
int64_t split_slots_needed(const gqa_cache* c, int32_t B, int64_t ncol, const int32_t* T) {
  if (c->cfg.dtype != GQA_BF16 || B == 0) return 0;
  const int64_t ys = split_ys(c, ncol);
  const int pps = decode_pages_per_split(T, B, ys);
  int64_t total_splits = 0;
  for (int b = 0; b < B; ++b) total_splits += split_count(T[b], pps);
  return total_splits <= B ? 0 : total_splits * ys;
}

// Lengths a split-T call reads: start + count keys; a sequence with no query
// reads none (its single split only zeroes its rows of O).  The split path
// takes one entry per batch row, in batch order.
std::vector<int32_t> split_lengths(const std::vector<Entry>& es) {
  std::vector<int32_t> T(es.size());
  for (size_t b = 0; b < es.size(); ++b) T[b] = es[b].count ? es[b].start + es[b].count : 0;
  return T;
}

std::vector<int32_t> split_read_lengths(const gqa_cache* c, const std::vector<Entry>& es) {
  std::vector<int32_t> T(es.size());
  for (size_t b = 0; b < es.size(); ++b) T[b] = read_length(c, es[b].start, es[b].count);
  return T;
}

// read lengths of decode queries at T[b] - 1
std::vector<int32_t> decode_read_lengths(const gqa_cache* c, int32_t B, const int32_t* T) {
  std::vector<int32_t> r(B);
  for (int b = 0; b < B; ++b) r[b] = read_length(c, T[b] - 1, 1);
  return r;
}

int64_t split_ncol(const gqa_cache* c, int64_t Hq, const std::vector<Entry>& es) {
  int32_t longest = 1;
  for (const Entry& e : es) longest = std::max(longest, e.count);
  return static_cast<int64_t>(longest) * (Hq / c->cfg.num_kv_heads);
}

gqa_status check_split_workspace(const gqa_cache* c, int32_t B, int64_t Hq, int64_t n, const std::vector<Entry>& es,
                                 void* workspace, size_t ws_bytes) {
  const std::vector<int32_t> T = split_read_lengths(c, es);
  return check_workspace(c, B, split_ncol(c, Hq, es), T.data(), workspace, ws_bytes,
                         gqa_attention_workspace_size(c, B, static_cast<int32_t>(Hq), static_cast<int32_t>(n)));
}

gqa_status attend_split(gqa_cache* c, int32_t layer, const int32_t* seq_ids, const gqa_tensor* Q, const gqa_tensor* O,
                        int64_t n, const std::vector<Entry>& es, void* workspace, size_t ws_bytes, hipStream_t s) {
  const std::vector<int32_t> T = split_lengths(es);
  const int32_t B = static_cast<int32_t>(es.size());
  std::vector<int32_t> st0(B), count(B), row0(B);
  for (int b = 0; b < B; ++b) {
    count[b] = es[b].count;
    row0[b] = es[b].row0;
    st0[b] = T[b] - count[b];
  }
  return launch_split(c, layer, B, seq_ids, Q, O, st0.data(), count.data(), row0.data(), static_cast<int>(n),
                      static_cast<int>(split_ncol(c, Q->shape[1], es)), nullptr, nullptr, workspace, ws_bytes, s);
}

}  // namespace

GQA_EXPORT size_t gqa_workspace_size(const gqa_cache* c, int32_t B, int32_t Hq) {
  if (!c || B < 0 || Hq < 1) return 0;
  return ws_bytes_for(c, B, split_ys(c, std::max(1, Hq / c->cfg.num_kv_heads)));
}

GQA_EXPORT size_t gqa_attention_workspace_size(const gqa_cache* c, int32_t B, int32_t Hq, int32_t n) {
  if (!c || B < 0 || Hq < 1 || n < 1 || n > GQA_MAX_CHUNK_TOKENS || c->cfg.dtype != GQA_BF16) return 0;
  return ws_bytes_for(c, B, split_ys(c, static_cast<int64_t>(n) * std::max(1, Hq / c->cfg.num_kv_heads)));
}

GQA_EXPORT gqa_status gqa_workspace_status(const gqa_cache* c, void* workspace, size_t ws_bytes, int32_t clear,
                                           void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t count_d = 0;
  if (!workspace && ws_bytes == 0) {
    // the static scratch of the current device (set up here if no call has)
    hipError_t e = gqa::static_scratch(ws_zero_bytes(ws_slots(gqa::kStaticScratchBytes, 128)), s, &workspace);
    if (e != hipSuccess) return hip_fail(e, "static scratch set-up");
    ws_bytes = static_cast<size_t>(gqa::kStaticScratchBytes);
    count_d = 128;
  }
  const WsView wv = ws_view(workspace, ws_bytes, c->cfg.head_dim, count_d);
  if (!wv.slots) return fail(GQA_ERR_ARG, "workspace missing or smaller than one slot");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GQA_ERR_ARG, "workspace must be 256-byte aligned");
  int32_t word = 0;
  hipError_t e = hipMemcpyAsync(&word, wv.status, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "workspace status read");
  if (clear) {
    e = hipMemsetAsync(workspace, 0, static_cast<size_t>(wv.zero_bytes), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "workspace reset");
  }
  if (word)
    return fail(GQA_ERR_DEVICE,
                "a split merge gave up waiting for a split: some output written since the last clear holds NaN");
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_set_merge_wait(int32_t polls, int32_t unreachable) {
  if (polls < 0) return fail(GQA_ERR_ARG, "polls must be >= 0");
  g_spin_limit.store(polls);
  g_unreachable.store(unreachable ? 1 : 0);
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_decode(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                 const gqa_tensor* q, const int32_t* valid_lengths, const gqa_tensor* o,
                                 void* workspace, size_t ws_bytes, void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.num_layers) return fail(GQA_ERR_ARG, "layer out of range");
  gqa_status st = check_seqs(c, B, seq_ids);
  if (st != GQA_OK) return st;
  st = check_decode_args(c, B, q, o);
  if (st != GQA_OK) return st;
  if (B > 0 && !valid_lengths) return fail(GQA_ERR_ARG, "valid_lengths is null");
  for (int b = 0; b < B; ++b) {
    const int32_t have = c->len[static_cast<int64_t>(seq_ids[b]) * cf.num_layers + layer];
    if (valid_lengths[b] != have) return fail(GQA_ERR_CACHE, "valid length differs from the cache length");
    if (have < 1) return fail(GQA_ERR_CACHE, "decode needs at least one cached token");
  }
  if (B == 0) return GQA_OK;
  st = check_workspace(c, B, q->shape[1] / cf.num_kv_heads, decode_read_lengths(c, B, valid_lengths).data(),
                       workspace, ws_bytes,
                       gqa_workspace_size(c, B, static_cast<int32_t>(q->shape[1])));
  if (st != GQA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (cf.dtype != GQA_BF16) return launch_decode_f32(c, layer, B, seq_ids, q, o, valid_lengths, s);
  return launch_decode(c, layer, B, seq_ids, q, o, valid_lengths, nullptr, nullptr, workspace, ws_bytes, s);
}

namespace {

// gqa_decode_step on a caller's workspace, or (static_scratch) on the
// library's static scratch of the current device, which allocates nothing.
gqa_status decode_step(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids, const gqa_tensor* q,
                       const gqa_tensor* k_new, const gqa_tensor* v_new, const gqa_tensor* o, void* workspace,
                       size_t ws_bytes, void* stream, bool static_scratch) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (layer < 0 || layer >= cf.num_layers) return fail(GQA_ERR_ARG, "layer out of range");
  gqa_status st = check_seqs(c, B, seq_ids);
  if (st != GQA_OK) return st;
  st = check_decode_args(c, B, q, o);
  if (st != GQA_OK) return st;
  if (B == 0) return GQA_OK;
  // the new token sits at position c_b (the current length) of every sequence
  std::vector<uint8_t> mask(B, 1);
  std::vector<int32_t> pos(B);
  for (int b = 0; b < B; ++b) pos[b] = c->len[static_cast<int64_t>(seq_ids[b]) * cf.num_layers + layer];
  AppendPlan plan;
  st = plan_append(c, layer, B, seq_ids, k_new, v_new, mask.data(), pos.data(), &plan);
  if (st != GQA_OK) return st;
  if (plan.n != 1) return fail(GQA_ERR_SHAPE, "k_new and v_new must hold one token: [B, Hkv, 1, d]");
  std::vector<int32_t> T(B);
  for (int b = 0; b < B; ++b) T[b] = pos[b] + 1;
  const int64_t ncol = q->shape[1] / cf.num_kv_heads;
  const std::vector<int32_t> Tr = decode_read_lengths(c, B, T.data());
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (static_scratch) {
    const int64_t need = split_slots_needed(c, B, ncol, Tr.data());
    void* base = nullptr;
    if (need > 0) {
      const int64_t have = ws_slots(gqa::kStaticScratchBytes, 128);
      if (need > have)
        return fail(GQA_ERR_UNSUPPORTED, "the call needs " + std::to_string(need) + " split slots (" +
                                             std::to_string(2 * kWsHeader + need * ws_slot_bytes(128)) +
                                             " bytes), more than the static scratch holds (" +
                                             std::to_string(have) + " slots, " +
                                             std::to_string(gqa::kStaticScratchBytes) +
                                             " bytes): use gqa_decode_step with a workspace");
      hipError_t e = gqa::static_scratch(ws_zero_bytes(have), s, &base);
      if (e != hipSuccess) return hip_fail(e, "static scratch set-up");
    }
    workspace = base;
    ws_bytes = base ? static_cast<size_t>(gqa::kStaticScratchBytes) : 0;
  } else {
    st = check_workspace(c, B, ncol, Tr.data(), workspace, ws_bytes,
                         gqa_workspace_size(c, B, static_cast<int32_t>(q->shape[1])));
    if (st != GQA_OK) return st;
  }
  commit_append(c, layer, B, seq_ids, plan);
  if (cf.dtype != GQA_BF16) {
    st = sync_metadata(c, s);
    if (st != GQA_OK) return st;
    st = launch_append_all(c, layer, B, seq_ids, k_new, v_new, plan, s);
    if (st != GQA_OK) return st;
    return launch_decode_f32(c, layer, B, seq_ids, q, o, T.data(), s);
  }
  return launch_decode(c, layer, B, seq_ids, q, o, T.data(), k_new, v_new, workspace, ws_bytes, s,
                       static_scratch ? 128 : 0);
}

}  // namespace

GQA_EXPORT gqa_status gqa_decode_step(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                      const gqa_tensor* q, const gqa_tensor* k_new, const gqa_tensor* v_new,
                                      const gqa_tensor* o, void* workspace, size_t ws_bytes, void* stream) {
  return decode_step(c, layer, B, seq_ids, q, k_new, v_new, o, workspace, ws_bytes, stream, false);
}

GQA_EXPORT gqa_status gqa_decode_step_noalloc(gqa_cache* c, int32_t layer, int32_t B, const int32_t* seq_ids,
                                              const gqa_tensor* q, const gqa_tensor* k_new,
                                              const gqa_tensor* v_new, const gqa_tensor* o, void* stream) {
  return decode_step(c, layer, B, seq_ids, q, k_new, v_new, o, nullptr, 0, stream, true);
}

// ------------------------------------------------------------------ truncate / remap

GQA_EXPORT gqa_status kv_cache_truncate(gqa_cache* c, int32_t seq_id, int32_t m) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (seq_id < 0 || seq_id >= cf.max_seqs) return fail(GQA_ERR_ARG, "sequence id out of range");
  if (m < 0) return fail(GQA_ERR_ARG, "negative truncation point");
  if (cf.window && m > 0) {
    for (int l = 0; l < cf.num_layers; ++l)
      if (m < c->len[static_cast<int64_t>(seq_id) * cf.num_layers + l])
        return fail(GQA_ERR_UNSUPPORTED, "a ring sequence can only be released or left as it is");
  }
  int32_t longest = 0;
  for (int l = 0; l < cf.num_layers; ++l) {
    int32_t& n = c->len[static_cast<int64_t>(seq_id) * cf.num_layers + l];
    n = std::min(n, m);
    longest = std::max(longest, n);
  }
  const size_t keep = static_cast<size_t>(table_entries(cf, longest));
  std::vector<int32_t>& pl = c->pages[seq_id];
  for (size_t i = keep; i < pl.size(); ++i)
    if (--c->ref[pl[i]] == 0) c->free_list.push_back(pl[i]);
  if (pl.size() > keep) pl.resize(keep);
  return GQA_OK;
}

GQA_EXPORT gqa_status kv_cache_fork(gqa_cache* c, int32_t src, int32_t dst, int32_t m) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (src < 0 || src >= cf.max_seqs || dst < 0 || dst >= cf.max_seqs || src == dst)
    return fail(GQA_ERR_ARG, "bad sequence ids");
  if (m < 0) return fail(GQA_ERR_ARG, "negative fork length");
  if (cf.window) return fail(GQA_ERR_UNSUPPORTED, "ring sequences are not forked");
  int32_t src_len = INT32_MAX;
  for (int l = 0; l < cf.num_layers; ++l) {
    if (c->len[static_cast<int64_t>(dst) * cf.num_layers + l] != 0)
      return fail(GQA_ERR_CACHE, "the destination sequence is not empty");
    src_len = std::min(src_len, c->len[static_cast<int64_t>(src) * cf.num_layers + l]);
  }
  if (!c->pages[dst].empty()) return fail(GQA_ERR_CACHE, "the destination sequence is not empty");
  if (m > src_len) return fail(GQA_ERR_POSITION, "fork length beyond the source's length");
  const int64_t np = ceil_div(m, kPage);
  c->pages[dst].assign(c->pages[src].begin(), c->pages[src].begin() + np);
  for (int64_t lp = 0; lp < np; ++lp) {
    ++c->ref[c->pages[dst][lp]];
    c->pending.emplace_back(dst * cf.max_pages_per_seq + static_cast<int32_t>(lp), c->pages[dst][lp]);
  }
  for (int l = 0; l < cf.num_layers; ++l) c->len[static_cast<int64_t>(dst) * cf.num_layers + l] = m;
  return GQA_OK;
}

GQA_EXPORT gqa_status kv_cache_remap(gqa_cache* c, int32_t n, const int32_t* src, const int32_t* dst, void* stream) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  if (n < 0) return fail(GQA_ERR_ARG, "negative page count");
  if (n == 0) return GQA_OK;
  if (!src || !dst) return fail(GQA_ERR_ARG, "src or dst is null");
  std::vector<char> is_free(cf.num_pages, 0);
  for (int32_t p : c->free_list) is_free[p] = 1;
  std::vector<char> seen_src(cf.num_pages, 0), seen_dst(cf.num_pages, 0);
  for (int i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= cf.num_pages || dst[i] < 0 || dst[i] >= cf.num_pages)
      return fail(GQA_ERR_ARG, "page id out of range");
    if (seen_src[src[i]] || seen_dst[dst[i]]) return fail(GQA_ERR_ARG, "repeated page");
    seen_src[src[i]] = seen_dst[dst[i]] = 1;
  }
  for (int i = 0; i < n; ++i) {
    if (c->ref[src[i]] == 0) return fail(GQA_ERR_CACHE, "source page is not in use");
    if (!is_free[dst[i]]) return fail(GQA_ERR_CACHE, "destination page is not free");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  gqa_status st = sync_metadata(c, s);
  if (st != GQA_OK) return st;
  std::vector<std::pair<int32_t, int32_t>> moves(n);
  for (int i = 0; i < n; ++i) moves[i] = {src[i], dst[i]};
  st = launch_copies(c, moves, s);
  if (st != GQA_OK) return st;
  // every table entry that references a moved page (a shared page has several)
  std::vector<int32_t> moved_to(cf.num_pages, -1);
  for (int i = 0; i < n; ++i) moved_to[src[i]] = dst[i];
  for (int sq = 0; sq < cf.max_seqs; ++sq)
    for (size_t lp = 0; lp < c->pages[sq].size(); ++lp) {
      const int32_t to = moved_to[c->pages[sq][lp]];
      if (to < 0) continue;
      c->pages[sq][lp] = to;
      c->pending.emplace_back(sq * cf.max_pages_per_seq + static_cast<int32_t>(lp), to);
    }
  for (int i = 0; i < n; ++i) {
    c->ref[dst[i]] = c->ref[src[i]];
    c->ref[src[i]] = 0;
    c->free_list.erase(std::find(c->free_list.begin(), c->free_list.end(), dst[i]));
  }
  for (int i = 0; i < n; ++i) c->free_list.push_back(src[i]);
  return sync_metadata(c, s);
}

// ------------------------------------------------------------------ queries

GQA_EXPORT gqa_status gqa_cache_length(const gqa_cache* c, int32_t seq_id, int32_t layer, int32_t* out) {
  if (!c || !out) return fail(GQA_ERR_ARG, "null argument");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs || layer < 0 || layer >= c->cfg.num_layers)
    return fail(GQA_ERR_ARG, "sequence or layer out of range");
  *out = c->len[static_cast<int64_t>(seq_id) * c->cfg.num_layers + layer];
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_cache_page_table(const gqa_cache* c, int32_t seq_id, int32_t* out, int32_t cap,
                                           int32_t* n_out) {
  if (!c || !n_out) return fail(GQA_ERR_ARG, "null argument");
  if (seq_id < 0 || seq_id >= c->cfg.max_seqs) return fail(GQA_ERR_ARG, "sequence id out of range");
  const std::vector<int32_t>& pl = c->pages[seq_id];
  *n_out = static_cast<int32_t>(pl.size());
  if (static_cast<int64_t>(pl.size()) > cap) return fail(GQA_ERR_ARG, "output capacity too small");
  if (!pl.empty() && !out) return fail(GQA_ERR_ARG, "out is null");
  for (size_t i = 0; i < pl.size(); ++i) out[i] = pl[i];
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_cache_free_pages(const gqa_cache* c, int32_t* out) {
  if (!c || !out) return fail(GQA_ERR_ARG, "null argument");
  *out = static_cast<int32_t>(c->free_list.size());
  return GQA_OK;
}

GQA_EXPORT gqa_status gqa_cache_check(const gqa_cache* c) {
  if (!c) return fail(GQA_ERR_ARG, "cache is null");
  const gqa_cache_config& cf = c->cfg;
  std::vector<int> count(cf.num_pages, 0);
  for (int s = 0; s < cf.max_seqs; ++s) {
    int32_t lmin = INT32_MAX, lmax = 0;
    for (int l = 0; l < cf.num_layers; ++l) {
      const int32_t n = c->len[static_cast<int64_t>(s) * cf.num_layers + l];
      lmin = std::min(lmin, n);
      lmax = std::max(lmax, n);
    }
    if (lmin != lmax) return fail(GQA_ERR_CACHE, "sequence " + std::to_string(s) + ": layer lengths differ");
    if (static_cast<int64_t>(c->pages[s].size()) != table_entries(cf, lmax))
      return fail(GQA_ERR_CACHE, "sequence " + std::to_string(s) + ": page count does not match its length");
    std::vector<int32_t> own(c->pages[s]);
    std::sort(own.begin(), own.end());
    if (std::adjacent_find(own.begin(), own.end()) != own.end())
      return fail(GQA_ERR_CACHE, "sequence " + std::to_string(s) + ": a page appears twice in its table");
    for (int32_t p : c->pages[s]) ++count[p];
  }
  std::vector<int> listed(cf.num_pages, 0);
  for (int32_t p : c->free_list) ++listed[p];
  for (int p = 0; p < cf.num_pages; ++p) {
    if (count[p] != c->ref[p])
      return fail(GQA_ERR_CACHE, "page " + std::to_string(p) + ": reference count differs from the tables");
    if (listed[p] > 1 || (listed[p] == 1) == (count[p] > 0))
      return fail(GQA_ERR_CACHE, "page " + std::to_string(p) + " is lost, listed twice or free while referenced");
  }
  return GQA_OK;
}

namespace gqa {
// for the other host sources of the library (the prefix index)
void set_last_error(const char* msg) { g_err = msg; }
}  // namespace gqa

GQA_EXPORT const char* gqa_last_error(void) { return g_err.c_str(); }
