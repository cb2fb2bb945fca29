// Host work planner for the persistent attention kernels.
//
// The FlashInfer paper summary ("Research methodology" 3, dynamic
// load-balanced scheduling) describes the split this file implements:
// query-tile sizes are fixed when the kernels are compiled, while the
// runtime sequence lengths drive a CPU plan that spreads the work evenly
// over all compute units; the plan is copied to the GPU and a fixed-size
// launch runs it, so it stays compatible with graph capture.  The PR #5329
// analysis ("Code analysis" 1) shows the persistent kernel taking its grid
// from the plan and serving a 128-row and a 16-row query-tile class.
//
// The pages give no algorithm, so the plan is defined here, in integer
// arithmetic with explicit tie-breaks (the test oracle implements the same
// rules independently and must agree bit for bit):
//
//  1. Units: for each request r with qo_len > 0 and kv_len > 0, each kv
//     head h and each query tile t.  Rows of a request are (token i, group
//     member u) flattened as i*g + u; tile t covers rows
//     [t*tile_q, min((t+1)*tile_q, qo_len*g)).  With i_lo/i_hi its first and
//     last token and qpos(i) = kv_len - qo_len + i, the unit needs keys
//     [lo, hi): hi = min(kv_len, qpos(i_hi) + 1) if causal else kv_len;
//     lo = max(0, qpos(i_lo) - window + 1) if window > 0 else 0; plus the
//     sink range [0, min(sink, lo)) when window > 0 and lo > 0.
//  2. Total cost C = sum of (hi - lo) + |sink range| over units.
//  3. Chunk length L_c = max(min_chunk, roundup(ceil(C * (16 + s) / (16 W split)), tile_kv)),
//     then min(L_c, max_chunk) if max_chunk > 0.  The slack s is 1 when
//     tile_q = 16 (a plan of 16-row decode tiles only) and 0 otherwise:
//     decode chunks a sixteenth longer than an even share leave fewer short
//     remainder chunks, and for bandwidth-bound decode items one item fewer
//     outweighs the coarser balance.  Plans with 128-row tiles keep s = 0
//     (the mixed launch measured slower with the slack).
//  4. A unit's chunks: with lo_a = lo rounded down to a multiple of tile_kv,
//     [max(lo, lo_a + k L_c), min(hi, lo_a + (k+1) L_c)) for
//     k = 0 .. (hi-1-lo_a) / L_c, then the non-empty sink range (boundaries
//     stay tile_kv-aligned, and a window of n L_c keys is n chunks).
//  5. Items in unit order, then chunk order; id = creation index;
//     cost = keys + item_overhead.  Units with >= 2 chunks take consecutive
//     partial slots from a global counter; single-chunk units use slot -1.
//  6. Longest-processing-time assignment: items sorted by (cost desc, id
//     asc); a priority queue of (load, worker) starting at (0, w); each item
//     takes the lexicographic minimum, is appended to that worker's list,
//     and (load + cost, worker) is pushed back.
//  7. Merge table: one entry per multi-chunk unit, in unit order.
//  8. More than max_items_per_worker items on a worker, max_slots slots or
//     max_merge entries is a capacity error (no fallback).
//
// Composable batches (shared_prefix_len P > 0; the paper summary's
// composable formats, "Research methodology" 1): every request's KV is a
// dense prefix of P tokens shared by the batch, then its own paged suffix of
// kv_len keys (queries causal within the suffix, the whole prefix in their
// past).  Prefix units come first -- per kv head, tile_q tiles of the batch's
// global query rows (request r's rows are qo_indptr[r] * g + [0, qo_len * g)),
// keys [0, P), tile class 2, r = -1 -- then the suffix units by rules 1-2.
// Every unit takes partial slots, and each suffix unit's merge entry also
// names the first slot of its kv head's first prefix unit and the chunk
// count of a prefix unit: row rr of the entry is global row R = qo_indptr[r]
// * g + row_lo + rr, whose prefix partials are row R % tile_q of slots
// first + (R / tile_q) * n + c.

#include "plan.h"

#include <algorithm>
#include <array>
#include <cstring>
#include <utility>
#include <vector>

#include "layout.h"

namespace bsk {
namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int32_t kDecodeTileQ = 16;  // rows of a decode-class query tile (chunk slack, rule 3)
constexpr int kWorkerBits = 20;  // the LPT assignment packs (load, worker) into 64 bits
constexpr uint64_t kWorkerMask = (uint64_t(1) << kWorkerBits) - 1;
inline int64_t align4(int64_t x) { return (x + 3) & ~int64_t(3); }

struct Layout {
  int64_t off_items, off_merge, off_qo, off_kvlen, off_kvind, off_slotmap, off_count, total_words;
};

// Word offsets for a plan with `n_items` items, `n_merge` merge entries and `n_slots` slots.
Layout layout_for(int32_t W, int64_t n_items, int64_t n_merge, int64_t n_slots, int32_t batch) {
  Layout L;
  L.off_items = align4(HDR_WORDS + int64_t(W) + 1);
  L.off_merge = L.off_items + n_items * ITEM_WORDS;
  L.off_qo = L.off_merge + n_merge * MERGE_WORDS;
  L.off_kvlen = L.off_qo + batch + 1;
  L.off_kvind = L.off_kvlen + batch;
  L.off_slotmap = L.off_kvind + batch + 1;
  L.off_count = L.off_slotmap + n_slots;
  L.total_words = L.off_count + n_merge;
  return L;
}

struct Unit {
  int32_t r, h, row_lo, row_hi, lo, hi, sink_hi, cls;
};

struct Item {
  int32_t r, h, row_lo, row_hi, kv_lo, kv_hi, slot, cls;
  int64_t cost;
};

// Winner tree over unique 64-bit keys: leaves t[n + w] (n a power of two,
// padding leaves at UINT64_MAX), every inner node the smaller of its two
// children, so t[1] is the minimum.  Raising one leaf recomputes the path to
// the root.  The path is fixed by the leaf index, so the sibling loads are
// independent of each other and only the comparisons form a chain (a binary
// heap's sift-down chains its loads instead, one per level).
inline void raise_leaf(uint64_t* t, int32_t n, int32_t w, uint64_t key) {
  int32_t i = n + w;
  t[i] = key;
  while (i > 1) {
    const uint64_t sib = t[i ^ 1];
    key = sib < key ? sib : key;
    i >>= 1;
    t[i] = key;
  }
}

}  // namespace

size_t plan_workspace_bytes(const PlanParams& p) {
  const int64_t max_items = int64_t(p.num_workers) * p.max_items_per_worker;
  Layout L = layout_for(p.num_workers, max_items, p.max_merge, p.max_slots, p.max_batch);
  return size_t(L.total_words) * sizeof(int32_t);
}

PlanResult build_plan(const PlanParams& p, int32_t batch, const int32_t* qo_indptr, const int32_t* kv_len,
                      const int32_t* kv_indptr, int32_t* buf, size_t buf_bytes, PlanStats* stats,
                      std::string* err) {
  auto fail = [&](PlanResult code, const std::string& msg) {
    if (err) *err = msg;
    return code;
  };
  if (p.num_kv_heads <= 0 || p.num_qo_heads <= 0 || p.num_qo_heads % p.num_kv_heads != 0)
    return fail(PLAN_INVALID, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (p.tile_q <= 0 || p.tile_kv <= 0 || p.num_workers <= 0 || p.split_factor <= 0)
    return fail(PLAN_INVALID, "tile_q, tile_kv, num_workers and split_factor must be positive");
  if (p.num_workers > int32_t(kWorkerMask)) return fail(PLAN_INVALID, "num_workers must be below 2^20");
  if (p.min_chunk <= 0 || p.min_chunk % p.tile_kv != 0)
    return fail(PLAN_INVALID, "min_chunk must be a positive multiple of tile_kv");
  if (p.max_chunk < 0 || (p.max_chunk > 0 && (p.max_chunk % p.tile_kv != 0 || p.max_chunk < p.min_chunk)))
    return fail(PLAN_INVALID, "max_chunk must be 0 or a multiple of tile_kv that is >= min_chunk");
  if (p.item_overhead < 0) return fail(PLAN_INVALID, "item_overhead must be >= 0");
  if (p.shared_prefix_len < 0 || (p.shared_prefix_len > 0 && p.window > 0))
    return fail(PLAN_INVALID, "a shared prefix needs prefix length >= 0 and no sliding window");
  if (batch < 0 || batch > p.max_batch) return fail(PLAN_INVALID, "batch must be in [0, max_batch]");
  if (batch > 0 && (!qo_indptr || !kv_len || !kv_indptr)) return fail(PLAN_INVALID, "null length array");
  if (!buf) return fail(PLAN_INVALID, "null host workspace");
  if (buf_bytes < plan_workspace_bytes(p)) return fail(PLAN_WORKSPACE, "host workspace smaller than bsk_workspace_query");

  const int32_t g = p.num_qo_heads / p.num_kv_heads;
  const int32_t W = p.num_workers;
  if (batch > 0 && qo_indptr[0] != 0) return fail(PLAN_INVALID, "qo_indptr[0] must be 0");
  int32_t max_kv = 0, max_qo = 0;
  for (int32_t r = 0; r < batch; ++r) {
    const int64_t Q = int64_t(qo_indptr[r + 1]) - qo_indptr[r];
    const int64_t L = kv_len[r];
    if (Q < 0 || L < 0 || Q > L) return fail(PLAN_INVALID, "need 0 <= qo_len <= kv_len for every request");
    if (kv_indptr[r + 1] < kv_indptr[r]) return fail(PLAN_INVALID, "kv_indptr must be non-decreasing");
    if (Q * g > INT32_MAX) return fail(PLAN_INVALID, "too many query rows");
    max_kv = std::max<int32_t>(max_kv, int32_t(L));
    max_qo = std::max<int32_t>(max_qo, int32_t(Q));
  }

  // 1. units (scratch containers are kept per thread across calls); the shared prefix's first
  const int32_t P = p.shared_prefix_len;
  const int64_t T = batch > 0 ? int64_t(qo_indptr[batch]) : 0;
  if (P > 0 && T * g > INT32_MAX) return fail(PLAN_INVALID, "too many query rows");
  thread_local std::vector<Unit> units;
  units.clear();
  if (P > 0) {
    const int32_t rows = int32_t(T * g);
    for (int32_t h = 0; h < p.num_kv_heads; ++h)
      for (int32_t t = 0; t < int32_t(ceil_div(rows, p.tile_q)); ++t)
        units.push_back(Unit{-1, h, t * p.tile_q, std::min(rows, (t + 1) * p.tile_q), 0, P, 0, 2});
  }
  const size_t n_prefix_units = units.size();
  for (int32_t r = 0; r < batch; ++r) {
    const int32_t Q = qo_indptr[r + 1] - qo_indptr[r];
    const int32_t L = kv_len[r];
    if (Q == 0 || L == 0) continue;
    const int32_t rows = Q * g;
    // two tile classes: a request whose rows fit one decode tile gets one decode-class unit
    const bool small = p.decode_tile_q > 0 && rows <= p.decode_tile_q;
    const int32_t tq = small ? p.decode_tile_q : p.tile_q;
    for (int32_t h = 0; h < p.num_kv_heads; ++h) {
      for (int32_t t = 0; t < int32_t(ceil_div(rows, tq)); ++t) {
        Unit u;
        u.r = r;
        u.h = h;
        u.cls = small ? 1 : 0;
        u.row_lo = t * tq;
        u.row_hi = std::min(rows, (t + 1) * tq);
        const int32_t qpos_lo = L - Q + u.row_lo / g;
        const int32_t qpos_hi = L - Q + (u.row_hi - 1) / g;
        u.hi = p.causal ? std::min(L, qpos_hi + 1) : L;
        u.lo = p.window > 0 ? std::max(0, qpos_lo - p.window + 1) : 0;
        u.sink_hi = (p.window > 0 && u.lo > 0) ? std::min(p.sink, u.lo) : 0;
        units.push_back(u);
      }
    }
  }

  // 2-3. total cost and chunk length
  int64_t C = 0;
  for (const Unit& u : units) C += int64_t(u.hi - u.lo) + u.sink_hi;
  const int64_t slack = p.tile_q == kDecodeTileQ ? 1 : 0;
  int64_t Lc = ceil_div(ceil_div(C * (16 + slack), int64_t(W) * p.split_factor * 16), p.tile_kv) * p.tile_kv;
  Lc = std::max<int64_t>(p.min_chunk, Lc);
  if (p.max_chunk > 0) Lc = std::min<int64_t>(Lc, p.max_chunk);
  if (Lc > INT32_MAX) return fail(PLAN_INVALID, "chunk length overflows int32");
  if (C + int64_t(p.item_overhead) * (C / p.tile_kv + int64_t(units.size()) * 2 + 1) >= (int64_t(1) << 42))
    return fail(PLAN_INVALID, "total work too large for the planner's load counters");

  // 4-5. chunks -> items, slots, merge entries
  thread_local std::vector<Item> items;
  thread_local std::vector<std::array<int32_t, MERGE_WORDS>> merges;
  thread_local std::vector<int32_t> prefix_first;  // per kv head: first slot of its first prefix unit
  items.clear();
  merges.clear();
  prefix_first.assign(size_t(p.num_kv_heads), -1);
  int32_t prefix_n = 0;
  int64_t next_slot = 0;
  thread_local std::vector<std::pair<int32_t, int32_t>> chunks;
  for (size_t ui = 0; ui < units.size(); ++ui) {
    const Unit& u = units[ui];
    chunks.clear();
    const int64_t lo_a = int64_t(u.lo) / p.tile_kv * p.tile_kv;
    for (int64_t k = 0; k <= (int64_t(u.hi) - 1 - lo_a) / Lc; ++k)
      chunks.emplace_back(int32_t(std::max<int64_t>(u.lo, lo_a + k * Lc)),
                          int32_t(std::min<int64_t>(u.hi, lo_a + (k + 1) * Lc)));
    if (u.sink_hi > 0) chunks.emplace_back(0, u.sink_hi);
    const bool split = chunks.size() >= 2 || P > 0;
    const int64_t first = next_slot;
    if (split) {
      next_slot += int64_t(chunks.size());
      if (next_slot > p.max_slots) return fail(PLAN_CAPACITY, "more partial-state slots than max_slots");
      if (ui < n_prefix_units) {
        if (prefix_first[size_t(u.h)] < 0) prefix_first[size_t(u.h)] = int32_t(first);
        prefix_n = int32_t(chunks.size());
      } else {
        const bool pfx = P > 0;
        merges.push_back({u.r, u.h, u.row_lo, u.row_hi, int32_t(first), int32_t(chunks.size()),
                          pfx ? prefix_first[size_t(u.h)] : 0, pfx ? prefix_n : 0});
      }
    }
    for (size_t c = 0; c < chunks.size(); ++c) {
      Item it;
      it.r = u.r;
      it.h = u.h;
      it.row_lo = u.row_lo;
      it.row_hi = u.row_hi;
      it.kv_lo = chunks[c].first;
      it.kv_hi = chunks[c].second;
      it.slot = split ? int32_t(first + int64_t(c)) : -1;
      it.cls = u.cls;
      it.cost = int64_t(it.kv_hi - it.kv_lo) + p.item_overhead;
      items.push_back(it);
    }
  }
  if (int64_t(merges.size()) > p.max_merge) return fail(PLAN_CAPACITY, "more merge entries than max_merge");
  if (int64_t(items.size()) > int64_t(W) * p.max_items_per_worker)
    return fail(PLAN_CAPACITY, "more items than num_workers * max_items_per_worker");

  // 6. LPT assignment (flat arrays; the per-worker lists are built as CSR
  //    afterwards, each in assignment order)
  thread_local std::vector<int32_t> order, assign, counts, bucket;
  thread_local std::vector<uint64_t> tree;
  const int32_t n_items = int32_t(items.size());
  // order = items by (cost desc, id asc): a stable counting sort on cost
  // (costs are bounded by the chunk length plus the overhead)
  int64_t max_cost = 0;
  for (const Item& it : items) max_cost = std::max(max_cost, it.cost);
  bucket.assign(size_t(max_cost) + 2, 0);
  for (const Item& it : items) ++bucket[size_t(max_cost - it.cost)];
  int32_t run = 0;
  for (size_t c = 0; c < bucket.size(); ++c) {
    const int32_t k = bucket[c];
    bucket[c] = run;
    run += k;
  }
  order.resize(n_items);
  for (int32_t i = 0; i < n_items; ++i) order[size_t(bucket[size_t(max_cost - items[i].cost)]++)] = i;
  assign.resize(n_items);
  counts.assign(W + 1, 0);
  thread_local std::vector<int64_t> load;
  load.assign(W, 0);
  // All workers start at load 0 and ties go to the lower worker, so the
  // leading run of items with the largest cost is dealt round-robin: after
  // every full round all loads are equal again.  Exactly what the queue
  // would produce, without its per-item cost.
  int32_t k = 0;
  if (n_items > 0) {
    const int64_t c0 = items[order[0]].cost;
    while (k < n_items && items[order[k]].cost == c0) {
      const int32_t w = k % W;
      assign[k] = w;
      ++counts[w];
      load[w] += c0;
      ++k;
    }
  }
  // the rest: each item goes to the worker with the smallest (load, worker),
  // kept as load << 20 | worker so that one integer comparison gives the
  // lexicographic order, in a winner tree over the workers
  int32_t leaves = 1;
  while (leaves < W) leaves *= 2;
  tree.assign(size_t(2 * leaves), ~uint64_t(0));
  for (int32_t w = 0; w < W; ++w) tree[size_t(leaves + w)] = (uint64_t(load[w]) << kWorkerBits) | uint64_t(w);
  for (int32_t i = leaves - 1; i >= 1; --i)
    tree[size_t(i)] = std::min(tree[size_t(2 * i)], tree[size_t(2 * i + 1)]);
  for (; k < n_items; ++k) {
    const uint64_t top = tree[1];
    const int32_t w = int32_t(top & kWorkerMask);
    const int32_t id = order[k];
    assign[k] = w;
    ++counts[w];
    const uint64_t key = top + (uint64_t(items[id].cost) << kWorkerBits);
    load[w] = int64_t(key >> kWorkerBits);
    raise_leaf(tree.data(), leaves, w, key);
  }
  int32_t max_on_worker = 0;
  for (int32_t w = 0; w < W; ++w) max_on_worker = std::max(max_on_worker, counts[w]);
  if (max_on_worker > p.max_items_per_worker)
    return fail(PLAN_CAPACITY, "more items on one worker than max_items_per_worker");

  // 7. serialise
  const Layout L = layout_for(W, int64_t(items.size()), int64_t(merges.size()), next_slot, batch);
  // every word is written below; zeroed here are the header's padding before the items, and the
  // slot map (prefix slots belong to no merge entry) and the arrival counters after the arrays
  std::memset(buf, 0, size_t(L.off_items) * sizeof(int32_t));
  std::memset(buf + L.off_slotmap, 0, size_t(L.total_words - L.off_slotmap) * sizeof(int32_t));
  buf[HDR_NUM_ITEMS] = int32_t(items.size());
  buf[HDR_NUM_MERGE] = int32_t(merges.size());
  buf[HDR_NUM_SLOTS] = int32_t(next_slot);
  buf[HDR_NUM_WORKERS] = W;
  buf[HDR_BATCH] = batch;
  buf[HDR_CHUNK] = int32_t(Lc);
  buf[HDR_TILE_Q] = p.tile_q;
  buf[HDR_OFF_ITEMS] = int32_t(L.off_items);
  buf[HDR_OFF_MERGE] = int32_t(L.off_merge);
  buf[HDR_OFF_QO] = int32_t(L.off_qo);
  buf[HDR_OFF_KVLEN] = int32_t(L.off_kvlen);
  buf[HDR_OFF_KVIND] = int32_t(L.off_kvind);
  buf[HDR_MAX_KV_LEN] = max_kv;
  buf[HDR_MAX_QO_LEN] = max_qo;
  buf[HDR_OFF_SLOTMAP] = int32_t(L.off_slotmap);
  buf[HDR_OFF_COUNT] = int32_t(L.off_count);
  int32_t* wptr = buf + HDR_WORDS;
  int32_t* out = buf + L.off_items;
  wptr[0] = 0;
  for (int32_t w = 0; w < W; ++w) wptr[w + 1] = wptr[w] + counts[w];
  for (int32_t w = 0; w < W; ++w) counts[w] = wptr[w];  // reuse as fill cursors
  for (int32_t k = 0; k < n_items; ++k) {
    const int32_t id = order[k];
    const Item& it = items[id];
    int32_t* rec = out + int64_t(counts[assign[k]]++) * ITEM_WORDS;
    rec[IT_R] = it.r;
    rec[IT_H] = it.h;
    rec[IT_ROW_LO] = it.row_lo;
    rec[IT_ROW_HI] = it.row_hi;
    rec[IT_KV_LO] = it.kv_lo;
    rec[IT_KV_HI] = it.kv_hi;
    rec[IT_SLOT] = it.slot;
    rec[IT_ID] = id;
    if (it.r >= 0) {
      rec[IT_Q0] = qo_indptr[it.r];
      rec[IT_QLEN] = qo_indptr[it.r + 1] - qo_indptr[it.r];
      rec[IT_KVLEN] = kv_len[it.r];
      rec[IT_KBASE] = kv_indptr[it.r];
    } else {  // shared prefix: the batch's global query rows against the dense prefix
      rec[IT_Q0] = 0;
      rec[IT_QLEN] = int32_t(T);
      rec[IT_KVLEN] = P;
      rec[IT_KBASE] = 0;
    }
    rec[IT_CLASS] = it.cls;
    for (int w = IT_CLASS + 1; w < ITEM_WORDS; ++w) rec[w] = 0;
  }
  for (size_t m = 0; m < merges.size(); ++m) {
    int32_t* rec = buf + L.off_merge + int64_t(m) * MERGE_WORDS;
    for (int k = 0; k < MERGE_WORDS; ++k) rec[k] = merges[m][k];
    for (int32_t c = 0; c < merges[m][5]; ++c) buf[L.off_slotmap + merges[m][4] + c] = int32_t(m);
  }
  for (int32_t r = 0; r <= batch; ++r) buf[L.off_qo + r] = batch ? qo_indptr[r] : 0;
  for (int32_t r = 0; r < batch; ++r) buf[L.off_kvlen + r] = kv_len[r];
  for (int32_t r = 0; r <= batch; ++r) buf[L.off_kvind + r] = batch ? kv_indptr[r] : 0;

  if (stats) {
    stats->num_items = int32_t(items.size());
    stats->num_slots = int32_t(next_slot);
    stats->num_merge = int32_t(merges.size());
    stats->chunk = int32_t(Lc);
    stats->max_kv_len = max_kv;
    stats->max_qo_len = max_qo;
    stats->max_items_on_worker = max_on_worker;
    int64_t tc = 0, ml = 0;
    for (const Item& it : items) tc += it.cost;
    for (int64_t l : load) ml = std::max(ml, l);
    stats->total_cost = tc;
    stats->max_load = ml;
    stats->used_bytes = L.total_words * int64_t(sizeof(int32_t));
  }
  return PLAN_OK;
}

}  // namespace bsk
