"""Reference work partition (plan) for the persistent attention kernels (test infrastructure only).

The FlashInfer paper summary [FI-paper, research methodology 3: dynamic
load-balanced scheduling] says only that compile-time tile sizes are
decoupled from runtime scheduling, that a CPU plan built from the
requests' runtime lengths spreads the work evenly over all cores, and that
the plan is cached on the GPU so one fixed, graph-compatible launch
executes it; [FI-PR5329, code analysis 1] adds that the persistent kernel
runs two tile classes (128- and 16-row query tiles) on a grid fixed by the
plan.  The pages give no algorithm, so this module *defines* one, in
integer arithmetic with every tie broken explicitly, so that an
independent implementation can match it bit for bit:

1. Units.  For each request r with qo_len > 0 and kv_len > 0, each kv head
   h, and each query tile t: the request's rows are (token i, group member
   u) flattened as row = i*g + u; tile t covers rows
   [t*tile_q, min((t+1)*tile_q, qo_len*g)).  With i_lo / i_hi the first /
   last token of the tile and qpos(i) = kv_len - qo_len + i, the tile needs
   keys [lo, hi) with hi = min(kv_len, qpos(i_hi)+1) if causal else kv_len,
   lo = max(0, qpos(i_lo) - window + 1) if window > 0 else 0, plus the sink
   range [0, min(sink, lo)) when window > 0 and lo > 0.
   Two tile classes (one launch for a mixed batch): with decode_tile_q > 0,
   a request whose rows fit one decode tile (qo_len * g <= decode_tile_q)
   gets a single unit per kv head of class 1 (the decode tile); every other
   request is tiled by tile_q as above (class 0).  Nothing else changes.
2. Total cost C = sum over units of (hi - lo) + |sink range|.
3. Chunk length L_c = max(min_chunk, roundup(ceil(C*(16+s) / (16*W*split_factor)), tile_kv)),
   then min(L_c, max_chunk) when max_chunk > 0, where the slack s is 1 for
   a plan of 16-row (decode) query tiles only (tile_q == 16) and 0 for any
   other tile_q: decode chunks a sixteenth longer than an even share.
4. Chunks of a unit: with lo_a = lo rounded down to a multiple of tile_kv,
   for k = 0 .. (hi - 1 - lo_a) // L_c the range
   [max(lo, lo_a + k*L_c), min(hi, lo_a + (k+1)*L_c)) (boundaries at lo_a plus
   multiples of L_c: aligned to tile_kv, and a window of n*L_c keys is n
   chunks), then the non-empty sink range as the unit's last chunk.
5. Items are created in unit order (r, h, t ascending), then chunk order;
   item id = creation index; cost = length + item_overhead.  A unit with
   >= 2 chunks gives its items consecutive partial-state slots from a
   global counter; a single-chunk unit's item has slot -1 (writes the
   output directly).
6. Assignment (longest processing time first): items ordered by (cost
   descending, id ascending); a min-heap of (load, worker) starting at
   (0, w); each item pops the minimum (lexicographic), joins that worker's
   list, and (load + cost, worker) is pushed back.
7. Merge table: one entry per unit with >= 2 chunks, in unit order:
   (r, h, row_lo, row_hi, first_slot, n_chunks).
8. Capacities: more than max_items_per_worker items on a worker, more than
   max_slots slots or more than max_merge merge entries is an error.

Composable format with a shared prefix (shared_prefix_len P > 0): every
request's KV sequence is one dense prefix of P tokens shared by the whole
batch, followed by the request's own paged suffix (kv_len counts the suffix
only; the queries are its last tokens, causal within the suffix, and every
prefix token is in every query's past).  The FlashInfer paper summary
[FI-paper, research methodology 1: composable formats] processes the dense
shared part and the sparse per-request parts separately, each at its own
block size, and merges their states; here both parts are units of one plan:

   a. Prefix units first, class 2: for each kv head h and each tile_q tile t
      of the batch's global query rows (request r's rows are the global rows
      qo_indptr[r]*g + [0, qo_len*g)), rows [t*tile_q, min((t+1)*tile_q, T*g))
      with T the total query tokens, keys [0, P); r = -1.
   b. Then the suffix units of the requests, by rules 1-2 (the suffix is a
      normal request of kv_len keys; window and sinks are not used).
   c. Chunks, items and costs by rules 3-5 over all units, except that every
      unit takes partial-state slots (both parts of a row are merged), in unit
      order.
   d. Merge table: one entry per suffix unit, in unit order:
      (r, h, row_lo, row_hi, first_slot, n_chunks, pfx_first, pfx_n), where
      pfx_n is the chunk count of a prefix unit (the same for all) and
      pfx_first the first slot of kv head h's first prefix unit.  Row rr of
      the entry is global row R = qo_indptr[r]*g + row_lo + rr; its prefix
      partials are row R mod tile_q of slots pfx_first + (R div tile_q)*pfx_n
      + c, c < pfx_n.  Without a prefix the last two fields are 0.

Pinned by: the partition covers every (unit, visible key) exactly once,
chunk starts fall on lo_a plus multiples of L_c, the LPT makespan bound, greedy
optimality of each step, and a committed golden plan (tests).
"""
from __future__ import annotations

import dataclasses
import heapq

import numpy as np


class PlanError(Exception):
    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


@dataclasses.dataclass
class PlanParams:
    num_qo_heads: int
    num_kv_heads: int
    tile_q: int
    tile_kv: int
    num_workers: int
    split_factor: int
    min_chunk: int
    max_chunk: int
    item_overhead: int
    max_items_per_worker: int
    max_slots: int
    max_merge: int
    causal: bool = False
    window: int = 0
    sink: int = 0
    decode_tile_q: int = 0  # > 0: requests with qo_len * g <= decode_tile_q use one decode-class tile
    shared_prefix_len: int = 0  # > 0: a dense prefix of this many tokens shared by every request (composable)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan_ref(qo_len, kv_len, p: PlanParams) -> dict:
    qo_len = [int(x) for x in qo_len]
    kv_len = [int(x) for x in kv_len]
    if p.num_kv_heads <= 0 or p.num_qo_heads % p.num_kv_heads:
        raise PlanError("INVALID_ARG", "num_qo_heads must be a positive multiple of num_kv_heads")
    g = p.num_qo_heads // p.num_kv_heads
    for Q, L in zip(qo_len, kv_len):
        if Q < 0 or L < 0 or Q > L:
            raise PlanError("INVALID_ARG", "need 0 <= qo_len <= kv_len")
    W = p.num_workers

    P = p.shared_prefix_len
    if P < 0 or (P > 0 and p.window > 0):
        raise PlanError("INVALID_ARG", "a shared prefix needs prefix length >= 0 and no sliding window")
    units = []  # (r, h, row_lo, row_hi, lo, hi, sink_hi)
    unit_class = []
    if P > 0:
        T = sum(qo_len)
        for h in range(p.num_kv_heads):
            for t in range(_ceil_div(T * g, p.tile_q)):
                units.append((-1, h, t * p.tile_q, min(T * g, (t + 1) * p.tile_q), 0, P, 0))
                unit_class.append(2)
    n_prefix_units = len(units)
    for r, (Q, L) in enumerate(zip(qo_len, kv_len)):
        if Q == 0 or L == 0:
            continue
        rows = Q * g
        small = p.decode_tile_q > 0 and rows <= p.decode_tile_q
        tq = p.decode_tile_q if small else p.tile_q
        for h in range(p.num_kv_heads):
            for t in range(_ceil_div(rows, tq)):
                row_lo = t * tq
                row_hi = min(rows, (t + 1) * tq)
                unit_class.append(1 if small else 0)
                i_lo, i_hi = row_lo // g, (row_hi - 1) // g
                qpos_lo, qpos_hi = L - Q + i_lo, L - Q + i_hi
                hi = min(L, qpos_hi + 1) if p.causal else L
                lo = max(0, qpos_lo - p.window + 1) if p.window > 0 else 0
                sink_hi = min(p.sink, lo) if (p.window > 0 and lo > 0) else 0
                units.append((r, h, row_lo, row_hi, lo, hi, sink_hi))

    C = sum((hi - lo) + sink_hi for (_, _, _, _, lo, hi, sink_hi) in units)
    s = 1 if p.tile_q == 16 else 0
    Lc = max(p.min_chunk, _ceil_div(_ceil_div(C * (16 + s), 16 * W * p.split_factor), p.tile_kv) * p.tile_kv)
    if p.max_chunk > 0:
        Lc = min(Lc, p.max_chunk)

    items = []   # (r, h, row_lo, row_hi, kv_lo, kv_hi, slot)
    item_class = []
    merges = []  # (r, h, row_lo, row_hi, first_slot, n, pfx_first, pfx_n)
    next_slot = 0
    prefix_first = {}  # kv head -> first slot of its first prefix unit
    pfx_n = 0
    for u, (r, h, row_lo, row_hi, lo, hi, sink_hi) in enumerate(units):
        lo_a = lo // p.tile_kv * p.tile_kv
        chunks = [(max(lo, lo_a + k * Lc), min(hi, lo_a + (k + 1) * Lc)) for k in range((hi - 1 - lo_a) // Lc + 1)]
        if sink_hi > 0:
            chunks.append((0, sink_hi))
        if len(chunks) >= 2 or P > 0:
            first = next_slot
            next_slot += len(chunks)
            if u < n_prefix_units:
                prefix_first.setdefault(h, first)
                pfx_n = len(chunks)
            elif P > 0:
                merges.append((r, h, row_lo, row_hi, first, len(chunks), prefix_first[h], pfx_n))
            else:
                merges.append((r, h, row_lo, row_hi, first, len(chunks), 0, 0))
            for c, (a, b) in enumerate(chunks):
                items.append((r, h, row_lo, row_hi, a, b, first + c))
                item_class.append(unit_class[u])
        else:
            a, b = chunks[0]
            items.append((r, h, row_lo, row_hi, a, b, -1))
            item_class.append(unit_class[u])

    cost = [(it[5] - it[4]) + p.item_overhead for it in items]
    order = sorted(range(len(items)), key=lambda i: (-cost[i], i))
    heap = [(0, w) for w in range(W)]
    heapq.heapify(heap)
    worker_items = [[] for _ in range(W)]
    load = [0] * W
    for i in order:
        ld, w = heapq.heappop(heap)
        worker_items[w].append(i)
        load[w] = ld + cost[i]
        heapq.heappush(heap, (load[w], w))

    if any(len(x) > p.max_items_per_worker for x in worker_items):
        raise PlanError("CAPACITY", "too many items on one worker")
    if next_slot > p.max_slots:
        raise PlanError("CAPACITY", "too many partial-state slots")
    if len(merges) > p.max_merge:
        raise PlanError("CAPACITY", "too many merge entries")

    return {
        "group": g,
        "units": np.asarray(units, dtype=np.int64).reshape(-1, 7),
        "total_cost": C,
        "chunk": Lc,
        "items": np.asarray(items, dtype=np.int64).reshape(-1, 7),
        "item_class": np.asarray(item_class, dtype=np.int64),
        "cost": np.asarray(cost, dtype=np.int64),
        "worker_items": worker_items,
        "load": np.asarray(load, dtype=np.int64),
        "merge": np.asarray(merges, dtype=np.int64).reshape(-1, 8),
        "num_slots": next_slot,
    }
