// Int-workspace layout shared by the host planner and the device kernels.
//
// The plan lives in one int32 buffer that is built on the host and copied
// to the device in a single transfer.  Everything a run needs per step is
// in it, so the kernels' launch arguments never change between plans (the
// launches can be captured in a graph once and replayed).
//
//   [0, HDR_WORDS)            header (HDR_* indices below)
//   [HDR_WORDS, +W+1)         worker_ptr: items of worker w are
//                             items[worker_ptr[w] .. worker_ptr[w+1])
//   [hdr[HDR_OFF_ITEMS], ...) items, ITEM_WORDS int32 each, worker-major,
//                             each worker's items in assignment order
//   [hdr[HDR_OFF_MERGE], ...) merge table, MERGE_WORDS int32 each
//   [hdr[HDR_OFF_QO], ...)    qo_indptr[batch+1]
//   [hdr[HDR_OFF_KVLEN], ...) kv_len[batch]
//   [hdr[HDR_OFF_KVIND], ...) kv_indptr[batch+1] (page offsets or dense token offsets)
//   [hdr[HDR_OFF_SLOTMAP], ...) slot_merge[num_slots]: merge entry of each partial slot
//   [hdr[HDR_OFF_COUNT], ...) arrivals[num_merge]: chunks of each split unit that have
//                             finished in the current run; zero in the uploaded plan and
//                             reset to zero by the chunk that completes the unit
#pragma once

namespace bsk {

enum : int {
  HDR_NUM_ITEMS = 0,
  HDR_NUM_MERGE = 1,
  HDR_NUM_SLOTS = 2,
  HDR_NUM_WORKERS = 3,
  HDR_BATCH = 4,
  HDR_CHUNK = 5,
  HDR_TILE_Q = 6,
  HDR_OFF_ITEMS = 7,
  HDR_OFF_MERGE = 8,
  HDR_OFF_QO = 9,
  HDR_OFF_KVLEN = 10,
  HDR_OFF_KVIND = 11,
  HDR_MAX_KV_LEN = 12,
  HDR_MAX_QO_LEN = 13,
  HDR_OFF_SLOTMAP = 14,
  HDR_OFF_COUNT = 15,
  HDR_WORDS = 16,
};

// item record (64 bytes: one scalar load brings everything a worker needs to start the item)
enum : int {
  IT_R = 0,       // request
  IT_H = 1,       // kv head
  IT_ROW_LO = 2,  // first query row (row = token * g + group member)
  IT_ROW_HI = 3,  // one past the last row
  IT_KV_LO = 4,   // first key
  IT_KV_HI = 5,   // one past the last key
  IT_SLOT = 6,    // partial-state slot, or -1: write the output directly
  IT_ID = 7,      // creation index
  IT_Q0 = 8,      // the request's qo_indptr[r]: its first query token
  IT_QLEN = 9,    // the request's query length
  IT_KVLEN = 10,  // the request's kv_len
  IT_KBASE = 11,  // the request's kv_indptr[r]: first page (paged) or token (dense) offset
  IT_CLASS = 12,  // tile class: 0 = the plan's tile_q, 1 = the decode tile (mixed launches),
                  // 2 = the shared dense prefix (r = -1; rows are the batch's global query rows)
  ITEM_WORDS = 16,  // words 13..15 are zero
};

// merge record
enum : int {
  MG_R = 0,
  MG_H = 1,
  MG_ROW_LO = 2,
  MG_ROW_HI = 3,
  MG_FIRST_SLOT = 4,
  MG_N = 5,
  MG_PFX_FIRST = 6,  // shared prefix: first slot of this kv head's first prefix unit
  MG_PFX_N = 7,      // shared prefix: chunks per prefix unit (0: no prefix part)
  MERGE_WORDS = 8,
};

}  // namespace bsk
