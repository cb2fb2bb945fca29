"""Decode the int-workspace plan written by bsk_plan (layout documented in
block_sparse_kv_plan_amd/csrc/layout.h).  Test infrastructure only."""
import numpy as np

HDR_WORDS = 16
ITEM_WORDS = 16  # 8 plan fields, 4 copied request fields (q0, qo_len, kv_len, kv_indptr), tile class, 3 zero
MERGE_WORDS = 8


def decode(buf) -> dict:
    w = np.frombuffer(np.asarray(buf).tobytes(), dtype=np.int32)
    n_items, n_merge, n_slots, W, batch, chunk, tile_q = (int(x) for x in w[:7])
    off_items, off_merge, off_qo, off_kvlen, off_kvind = (int(x) for x in w[7:12])
    wptr = w[HDR_WORDS:HDR_WORDS + W + 1]
    items = w[off_items:off_items + n_items * ITEM_WORDS].reshape(-1, ITEM_WORDS)
    merge = w[off_merge:off_merge + n_merge * MERGE_WORDS].reshape(-1, MERGE_WORDS)
    return {
        "num_items": n_items, "num_merge": n_merge, "num_slots": n_slots, "W": W, "batch": batch, "chunk": chunk,
        "tile_q": tile_q, "max_kv_len": int(w[12]), "max_qo_len": int(w[13]),
        "worker_items": [items[wptr[k]:wptr[k + 1], :8] for k in range(W)],
        "worker_req": [items[wptr[k]:wptr[k + 1], 8:12] for k in range(W)],
        "worker_class": [items[wptr[k]:wptr[k + 1], 12] for k in range(W)],
        "item_pad": items[:, 13:],
        "merge": merge,
        "qo_indptr": w[off_qo:off_qo + batch + 1], "kv_len": w[off_kvlen:off_kvlen + batch],
        "kv_indptr": w[off_kvind:off_kvind + batch + 1],
        "slot_merge": w[int(w[14]):int(w[14]) + n_slots],
        "arrivals": w[int(w[15]):int(w[15]) + n_merge],
    }
