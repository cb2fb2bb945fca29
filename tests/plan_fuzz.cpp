// Host-only driver for the planner, built with g++ and host sanitizers by
// tests/test_plan.py: random lengths and parameters, every plan checked for
// consistency (each worker's items inside the buffer, slots in range).
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "layout.h"
#include "plan.h"

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 100;
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int planned = 0;
  for (int it = 0; it < iters; ++it) {
    bsk::PlanParams p;
    p.num_kv_heads = uni(1, 8);
    p.num_qo_heads = p.num_kv_heads * uni(1, 8);
    p.tile_q = uni(0, 1) ? 16 : 128;
    p.tile_kv = 16 << uni(0, 2);
    p.num_workers = uni(1, 300);
    p.split_factor = uni(1, 4);
    p.min_chunk = p.tile_kv * uni(1, 4);
    p.max_chunk = uni(0, 1) ? 0 : p.min_chunk * uni(1, 8);
    p.item_overhead = uni(0, 50);
    p.max_batch = 64;
    p.max_items_per_worker = uni(1, 64);
    p.max_slots = uni(0, 5000);
    p.max_merge = uni(0, 3000);
    p.causal = uni(0, 1);
    p.window = uni(0, 2) ? 0 : uni(1, 4000);
    p.sink = uni(0, 8);
    if (uni(0, 3) == 0) {  // composable batch: a shared dense prefix before every request's pages
      p.tile_q = 128;
      p.decode_tile_q = 16;
      p.window = 0;
      p.shared_prefix_len = uni(1, 50000);
    }
    const int B = uni(0, p.max_batch);
    std::vector<int32_t> qo(B + 1, 0), kv(B), ki(B + 1, 0);
    for (int r = 0; r < B; ++r) {
      kv[r] = uni(0, 20000);
      qo[r + 1] = qo[r] + std::min(kv[r], uni(0, 300));
      ki[r + 1] = ki[r] + (kv[r] + 15) / 16;
    }
    std::vector<int32_t> buf(bsk::plan_workspace_bytes(p) / 4 + 1);
    bsk::PlanStats st;
    std::string err;
    const bsk::PlanResult res = bsk::build_plan(p, B, qo.data(), kv.data(), ki.data(), buf.data(), buf.size() * 4,
                                                &st, &err);
    if (res != bsk::PLAN_OK) continue;
    ++planned;
    const int32_t* wptr = buf.data() + bsk::HDR_WORDS;
    const int32_t* items = buf.data() + buf[bsk::HDR_OFF_ITEMS];
    if (wptr[p.num_workers] != st.num_items) return std::printf("bad worker_ptr\n"), 1;
    for (int w = 0; w < p.num_workers; ++w) {
      for (int i = wptr[w]; i < wptr[w + 1]; ++i) {
        const int32_t* rec = items + int64_t(i) * bsk::ITEM_WORDS;
        const int32_t r = rec[bsk::IT_R];
        const int32_t len = r >= 0 ? kv[r] : p.shared_prefix_len;
        if ((r < 0) != (rec[bsk::IT_CLASS] == 2) || (r < 0 && p.shared_prefix_len == 0))
          return std::printf("bad prefix item\n"), 1;
        if (rec[bsk::IT_KV_LO] >= rec[bsk::IT_KV_HI] || rec[bsk::IT_KV_HI] > len)
          return std::printf("bad range\n"), 1;
        if (r < 0 && (rec[bsk::IT_ROW_HI] > rec[bsk::IT_QLEN] * (p.num_qo_heads / p.num_kv_heads) ||
                      rec[bsk::IT_SLOT] < 0))
          return std::printf("bad prefix rows\n"), 1;
        if (rec[bsk::IT_SLOT] >= st.num_slots) return std::printf("bad slot\n"), 1;
        if (rec[bsk::IT_KV_HI] - rec[bsk::IT_KV_LO] > st.chunk) return std::printf("chunk too long\n"), 1;
      }
    }
    // merge records: every chunk slot named (suffix and prefix parts) lies inside the plan's slots
    const int32_t* merge = buf.data() + buf[bsk::HDR_OFF_MERGE];
    const int32_t g = p.num_qo_heads / p.num_kv_heads;
    for (int m = 0; m < st.num_merge; ++m) {
      const int32_t* rec = merge + int64_t(m) * bsk::MERGE_WORDS;
      if (rec[bsk::MG_FIRST_SLOT] < 0 || rec[bsk::MG_FIRST_SLOT] + rec[bsk::MG_N] > st.num_slots)
        return std::printf("bad merge slots\n"), 1;
      if (rec[bsk::MG_PFX_N] > 0) {
        const int64_t last_row = int64_t(qo[rec[bsk::MG_R]]) * g + rec[bsk::MG_ROW_HI] - 1;
        const int64_t last = rec[bsk::MG_PFX_FIRST] + (last_row / p.tile_q + 1) * rec[bsk::MG_PFX_N];
        if (rec[bsk::MG_PFX_FIRST] < 0 || last > st.num_slots) return std::printf("bad prefix slots\n"), 1;
      }
    }
  }
  std::printf("ok %d planned\n", planned);
  return 0;
}
