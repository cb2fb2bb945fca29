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
        if (rec[bsk::IT_KV_LO] >= rec[bsk::IT_KV_HI] || rec[bsk::IT_KV_HI] > kv[rec[bsk::IT_R]])
          return std::printf("bad range\n"), 1;
        if (rec[bsk::IT_SLOT] >= st.num_slots) return std::printf("bad slot\n"), 1;
        if (rec[bsk::IT_KV_HI] - rec[bsk::IT_KV_LO] > st.chunk) return std::printf("chunk too long\n"), 1;
      }
    }
  }
  std::printf("ok %d planned\n", planned);
  return 0;
}
