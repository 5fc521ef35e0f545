// Host-only fuzz driver of the planner (build_host_plan, block_table_csr),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// test_planner_sanitized.py. Random parameters and page tables, valid and
// invalid; for every accepted plan it checks what the decode kernel relies
// on: the units of each (request, kv head) tile the attended tokens
// [start, kv_len) in chunk order, workspace slots are distinct and counted,
// every item field is in range, and a graph plan whose capacity is the
// table's page count would hold the plan. Prints "ok <plans> <rejected>" and exits
// 0, or names the first violation and exits 1.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pkd_internal.h"

namespace {

int check(const pkd_plan_params& p, const std::vector<int32_t>& indptr,
          const std::vector<int32_t>& last, const pkd::HostPlan& h) {
  // heads of the items: each kv head once per block of its query heads
  const int B = p.batch_size, H = p.num_kv_heads * h.kv_blocks, P = p.page_size;
  const int Q = p.q_len_per_req > 1 ? p.q_len_per_req : 1;
  // expected[i][h]: next token the units must start at, per (request, head)
  std::vector<std::vector<int64_t>> next(B, std::vector<int64_t>(H, -1));
  std::vector<std::vector<int>> chunks(B, std::vector<int>(H, 0));
  std::vector<int64_t> kv(B), start(B);
  for (int i = 0; i < B; ++i) {
    kv[i] = (int64_t)P * (indptr[i + 1] - indptr[i] - 1) + last[i];
    start[i] = p.window_left < 0 ? 0 : std::max<int64_t>(0, kv[i] - Q - p.window_left);
  }
  std::vector<int> slot_used(h.info.num_partials, 0);
  // units of a request and head, sorted by chunk (items are in launch order)
  std::vector<std::vector<std::vector<const pkd_work_item*>>> by(
      B, std::vector<std::vector<const pkd_work_item*>>(H));
  if ((int)h.items.size() != h.info.num_items) return fprintf(stderr, "num_items\n"), 1;
  for (const auto& it : h.items) {
    if (it.request < 0 || it.request >= B || it.kv_head < 0 || it.kv_head >= H)
      return fprintf(stderr, "item request/head out of range\n"), 1;
    if (it.num_chunks < 1 || it.chunk < 0 || it.chunk >= it.num_chunks)
      return fprintf(stderr, "chunk %d of %d\n", it.chunk, it.num_chunks), 1;
    if (it.token_begin < 0 || it.token_begin >= it.token_end || it.token_end > kv[it.request])
      return fprintf(stderr, "token range [%d, %d) of kv_len %lld\n", it.token_begin,
                     it.token_end, (long long)kv[it.request]), 1;
    if (it.page_base != indptr[it.request]) return fprintf(stderr, "page_base\n"), 1;
    if (it.query_pos != kv[it.request] - Q) return fprintf(stderr, "query_pos\n"), 1;
    if ((it.num_chunks == 1) != (it.partial < 0)) return fprintf(stderr, "partial\n"), 1;
    if (it.partial >= 0) {
      if (it.partial >= h.info.num_partials) return fprintf(stderr, "slot range\n"), 1;
      ++slot_used[it.partial];
    }
    by[it.request][it.kv_head].push_back(&it);
  }
  for (int i = 0; i < B; ++i)
    for (int hh = 0; hh < H; ++hh) {
      auto& v = by[i][hh];
      if (v.empty()) return fprintf(stderr, "request %d head %d has no unit\n", i, hh), 1;
      std::vector<const pkd_work_item*> o(v.size(), nullptr);
      for (auto* it : v) {
        if (it->num_chunks != (int)v.size() || o[it->chunk] != nullptr)
          return fprintf(stderr, "chunks of request %d\n", i), 1;
        o[it->chunk] = it;
      }
      int64_t t = start[i];
      for (size_t c = 0; c < o.size(); ++c) {
        if (o[c]->token_begin != t) return fprintf(stderr, "gap or overlap in request %d\n", i), 1;
        if (c > 0 && o[c]->partial != o[c - 1]->partial + 1)
          return fprintf(stderr, "slots of request %d not consecutive\n", i), 1;
        t = o[c]->token_end;
      }
      if (t != kv[i]) return fprintf(stderr, "request %d ends at %lld\n", i, (long long)t), 1;
    }
  for (int s = 0; s < h.info.num_partials; ++s)
    if (slot_used[s] != H) return fprintf(stderr, "slot %d used %d times\n", s, slot_used[s]), 1;
  if (h.steal_limit < 0 || h.steal_limit > h.info.num_items) return fprintf(stderr, "steal\n"), 1;
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 2000;
  std::mt19937_64 rng(argc > 2 ? atoll(argv[2]) : 1);
  auto U = [&](int lo, int hi) { return (int)std::uniform_int_distribution<int>(lo, hi)(rng); };
  int plans = 0, rejected = 0;
  for (int n = 0; n < iters; ++n) {
    pkd_plan_params p{};
    p.batch_size = U(0, 40);
    p.num_kv_heads = U(1, 8);
    p.num_qo_heads = p.num_kv_heads * (U(0, 9) == 0 ? U(1, 40) : U(1, 8));
    const int hds[3] = {64, 128, 256};
    p.head_dim = U(0, 19) == 0 ? U(1, 300) : hds[U(0, 2)];
    p.page_size = U(0, 19) == 0 ? U(0, 300) : 1 << U(0, 6);
    p.layout = U(0, 1);
    p.q_dtype = U(0, 1);
    p.kv_dtype = U(0, 3) == 0 ? PKD_E4M3 : p.q_dtype;
    p.o_dtype = p.q_dtype;
    p.sm_scale = 0.1f;
    p.window_left = U(0, 3) == 0 ? U(-2, 3000) : -1;
    p.fixed_split_size = U(0, 3) == 0 ? U(-1, 40) : 0;
    p.disable_split_kv = U(0, 9) == 0;
    p.q_len_per_req = U(0, 3) == 0 ? U(-1, 6) : 0;
    p.pos_encoding_mode = U(0, 9) == 0 ? U(-1, 3) : 0;
    p.rope_scale = 1.0f;
    p.rope_theta = 1e4f;
    const int B = std::max(0, p.batch_size);
    const int Ps = std::max(1, p.page_size);
    std::vector<int32_t> indptr(B + 1, 0), last(B, 1), seq(B, 1);
    const int maxlen = U(0, 2) == 0 ? 200000 : 5000;
    for (int i = 0; i < B; ++i) {
      const int L = U(0, 49) == 0 ? U(-2, 3) : U(1, maxlen);
      seq[i] = L;
      const int np = L >= 1 ? (L + Ps - 1) / Ps : U(0, 1);
      indptr[i + 1] = indptr[i] + np;
      last[i] = L >= 1 ? L - Ps * (np - 1) : U(-1, Ps + 1);
    }
    const int slots = U(0, 9) == 0 ? U(0, 4) : 256 * U(1, 3);
    pkd::HostPlan h;
    pkd_status st;
    std::vector<int32_t> ip2, last2, base2;
    if (U(0, 3) == 0) {
      // block-table input: CSR counts from seq_lens, then the planner
      const int maxb = U(0, 9) == 0 ? U(0, 3) : (maxlen + Ps - 1) / Ps + U(0, 5);
      st = pkd::block_table_csr(p, seq.data(), maxb, &ip2, &last2, &base2);
      if (st == PKD_OK) {
        st = pkd::build_host_plan(p, ip2.data(), last2.data(), slots, &h, base2.data());
        if (st == PKD_OK) {
          // page_base is i * max_blocks here: check the tiling with the CSR
          // counts, then the bases themselves
          for (auto& it : h.items) {
            if (it.page_base != base2[it.request]) return fprintf(stderr, "block base\n"), 1;
            it.page_base = ip2[it.request];
          }
          if (check(p, ip2, last2, h)) return fprintf(stderr, "iteration %d\n", n), 1;
          ++plans;
          continue;
        }
      }
    } else {
      st = pkd::build_host_plan(p, indptr.data(), last.data(), slots, &h);
      if (st == PKD_OK) {
        if (check(p, indptr, last, h)) return fprintf(stderr, "iteration %d\n", n), 1;
        // a graph plan with a capacity of this table's pages holds the plan
        int64_t tot = 0, one = 0, most = 0;
        pkd::graph_capacities(p, indptr[B], std::max(1, slots), &tot, &one);
        for (const auto& it : h.items) most = std::max<int64_t>(most, it.num_chunks);
        const int heads = p.num_kv_heads * h.kv_blocks;
        if (h.kv_blocks != pkd::kv_blocks(p) ||
            (int64_t)(p.num_qo_heads / heads) * (p.q_len_per_req > 1 ? p.q_len_per_req : 1) > 16 ||
            p.num_qo_heads % heads != 0)
          return fprintf(stderr, "kv_blocks %d (iteration %d)\n", h.kv_blocks, n), 1;
        if ((int64_t)h.items.size() > tot * heads || most > one)
          return fprintf(stderr, "graph capacity %lld x %d heads / %lld below %zu items / %lld "
                         "chunks (iteration %d)\n", (long long)tot, heads,
                         (long long)one, h.items.size(), (long long)most, n), 1;
        ++plans;
        continue;
      }
    }
    if (st == PKD_OK) return fprintf(stderr, "unreachable\n"), 1;
    if (pkd_last_error()[0] == 0) return fprintf(stderr, "rejection without a message\n"), 1;
    ++rejected;
  }
  printf("ok %d %d\n", plans, rejected);
  return 0;
}
