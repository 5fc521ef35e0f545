// Host planner of the paged-KV batch decode: validation of the CSR page table,
// choice of the split size and construction of the work list.
//
// plan() of flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper ("FlashInfer
// attention kernels" page) builds auxiliary structures once and reuses them
// for every run() of the same batch (the note under the class example). This
// is that step: everything here is host work; the result is uploaded once.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "pkd_internal.h"

namespace pkd {

namespace {
thread_local std::string g_error;

std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Per request: attended token range and page count.
struct Req {
  int32_t kv_len;
  int32_t start;   // first attended token (window start)
  int32_t pages;   // pages of the request
};

// Number of chunks of `split` pages that hold attended tokens.
int64_t chunks_of(const Req& r, int32_t split, int32_t page_size) {
  if (split <= 0) return 1;
  int64_t first = (int64_t)(r.start / page_size) / split;
  int64_t last = (int64_t)(r.pages - 1) / split;
  return last - first + 1;
}

// Work units per workgroup the planner aims for when it chooses the split:
// enough for the longest-first assignment to even out the workgroups. It
// aims for fewer when a unit carries more than kSplitRowsRef query rows
// (G * q_len_per_req): every unit of a split request writes a partial state
// of rows x head_dim fp32 values and the merge reads it back, so the cost of
// a split grows with the rows (16 rows: no split at all in the serving batch
// with four query tokens, 117.5 -> 109.7 us per call; E4M3 KV with 8 rows:
// unchanged within 1 us).
constexpr int kUnitsPerWorkgroup = 4;
constexpr int kSplitRowsRef = 4;
// Units the planner sizes itself are multiples of this many tokens: two steps
// for each wavefront of a workgroup, so that every wavefront runs an even
// number of steps (its loop takes steps in pairs).
constexpr int kUnitQuantum = kUnitQuantumTokens;
// Smallest unit the planner creates on its own, in tokens, except for a batch
// too small to fill the workgroups with such units: there the quantum is one
// step for each wavefront.
constexpr int kMinUnitTokens = kUnitQuantum;
constexpr int kSmallUnitQuantum = kWaves * kStepTokens;
// Under a fixed split, chunks longer than this are processed as sub-chunks of
// this many tokens (cut at fixed offsets from the chunk start), so that the
// work can be spread over all workgroups. The cut depends only on the
// request's own length, so results stay batch invariant. A chunk of 4096
// tokens becomes a unit of 3072 and one of 1024: the short units, taken
// last, even out the workgroups' ends better than two units of 2048.
constexpr int kMaxUnitTokens = kFixedUnitMaxTokens;

}  // namespace

pkd_status fail(pkd_status st, const std::string& msg) {
  g_error = msg;
  return st;
}
void clear_error() { g_error.clear(); }

}  // namespace pkd

extern "C" const char* pkd_last_error(void) { return pkd::g_error.c_str(); }

namespace pkd {

pkd_status check_params(const pkd_plan_params& p) {
  if (p.batch_size < 0)
    return fail(PKD_EINVAL, fmt("batch_size %d < 0", p.batch_size));
  if (p.num_qo_heads < 1 || p.num_kv_heads < 1)
    return fail(PKD_EINVAL, fmt("num_qo_heads %d / num_kv_heads %d must be >= 1",
                                p.num_qo_heads, p.num_kv_heads));
  if (p.num_qo_heads % p.num_kv_heads != 0)
    return fail(PKD_EINVAL,
                fmt("num_qo_heads %d is not a multiple of num_kv_heads %d",
                    p.num_qo_heads, p.num_kv_heads));
  if (p.pos_encoding_mode == PKD_POS_ROPE_LLAMA) {
    if (!(p.rope_scale > 0.0f) || !std::isfinite(p.rope_scale) || !(p.rope_theta > 0.0f) ||
        !std::isfinite(p.rope_theta))
      return fail(PKD_EINVAL, fmt("rope_scale %g and rope_theta %g must be positive and finite",
                                  p.rope_scale, p.rope_theta));
  }
  if (p.pos_encoding_mode != PKD_POS_NONE && p.pos_encoding_mode != PKD_POS_ALIBI &&
      p.pos_encoding_mode != PKD_POS_ROPE_LLAMA)
    return fail(PKD_EINVAL, fmt("pos_encoding_mode %d is not NONE (0), ROPE_LLAMA (1) or ALIBI (2)",
                                p.pos_encoding_mode));
  if (p.q_len_per_req < 0)
    return fail(PKD_EINVAL, fmt("q_len_per_req %d < 0", p.q_len_per_req));
  if (q_len_of(p) > kMaxGroup)
    return fail(PKD_EUNSUPPORTED,
                fmt("q_len_per_req %d exceeds %d query rows per kv head", q_len_of(p),
                    kMaxGroup));
  if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256)
    return fail(PKD_EUNSUPPORTED,
                fmt("head_dim %d not in {64, 128, 256}", p.head_dim));
  if (!is_pow2(p.page_size) || p.page_size > 256)
    return fail(PKD_EUNSUPPORTED,
                fmt("page_size %d is not a power of two in [1, 256]",
                    p.page_size));
  if (p.layout != PKD_NHD && p.layout != PKD_HND)
    return fail(PKD_EINVAL, fmt("layout %d is neither NHD (0) nor HND (1)",
                                p.layout));
  if (p.q_dtype != PKD_F16 && p.q_dtype != PKD_BF16)
    return fail(PKD_EUNSUPPORTED, fmt("q_dtype %d not in {F16, BF16}", p.q_dtype));
  if (p.kv_dtype != p.q_dtype && p.kv_dtype != PKD_E4M3)
    return fail(PKD_EUNSUPPORTED,
                fmt("kv_dtype %d must equal q_dtype %d or be E4M3", p.kv_dtype,
                    p.q_dtype));
  if (p.o_dtype != PKD_F16 && p.o_dtype != PKD_BF16)
    return fail(PKD_EUNSUPPORTED, fmt("o_dtype %d not in {F16, BF16}", p.o_dtype));
  if (!std::isfinite(p.sm_scale))
    return fail(PKD_EINVAL, "sm_scale is not finite");
  if (std::isnan(p.logits_soft_cap) || std::isinf(p.logits_soft_cap))
    return fail(PKD_EINVAL, "logits_soft_cap is not finite");
  if (p.window_left < -1)
    return fail(PKD_EINVAL, fmt("window_left %d < -1", p.window_left));
  if (p.fixed_split_size < 0)
    return fail(PKD_EINVAL, fmt("fixed_split_size %d < 0", p.fixed_split_size));
  if (p.fixed_split_size > 0 && p.disable_split_kv)
    return fail(PKD_EINVAL,
                "fixed_split_size and disable_split_kv are mutually exclusive");
  return PKD_OK;
}

int32_t kv_blocks(const pkd_plan_params& p) {
  const int32_t G = p.num_qo_heads / p.num_kv_heads, Q = q_len_of(p);
  for (int32_t nb = 1; nb < G; ++nb)
    if (G % nb == 0 && (int64_t)(G / nb) * Q <= kMaxGroup) return nb;
  return G;
}

int32_t decode_wgs_per_cu_table(const pkd_plan_params& p) {
  return decode_waves_per_simd(p.head_dim, p.kv_dtype == PKD_E4M3,
                               p.pos_encoding_mode == PKD_POS_ROPE_LLAMA, decode_single(p));
}

size_t workspace_lse_offset(int32_t num_partials, int32_t num_qo_heads,
                            int32_t head_dim) {
  size_t o_bytes = (size_t)num_partials * num_qo_heads * head_dim * 4;
  return (o_bytes + 255) & ~(size_t)255;
}

pkd_status block_table_csr(const pkd_plan_params& p, const int32_t* seq_lens,
                           int32_t max_blocks, std::vector<int32_t>* indptr,
                           std::vector<int32_t>* last_page_len,
                           std::vector<int32_t>* page_base) {
  const int32_t B = p.batch_size;
  if (B > 0 && seq_lens == nullptr) return fail(PKD_EINVAL, "seq_lens must not be NULL");
  if (max_blocks < 1)
    return fail(PKD_EINVAL, fmt("max_blocks_per_seq %d < 1", max_blocks));
  if ((int64_t)B * max_blocks > INT32_MAX)
    return fail(PKD_EUNSUPPORTED, fmt("block table of %d x %d entries exceeds 2^31",
                                      B, max_blocks));
  indptr->assign(B + 1, 0);
  last_page_len->assign(B, 0);
  page_base->assign(B, 0);
  const int64_t P = p.page_size;
  for (int32_t i = 0; i < B; ++i) {
    const int64_t L = seq_lens[i];
    if (L < 1) return fail(PKD_EINVAL, fmt("seq_lens[%d] = %lld < 1", i, (long long)L));
    const int64_t np = (L + P - 1) / P;
    if (np > max_blocks)
      return fail(PKD_EINVAL, fmt("seq_lens[%d] = %lld needs %lld pages > max_blocks_per_seq %d",
                                  i, (long long)L, (long long)np, max_blocks));
    if ((*indptr)[i] + np > INT32_MAX)
      return fail(PKD_EUNSUPPORTED, "more than 2^31 pages in the batch");
    (*indptr)[i + 1] = (*indptr)[i] + (int32_t)np;
    (*last_page_len)[i] = (int32_t)(L - P * (np - 1));
    (*page_base)[i] = i * max_blocks;
  }
  return PKD_OK;
}

pkd_status build_host_plan(const pkd_plan_params& p, const int32_t* indptr,
                           const int32_t* last_page_len, int32_t num_slots,
                           HostPlan* out, const int32_t* page_base) {
  pkd_status st = check_params(p);
  if (st != PKD_OK) return st;
  const int32_t B = p.batch_size;
  // heads of the items: every kv head once per block of its query heads
  const int32_t nb = kv_blocks(p);
  const int32_t H = p.num_kv_heads * nb;
  if (B > 0 && (indptr == nullptr || last_page_len == nullptr))
    return fail(PKD_EINVAL, "indptr / last_page_len must not be NULL");
  if (num_slots < 1) return fail(PKD_EINVAL, fmt("num_slots %d < 1", num_slots));
  if (B > 0 && indptr[0] != 0)
    return fail(PKD_EINVAL, fmt("indptr[0] = %d, must be 0", indptr[0]));

  const int32_t P = p.page_size;
  const int32_t Q = q_len_of(p);
  std::vector<Req> reqs(B);
  int64_t attended = 0;
  int32_t max_pages = 0;
  for (int32_t i = 0; i < B; ++i) {
    const int64_t np = (int64_t)indptr[i + 1] - indptr[i];
    if (np < 1)
      return fail(PKD_EINVAL,
                  fmt("request %d has %lld pages (indptr[%d]=%d, indptr[%d]=%d); "
                      "every request needs at least one page",
                      i, (long long)np, i, indptr[i], i + 1, indptr[i + 1]));
    const int32_t last = last_page_len[i];
    if (last < 1 || last > P)
      return fail(PKD_EINVAL, fmt("last_page_len[%d] = %d outside [1, page_size=%d]",
                                  i, last, P));
    const int64_t L = (int64_t)P * (np - 1) + last;
    if (L > INT32_MAX / 2)
      return fail(PKD_EUNSUPPORTED,
                  fmt("request %d has kv_len %lld > %d", i, (long long)L,
                      INT32_MAX / 2));
    if (p.pos_encoding_mode == PKD_POS_ROPE_LLAMA && L > (1 << 24))
      return fail(PKD_EUNSUPPORTED, fmt("request %d has kv_len %lld > 2^24, beyond the exact "
                                        "positions of the rotary angles", i, (long long)L));
    if (L < Q)
      return fail(PKD_EINVAL, fmt("request %d has kv_len %lld < q_len_per_req %d: its "
                                  "first query token would have no position",
                                  i, (long long)L, Q));
    Req r;
    r.kv_len = (int32_t)L;
    // the first query token (position L-Q) has the earliest window start
    r.start = p.window_left < 0 ? 0 : std::max<int32_t>(0, r.kv_len - Q - p.window_left);
    r.pages = (int32_t)np;
    reqs[i] = r;
    attended += r.kv_len - r.start;
    max_pages = std::max(max_pages, r.pages);
  }

  // ---- chunk size, in pages (0 = one chunk per request), and the largest
  // unit in tokens.
  const int64_t slots = std::max<int64_t>(1, num_slots);
  int32_t split = 0;
  int64_t unit_cap = INT64_MAX;
  // the units are the split's chunks on the grid of multiples of the chunk
  // (a fixed split, and the planner's split of a small batch), else equal
  // pieces of each request
  bool grid = p.fixed_split_size > 0;
  if (p.disable_split_kv) {
    split = 0;
  } else if (p.fixed_split_size > 0) {
    split = p.fixed_split_size;
    unit_cap = std::min<int64_t>((int64_t)split * P, kMaxUnitTokens);
  } else if (B > 0) {
    // units of about a kUnitsPerWorkgroup-th of a workgroup's share, so
    // that no single long request decides when the last workgroup ends
    const int64_t rows = (int64_t)(p.num_qo_heads / H) * q_len_of(p);
    const int64_t units_wanted =
        std::max<int64_t>(1, slots * kUnitsPerWorkgroup * kSplitRowsRef /
                                 std::max<int64_t>(kSplitRowsRef, rows));
    {
      const int64_t total = attended * H;
      int64_t quantum = kUnitQuantum, unit;
      if (total <= slots * kUnitQuantum) {
        // A batch too small to give every workgroup a unit of the usual
        // quantum (a launch-bound call: the time is a chain of dependent
        // memory round trips): units of one step per wavefront, no more of
        // them than workgroups, so that as many compute units as possible
        // stream their share at once, cut as a fixed split cuts (whole
        // chunks and a remainder). (The class example's batch, 32 layers:
        // 11.8 us per call with 160 such units; 12.2 us with 160 equal pieces
        // or 96 of at most 256 tokens; 19.5 us with units of 64 tokens, more
        // than the workgroups.)
        quantum = kSmallUnitQuantum;
        unit = std::max<int64_t>(quantum, (total + slots - 1) / slots);
        grid = true;
      } else {
        unit = std::max<int64_t>(kMinUnitTokens, (total + units_wanted - 1) / units_wanted);
      }
      // (with the usual quantum, an even number of steps for every wavefront)
      unit = (unit + quantum - 1) / quantum * quantum;
      int64_t pages_per_unit = (unit + P - 1) / P;
      split = pages_per_unit >= max_pages ? 0 : (int32_t)pages_per_unit;
    }
  }
  if (split > 0 && unit_cap == INT64_MAX) unit_cap = (int64_t)split * P;

  // ---- work units: chunks of `split` pages, cut into sub-chunks of at most
  // unit_cap tokens at offsets from the chunk start
  struct Unit {
    pkd_work_item it;
    int64_t tokens;
  };
  std::vector<Unit> units;
  out->params = p;
  out->kv_blocks = nb;
  out->items.clear();
  out->merges.clear();
  out->max_units = 0;
  int32_t partials = 0;
  for (int32_t i = 0; i < B; ++i) {
    const Req& r = reqs[i];
    // token ranges of this request's units, in order
    std::vector<std::pair<int64_t, int64_t>> ranges;
    if (split <= 0) {
      ranges.emplace_back(r.start, r.kv_len);
    } else if (!grid) {
      // the planner's own split: the attended tokens in the fewest units of
      // at most `split` pages, all of about the same length (units that
      // differ less leave less for the longest-first order to even out)
      const int64_t att = r.kv_len - r.start;
      const int64_t cap = (int64_t)split * P;
      const int64_t n = (att + cap - 1) / cap;
      // The cuts go to the nearest multiple of the kernel's step (steps start
      // at multiples of kStepTokens): a cut inside a step would have both
      // units load that step's rows. Should that make a unit longer than the
      // cap (or empty), the request keeps the exact cuts.
      std::vector<int64_t> cut(n + 1);
      cut[0] = r.start;
      cut[n] = r.kv_len;
      bool aligned = true;
      for (int64_t c = 1; c < n; ++c) {
        const int64_t e = r.start + att * c / n;
        cut[c] = (e + kStepTokens / 2) / kStepTokens * kStepTokens;
      }
      for (int64_t c = 0; c < n && aligned; ++c)
        aligned = cut[c + 1] > cut[c] && cut[c + 1] - cut[c] <= cap;
      for (int64_t c = 0; c < n; ++c) {
        if (aligned)
          ranges.emplace_back(cut[c], cut[c + 1]);
        else
          ranges.emplace_back(r.start + att * c / n, r.start + att * (c + 1) / n);
      }
    } else {
      const int64_t chunk_tokens = (int64_t)split * P;
      const int64_t first = (r.start / P) / split;
      const int64_t nch = chunks_of(r, split, P);
      for (int64_t c = 0; c < nch; ++c) {
        const int64_t cb = (first + c) * chunk_tokens;
        const int64_t ce = std::min<int64_t>(cb + chunk_tokens, r.kv_len);
        for (int64_t sb = cb; sb < ce; sb += unit_cap) {
          const int64_t lo = std::max<int64_t>(sb, r.start);
          const int64_t hi = std::min<int64_t>(sb + unit_cap, ce);
          if (lo < hi) ranges.emplace_back(lo, hi);
        }
      }
    }
    const int64_t n = (int64_t)ranges.size();
    const bool split_req = n > 1;
    out->max_units = std::max<int32_t>(out->max_units, (int32_t)n);
    if (split_req) {
      if ((int64_t)partials + n > INT32_MAX / 2)
        return fail(PKD_EUNSUPPORTED, "too many chunks");
      out->merges.push_back(MergeRow{i, partials, (int32_t)n, 0});
    }
    for (int64_t c = 0; c < n; ++c) {
      for (int32_t h = 0; h < H; ++h) {
        Unit u;
        u.it.request = i;
        u.it.kv_head = h;
        u.it.token_begin = (int32_t)ranges[c].first;
        u.it.token_end = (int32_t)ranges[c].second;
        u.it.page_base = page_base != nullptr ? page_base[i] : indptr[i];
        u.it.partial = split_req ? partials + (int32_t)c : -1;
        u.it.chunk = (int32_t)c;
        u.it.num_chunks = (int32_t)n;
        u.it.query_pos = r.kv_len - Q;
        u.tokens = ranges[c].second - ranges[c].first;
        units.push_back(u);
      }
    }
    if (split_req) partials += (int32_t)n;
    // unit indices are published in 24 bits (the reserve slots)
    if (units.size() >= (size_t)kMaxItems)
      return fail(PKD_EUNSUPPORTED, fmt("more than %u work units", kMaxItems - 1));
  }

  // ---- launch order: longest units first. The decode workgroups take
  // units in this order from a shared counter, so a faster workgroup simply
  // takes more of them. Only the schedule depends on it: each unit's
  // arithmetic depends on its own range alone.
  const int64_t nwg = std::min<int64_t>(slots, (int64_t)units.size());
  // Among equal lengths, requests with more units go first: the last unit of
  // a split request merges all of them, and the short merges then come last.
  std::stable_sort(units.begin(), units.end(), [](const Unit& a, const Unit& b) {
    if (a.tokens != b.tokens) return a.tokens > b.tokens;
    return a.it.num_chunks > b.it.num_chunks;
  });
  out->items.resize(units.size());
  for (size_t k = 0; k < units.size(); ++k) out->items[k] = units[k].it;
  const int64_t token_bytes = 2LL * p.head_dim * (p.kv_dtype == PKD_E4M3 ? 1 : 2);
  out->steal_limit = 0;
  while (out->steal_limit < (int32_t)units.size() &&
         units[out->steal_limit].tokens * token_bytes >= kStealMinBytes)
    ++out->steal_limit;
  // The units held when workgroups start to run out of work are about the
  // last nwg: if none of them is long enough, nothing is published at all.
  if (out->steal_limit <= (int64_t)units.size() - nwg) out->steal_limit = 0;

  // the merge counters are addressed with 32-bit byte offsets
  if ((int64_t)B * H * (1 + (out->max_units + kMergeGroup - 1) / kMergeGroup) * 4 >
      INT32_MAX / 2)
    return fail(PKD_EUNSUPPORTED, "too many split requests for the merge counters");
  // the merge addresses one request's partial states with 32-bit offsets
  if ((int64_t)partials * Q * p.num_qo_heads * p.head_dim * 4 > INT32_MAX)
    return fail(PKD_EUNSUPPORTED, fmt("%d partial states of %d query rows x %d exceed the "
                                      "2 GiB workspace limit",
                                      partials, Q * p.num_qo_heads, p.head_dim));
  pkd_plan_info& info = out->info;
  info.num_items = (int32_t)out->items.size();
  info.num_workgroups = (int32_t)nwg;
  info.workgroups_per_cu = decode_wgs_per_cu_table(p);
  info.num_split_requests = (int32_t)out->merges.size();
  info.num_partials = partials;
  info.split_pages = split;
  info.attended_tokens = attended;
  info.workspace_bytes =
      partials == 0
          ? 0
          : workspace_lse_offset(partials, Q * p.num_qo_heads, p.head_dim) +
                (size_t)partials * Q * p.num_qo_heads * 4;
  clear_error();
  return PKD_OK;
}

// Capacities of a graph plan for B requests holding at most max_pages pages
// in all: units per item head (all requests, and one request) from the
// planner's rules (at most one unit per started chunk and sub-chunk under a
// fixed split). Under its own split the units are of at least kUnitQuantum
// tokens, beyond one per request, or, for a batch of at most
// slots * kUnitQuantum tokens over all kv heads, chunks of at least half that
// on the chunk grid: at most 2 * slots / item heads of them per item head,
// beyond two per request.
void graph_capacities(const pkd_plan_params& p, int32_t max_pages, int64_t slots,
                      int64_t* units_total, int64_t* units_one) {
  const int64_t B = p.batch_size, P = p.page_size, M = max_pages;
  if (p.disable_split_kv) {
    *units_total = B;
    *units_one = 1;
  } else if (p.fixed_split_size > 0) {
    const int64_t S = p.fixed_split_size;
    const int64_t cap = std::min<int64_t>(S * P, kFixedUnitMaxTokens);
    const int64_t sub = (S * P + cap - 1) / cap;
    *units_total = (M / S + B) * sub;
    *units_one = (M / S + 1) * sub;
  } else {
    // (a small batch's units are chunks on the grid: a request's first one
    // may start inside a chunk, one more unit per request)
    const int64_t small = std::min<int64_t>(M * P / (kUnitQuantumTokens / 2),
                                            2 * slots / ((int64_t)p.num_kv_heads * kv_blocks(p)));
    const int64_t full = M * P / kUnitQuantumTokens;
    *units_total = std::max(full + B, small + 2 * B);
    *units_one = std::max(full + 1, small + 2);
  }
}


}  // namespace pkd
