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

// Target number of work items when the planner chooses the split: enough
// workgroups to keep every compute unit busy through the tail.
constexpr int kItemsPerCu = 8;
// Smallest chunk the planner creates on its own, in tokens: one step for each
// wavefront of a workgroup, twice.
constexpr int kMinChunkTokens = 2 * kWaves * kStepTokens;

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
  const int32_t group = p.num_qo_heads / p.num_kv_heads;
  if (group > kMaxGroup)
    return fail(PKD_EUNSUPPORTED,
                fmt("group size %d (num_qo_heads/num_kv_heads) exceeds %d",
                    group, kMaxGroup));
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

size_t workspace_lse_offset(int32_t num_partials, int32_t num_qo_heads,
                            int32_t head_dim) {
  size_t o_bytes = (size_t)num_partials * num_qo_heads * head_dim * 4;
  return (o_bytes + 255) & ~(size_t)255;
}

pkd_status build_host_plan(const pkd_plan_params& p, const int32_t* indptr,
                           const int32_t* last_page_len, int32_t num_cus,
                           HostPlan* out) {
  pkd_status st = check_params(p);
  if (st != PKD_OK) return st;
  const int32_t B = p.batch_size;
  if (B > 0 && (indptr == nullptr || last_page_len == nullptr))
    return fail(PKD_EINVAL, "indptr / last_page_len must not be NULL");
  if (num_cus < 1) return fail(PKD_EINVAL, fmt("num_cus %d < 1", num_cus));
  if (B > 0 && indptr[0] != 0)
    return fail(PKD_EINVAL, fmt("indptr[0] = %d, must be 0", indptr[0]));

  const int32_t P = p.page_size;
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
    Req r;
    r.kv_len = (int32_t)L;
    r.start = p.window_left < 0 ? 0 : std::max<int32_t>(0, r.kv_len - 1 - p.window_left);
    r.pages = (int32_t)np;
    reqs[i] = r;
    attended += r.kv_len - r.start;
    max_pages = std::max(max_pages, r.pages);
  }

  // ---- split size, in pages (0 = one chunk per request)
  int32_t split = 0;
  if (p.disable_split_kv) {
    split = 0;
  } else if (p.fixed_split_size > 0) {
    split = p.fixed_split_size;
  } else if (B > 0) {
    const int64_t target = (int64_t)num_cus * kItemsPerCu;
    auto items_for = [&](int32_t s) {
      int64_t n = 0;
      for (const Req& r : reqs) n += chunks_of(r, s, P);
      return n * p.num_kv_heads;
    };
    if (items_for(0) < target) {
      int32_t lo = std::max(1, (kMinChunkTokens + P - 1) / P);
      int32_t hi = std::max(lo, max_pages);
      // smallest split with items <= target (items_for is non-increasing)
      while (lo < hi) {
        int32_t mid = lo + (hi - lo) / 2;
        if (items_for(mid) <= target) hi = mid; else lo = mid + 1;
      }
      split = lo >= max_pages ? 0 : lo;
    }
  }

  // ---- work items and merge rows
  out->params = p;
  out->items.clear();
  out->merges.clear();
  int32_t partials = 0;
  for (int32_t i = 0; i < B; ++i) {
    const Req& r = reqs[i];
    const int64_t nch = chunks_of(r, split, P);
    const bool split_req = nch > 1;
    if (split_req) {
      if ((int64_t)partials + nch > INT32_MAX)
        return fail(PKD_EUNSUPPORTED, "too many chunks");
      out->merges.push_back(MergeRow{i, partials, (int32_t)nch, 0});
    }
    const int64_t chunk_tokens = (int64_t)split * P;
    const int64_t first_chunk = split > 0 ? (r.start / P) / split : 0;
    for (int64_t c = 0; c < nch; ++c) {
      int64_t b = split > 0 ? (first_chunk + c) * chunk_tokens : 0;
      int64_t e = split > 0 ? b + chunk_tokens : r.kv_len;
      b = std::max<int64_t>(b, r.start);
      e = std::min<int64_t>(e, r.kv_len);
      for (int32_t h = 0; h < p.num_kv_heads; ++h) {
        pkd_work_item it;
        it.request = i;
        it.kv_head = h;
        it.token_begin = (int32_t)b;
        it.token_end = (int32_t)e;
        it.page_base = indptr[i];
        it.partial = split_req ? partials + (int32_t)c : -1;
        it.chunk = (int32_t)c;
        it.reserved = 0;
        out->items.push_back(it);
      }
    }
    if (split_req) partials += (int32_t)nch;
  }
  if (out->items.size() > (size_t)INT32_MAX)
    return fail(PKD_EUNSUPPORTED, "too many work items");
  // Longest items first so that short ones fill the tail; ties keep the
  // (request, chunk, kv head) order. The order changes scheduling only: each
  // item's arithmetic depends on its own token range alone.
  std::stable_sort(out->items.begin(), out->items.end(),
                   [](const pkd_work_item& a, const pkd_work_item& b) {
                     return (a.token_end - a.token_begin) >
                            (b.token_end - b.token_begin);
                   });

  pkd_plan_info& info = out->info;
  info.num_items = (int32_t)out->items.size();
  info.num_split_requests = (int32_t)out->merges.size();
  info.num_partials = partials;
  info.split_pages = split;
  info.attended_tokens = attended;
  info.workspace_bytes =
      partials == 0
          ? 0
          : workspace_lse_offset(partials, p.num_qo_heads, p.head_dim) +
                (size_t)partials * p.num_qo_heads * 4;
  clear_error();
  return PKD_OK;
}

}  // namespace pkd
