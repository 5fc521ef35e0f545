// C-ABI of the paged-KV batch decode library (declared in include/pkd.h).
//
// plan/run split of flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper
// ("FlashInfer attention kernels" page): plan() does the host work once and
// uploads the work list; run() only enqueues one kernel on the caller's
// stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "pkd_internal.h"

namespace {

// Stream order of the launches that share some device state (a plan's
// counters, or a GPU's static workspace): an event recorded after the last
// such launch on its stream. A launch on another stream first waits for that
// event on the GPU, so launches that share the state never overlap, with no
// host synchronisation. Launches recorded into a HIP graph are not tracked.
// The event of a RunOrder is only ever waited on by another stream of the
// same GPU (hipStreamWaitEvent), never synchronised with or queried from the
// host. It is created without timing and without the system-scope fence that
// hipEventRecord otherwise adds: what the later launch needs is the earlier
// kernel's completion (its writes to the plan's state are device-scope
// atomics and device-coherent stores). Recorded after every launch, the
// fence cost each eager call about 1.7 us of GPU time (the class example's
// batch: 15.2 against 13.6 us per call; no record at all: 12.4 us).
constexpr unsigned kOrderEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

struct RunOrder {
  std::mutex mu;
  hipEvent_t ev = nullptr;    // created before the first launch
  hipStream_t on = nullptr;   // stream of the last tracked launch
  bool any = false;           // ev holds the last tracked launch
};

}  // namespace

struct pkd_plan {
  pkd::HostPlan host;
  const int32_t* indices = nullptr;   // borrowed device pointer
  void* dev = nullptr;                // counters, merge counters, items
  void* staging = nullptr;            // pinned host copy used by the upload
  hipEvent_t uploaded = nullptr;
  // Runs share the plan's work, reserve and merge counters: a run (or an
  // update) on another stream than the previous run is ordered after it.
  mutable RunOrder order;
  int device = 0;
  int32_t slots = 0;                  // decode workgroups that fit on the GPU
  // A graph plan (pkd_plan_create_graph) keeps its device memory, its launch
  // size and its workspace layout for its whole life, sized for capacities;
  // pkd_plan_update rewrites the contents, and the kernel reads the item
  // count, the stealing limit and the merge-counter stride from the header.
  bool graph = false;
  int32_t max_pages = 0;              // capacity of the page index buffer
  int32_t cap_items = 0;
  int32_t cap_partials = 0;
  int32_t cap_merge_stride = 0;
  // Device copy, all uploaded from the staging copy: the work counters
  // (zeros) and the header, the reserve slots (0xFFFFFFFF: never published),
  // the per-(request, kv head) merge counters (zeros), the items.
  static constexpr size_t kCounterBytes = 64;
  static constexpr int kHeaderWord = 4;   // header: int32 words 4, 5, 6
  int32_t merge_stride() const {
    if (graph) return cap_merge_stride;
    return 1 + (host.max_units + pkd::kMergeGroup - 1) / pkd::kMergeGroup;
  }
  size_t merge_counter_bytes() const {
    const size_t n =
        (size_t)host.params.batch_size * host.params.num_kv_heads * host.kv_blocks *
            merge_stride() * 4;
    return (n + 63) & ~(size_t)63;
  }
  size_t reserve_bytes() const {
    return ((size_t)host.info.num_workgroups * 2 * 4 + 63) & ~(size_t)63;   // two per workgroup
  }
  size_t item_capacity() const { return graph ? (size_t)cap_items : host.items.size(); }
  // ROPE_LLAMA: [head_dim/2][2] rotary frequencies (revolutions per token as
  // an unevaluated float sum hi + lo)
  bool rope() const { return host.params.pos_encoding_mode == PKD_POS_ROPE_LLAMA; }
  size_t rope_bytes() const {
    return rope() ? ((size_t)host.params.head_dim / 2 * 8 + 63) & ~(size_t)63 : 0;
  }
  int32_t ws_partials() const { return graph ? cap_partials : host.info.num_partials; }
  int32_t* d_counters() const { return reinterpret_cast<int32_t*>(dev); }
  int32_t* d_reserve() const {
    return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(dev) + kCounterBytes);
  }
  int32_t* d_merge_counters() const {
    return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(dev) + kCounterBytes +
                                      reserve_bytes());
  }
  size_t rope_offset() const { return kCounterBytes + reserve_bytes() + merge_counter_bytes(); }
  const float* d_rope() const {
    return rope() ? reinterpret_cast<const float*>(reinterpret_cast<const char*>(dev) +
                                                   rope_offset())
                  : nullptr;
  }
  const pkd_work_item* d_items() const {
    return reinterpret_cast<const pkd_work_item*>(reinterpret_cast<const char*>(dev) +
                                                  rope_offset() + rope_bytes());
  }
};

namespace {

pkd_status hip_fail(hipError_t e, const char* what) {
  return pkd::fail(PKD_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

void free_plan(pkd_plan* p) {
  if (p == nullptr) return;
  if (p->uploaded != nullptr) {
    (void)hipEventSynchronize(p->uploaded);
    (void)hipEventDestroy(p->uploaded);
  }
  if (p->order.ev != nullptr) (void)hipEventDestroy(p->order.ev);
  if (p->dev != nullptr) (void)hipFree(p->dev);
  if (p->staging != nullptr) (void)hipHostFree(p->staging);
  delete p;
}

size_t plan_bytes(const pkd_plan& p) {
  if (p.item_capacity() == 0) return 0;
  return pkd_plan::kCounterBytes + p.reserve_bytes() + p.merge_counter_bytes() +
         p.rope_bytes() + p.item_capacity() * sizeof(pkd_work_item);
}

// Fills the staging copy from the host plan and uploads it on `stream`
// (after the previous upload from the same staging memory has finished).
pkd_status upload(pkd_plan* p, void* stream) {
  const size_t bytes = plan_bytes(*p);
  if (bytes == 0) return PKD_OK;
  hipError_t e;
  if (p->uploaded != nullptr) {
    e = hipEventSynchronize(p->uploaded);
    if (e != hipSuccess) return hip_fail(e, "waiting for the previous upload");
  }
  char* s = reinterpret_cast<char*>(p->staging);
  std::memset(s, 0, pkd_plan::kCounterBytes);
  int32_t* header = reinterpret_cast<int32_t*>(s) + pkd_plan::kHeaderWord;
  header[0] = p->host.info.num_items;
  header[1] = p->host.steal_limit;
  header[2] = p->merge_stride();
  std::memset(s + pkd_plan::kCounterBytes, 0xFF, p->reserve_bytes());
  const size_t zeros = pkd_plan::kCounterBytes + p->reserve_bytes();
  std::memset(s + zeros, 0, p->merge_counter_bytes());
  if (p->rope()) {
    // pair i turns by position / rope_scale * rope_theta^(-2i/head_dim)
    // radians per token; in revolutions, as a hi + lo float pair
    const pkd_plan_params& pp = p->host.params;
    float* f = reinterpret_cast<float*>(s + p->rope_offset());
    for (int i = 0; i < pp.head_dim / 2; ++i) {
      const double rev = std::pow((double)pp.rope_theta, -2.0 * i / pp.head_dim) /
                         ((double)pp.rope_scale * 2.0 * 3.14159265358979323846);
      f[2 * i] = (float)rev;
      f[2 * i + 1] = (float)(rev - (double)f[2 * i]);
    }
  }
  std::memcpy(s + p->rope_offset() + p->rope_bytes(), p->host.items.data(),
              p->host.items.size() * sizeof(pkd_work_item));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  e = hipMemcpyAsync(p->dev, p->staging, bytes, hipMemcpyHostToDevice, hs);
  if (e == hipSuccess && p->uploaded == nullptr)
    e = hipEventCreateWithFlags(&p->uploaded, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(p->uploaded, hs);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(hs);
    return hip_fail(e, "uploading the work list");
  }
  return PKD_OK;
}

// True when `stream` is being captured into a graph (then no event is
// queried or recorded: the capture would record or forbid it).
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

// Makes `stream` wait on the GPU for the last launch tracked by `r` when
// that went to another stream. Caller holds r.mu.
pkd_status order_after(RunOrder& r, hipStream_t stream, const char* what) {
  if (!r.any || r.on == stream) return PKD_OK;
  const hipError_t e = hipStreamWaitEvent(stream, r.ev, 0);
  if (e != hipSuccess) return hip_fail(e, what);
  return PKD_OK;
}

// Records a launch just made on `stream`. Caller holds r.mu. Should the
// record fail, the launch (already made) goes untracked: the next launch on
// another stream is then not ordered after it.
void note_launch(RunOrder& r, hipStream_t stream) {
  r.any = r.ev != nullptr && hipEventRecord(r.ev, stream) == hipSuccess;
  r.on = stream;
}

// The order of the launches that use a GPU's static workspace
// (pkd_run_static_workspace, for plans of any kind); its event is created
// with the first plan made on the device.
constexpr int kMaxDevices = 64;
RunOrder g_static_order[kMaxDevices];

pkd_status prepare_static_order(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return PKD_OK;
  std::lock_guard<std::mutex> lock(g_static_order[dev].mu);
  if (g_static_order[dev].ev != nullptr) return PKD_OK;
  const hipError_t e = hipEventCreateWithFlags(&g_static_order[dev].ev, kOrderEventFlags);
  if (e != hipSuccess) return hip_fail(e, "creating the static workspace's order event");
  return PKD_OK;
}

pkd_status check_run(const pkd_plan* plan, const void* q, const void* k,
                     const void* v, int64_t page_stride, void* o,
                     void* workspace, size_t workspace_bytes) {
  if (plan == nullptr) return pkd::fail(PKD_EINVAL, "plan is NULL (run before plan)");
  const pkd_plan_params& p = plan->host.params;
  if (p.batch_size == 0) return PKD_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return pkd::fail(PKD_EINVAL, "q, k_cache, v_cache and o must not be NULL");
  const int64_t page_elems = (int64_t)p.page_size * p.num_kv_heads * p.head_dim;
  if (page_stride < page_elems)
    return pkd::fail(PKD_EINVAL, "page_stride " + std::to_string(page_stride) +
                                     " < page_size*num_kv_heads*head_dim = " +
                                     std::to_string(page_elems));
  const int kv_bytes = p.kv_dtype == PKD_E4M3 ? 1 : 2;
  if ((page_stride * kv_bytes) % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(k) % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(v) % 16) != 0 ||
      (reinterpret_cast<uintptr_t>(q) % 16) != 0)
    return pkd::fail(PKD_EINVAL,
                     "q, k_cache and v_cache must be 16-byte aligned and the page "
                     "stride a multiple of 16 bytes");
  if (reinterpret_cast<uintptr_t>(o) % 8 != 0)
    return pkd::fail(PKD_EINVAL, "o must be 8-byte aligned");
  const size_t need = plan->host.info.workspace_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return pkd::fail(PKD_EWORKSPACE, "workspace of " + std::to_string(workspace_bytes) +
                                         " bytes < required " + std::to_string(need));
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return pkd::fail(PKD_EINVAL, "workspace must be 256-byte aligned");
  return PKD_OK;
}

}  // namespace

extern "C" {

int32_t pkd_abi_version(void) { return PKD_ABI_VERSION; }

}  // extern "C"

namespace {

pkd_status query_plan(const pkd_plan_params* params, const int32_t* indptr,
                      const int32_t* last_page_len, const int32_t* page_base,
                      int32_t num_cus, pkd_plan_info* info, pkd_work_item* items,
                      int32_t capacity) {
  pkd::HostPlan h;
  pkd_status st = pkd::check_params(*params);
  if (st != PKD_OK) return st;
  if (num_cus < 1) return pkd::fail(PKD_EINVAL, "num_cus " + std::to_string(num_cus) + " < 1");
  st = pkd::build_host_plan(*params, indptr, last_page_len,
                            num_cus * pkd::decode_wgs_per_cu_table(*params), &h, page_base);
  if (st != PKD_OK) return st;
  *info = h.info;
  if (items != nullptr) {
    const size_t n = std::min<size_t>(h.items.size(), capacity < 0 ? 0 : (size_t)capacity);
    std::memcpy(items, h.items.data(), n * sizeof(pkd_work_item));
  }
  return PKD_OK;
}

pkd_status create_plan(const pkd_plan_params* params, const int32_t* indptr,
                       const int32_t* last_page_len, const int32_t* page_base,
                       const int32_t* indices, void* stream, pkd_plan** out,
                       int32_t graph_max_pages = 0) {
  pkd_status st = pkd::check_params(*params);
  if (st != PKD_OK) return st;
  if (params->batch_size > 0 && indices == nullptr)
    return pkd::fail(PKD_EINVAL, "indices must not be NULL");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");

  // Size the launch for the residency the kernel is built for; should the
  // runtime report less, use that so that no workgroup waits for a slot.
  const int32_t per_cu = std::min(pkd::decode_wgs_per_cu_table(*params),
                                  pkd::decode_wgs_per_cu(*params));
  if (per_cu < 1) return pkd::fail(PKD_EHIP, "occupancy query of the decode kernel failed");
  pkd_plan* p = new (std::nothrow) pkd_plan();
  if (p == nullptr) return pkd::fail(PKD_ENOMEM, "plan allocation failed");
  p->slots = cus * per_cu;
  st = pkd::build_host_plan(*params, indptr, last_page_len, p->slots, &p->host, page_base);
  if (st == PKD_OK) p->host.info.workgroups_per_cu = per_cu;
  if (st != PKD_OK) {
    delete p;
    return st;
  }
  p->indices = indices;
  p->device = dev;
  // The static workspace's device address on this device (looked up once
  // per device, here, outside any graph capture). A failed lookup only
  // disables pkd_run_static_workspace, which then reports it.
  (void)pkd::static_scratch_resolve(dev);
  if (graph_max_pages > 0) {
    int64_t total = 0, one = 0;
    pkd::graph_capacities(*params, graph_max_pages, p->slots, &total, &one);
    const int64_t heads = (int64_t)params->num_kv_heads * pkd::kv_blocks(*params);
    const int64_t items = total * heads;
    const int64_t stride = 1 + (one + pkd::kMergeGroup - 1) / pkd::kMergeGroup;
    const int32_t Q = pkd::q_len_of(*params);
    if (items >= (int64_t)pkd::kMaxItems ||
        (int64_t)params->batch_size * heads * stride * 4 > INT32_MAX / 2 ||
        total * Q * params->num_qo_heads * params->head_dim * 4 > INT32_MAX) {
      delete p;
      return pkd::fail(PKD_EUNSUPPORTED, "graph plan capacity of " +
                                             std::to_string(graph_max_pages) +
                                             " pages is too large for this batch");
    }
    p->graph = true;
    p->max_pages = graph_max_pages;
    p->cap_items = (int32_t)items;
    p->cap_partials = (int32_t)total;
    p->cap_merge_stride = (int32_t)stride;
    // the launch covers every slot: workgroups without a unit exit at once
    p->host.info.num_workgroups = p->slots;
    p->host.info.workspace_bytes =
        pkd::workspace_lse_offset(p->cap_partials, Q * params->num_qo_heads, params->head_dim) +
        (size_t)p->cap_partials * Q * params->num_qo_heads * 4;
  }
  e = hipEventCreateWithFlags(&p->order.ev, kOrderEventFlags);
  if (e == hipSuccess) {
    const pkd_status so = prepare_static_order(dev);
    if (so != PKD_OK) {
      free_plan(p);
      return so;
    }
  } else {
    free_plan(p);
    return hip_fail(e, "creating the plan's order event");
  }
  const size_t bytes = plan_bytes(*p);
  if (bytes > 0) {
    e = hipMalloc(&p->dev, bytes);
    if (e != hipSuccess) {
      free_plan(p);
      return pkd::fail(PKD_ENOMEM, std::string("hipMalloc of the work list: ") +
                                       hipGetErrorString(e));
    }
    e = hipHostMalloc(&p->staging, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      free_plan(p);
      return pkd::fail(PKD_ENOMEM, std::string("hipHostMalloc of the staging copy: ") +
                                       hipGetErrorString(e));
    }
    st = upload(p, stream);
    if (st != PKD_OK) {
      free_plan(p);
      return st;
    }
  }
  *out = p;
  pkd::clear_error();
  return PKD_OK;
}

}  // namespace

extern "C" {

pkd_status pkd_plan_query(const pkd_plan_params* params, const int32_t* indptr,
                          const int32_t* last_page_len, int32_t num_cus,
                          pkd_plan_info* info, pkd_work_item* items,
                          int32_t capacity) {
  if (params == nullptr || info == nullptr)
    return pkd::fail(PKD_EINVAL, "params and info must not be NULL");
  return query_plan(params, indptr, last_page_len, nullptr, num_cus, info, items, capacity);
}

pkd_status pkd_plan_query_block_table(const pkd_plan_params* params, const int32_t* seq_lens,
                                      int32_t max_blocks_per_seq, int32_t num_cus,
                                      pkd_plan_info* info, pkd_work_item* items,
                                      int32_t capacity) {
  if (params == nullptr || info == nullptr)
    return pkd::fail(PKD_EINVAL, "params and info must not be NULL");
  pkd_status st = pkd::check_params(*params);
  if (st != PKD_OK) return st;
  std::vector<int32_t> indptr, last, base;
  st = pkd::block_table_csr(*params, seq_lens, max_blocks_per_seq, &indptr, &last, &base);
  if (st != PKD_OK) return st;
  return query_plan(params, indptr.data(), last.data(), base.data(), num_cus, info, items,
                    capacity);
}

pkd_status pkd_plan_create(const pkd_plan_params* params, const int32_t* indptr,
                           const int32_t* last_page_len, const int32_t* indices,
                           void* stream, pkd_plan** out) {
  if (out == nullptr) return pkd::fail(PKD_EINVAL, "out must not be NULL");
  *out = nullptr;
  if (params == nullptr) return pkd::fail(PKD_EINVAL, "params must not be NULL");
  return create_plan(params, indptr, last_page_len, nullptr, indices, stream, out);
}

pkd_status pkd_plan_create_block_table(const pkd_plan_params* params, const int32_t* seq_lens,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       void* stream, pkd_plan** out) {
  if (out == nullptr) return pkd::fail(PKD_EINVAL, "out must not be NULL");
  *out = nullptr;
  if (params == nullptr) return pkd::fail(PKD_EINVAL, "params must not be NULL");
  pkd_status st = pkd::check_params(*params);
  if (st != PKD_OK) return st;
  std::vector<int32_t> indptr, last, base;
  st = pkd::block_table_csr(*params, seq_lens, max_blocks_per_seq, &indptr, &last, &base);
  if (st != PKD_OK) return st;
  return create_plan(params, indptr.data(), last.data(), base.data(), block_tables, stream,
                     out);
}

pkd_status pkd_plan_create_graph(const pkd_plan_params* params, int32_t max_pages,
                                 const int32_t* indptr, const int32_t* last_page_len,
                                 const int32_t* indices, void* stream, pkd_plan** out) {
  if (out == nullptr) return pkd::fail(PKD_EINVAL, "out must not be NULL");
  *out = nullptr;
  if (params == nullptr) return pkd::fail(PKD_EINVAL, "params must not be NULL");
  if (params->batch_size < 1)
    return pkd::fail(PKD_EINVAL, "a graph plan needs batch_size >= 1");
  if (max_pages < 1) return pkd::fail(PKD_EINVAL, "max_pages " + std::to_string(max_pages) + " < 1");
  if (indptr != nullptr && indptr[params->batch_size] > max_pages)
    return pkd::fail(PKD_EINVAL, "the page table holds " +
                                     std::to_string(indptr[params->batch_size]) +
                                     " pages > max_pages " + std::to_string(max_pages));
  return create_plan(params, indptr, last_page_len, nullptr, indices, stream, out, max_pages);
}

pkd_status pkd_plan_update(pkd_plan* plan, const int32_t* indptr, const int32_t* last_page_len,
                           void* stream) {
  if (plan == nullptr) return pkd::fail(PKD_EINVAL, "plan is NULL");
  if (!plan->graph)
    return pkd::fail(PKD_EINVAL, "pkd_plan_update needs a plan from pkd_plan_create_graph");
  const pkd_plan_params& p = plan->host.params;
  if (indptr == nullptr || last_page_len == nullptr)
    return pkd::fail(PKD_EINVAL, "indptr / last_page_len must not be NULL");
  if (indptr[p.batch_size] > plan->max_pages)
    return pkd::fail(PKD_EINVAL, "the page table holds " + std::to_string(indptr[p.batch_size]) +
                                     " pages > max_pages " + std::to_string(plan->max_pages));
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(plan->order.mu);
  if (!capturing(hs)) {
    // the upload overwrites what an earlier run on another stream may still read
    pkd_status ord = order_after(plan->order, hs, "ordering the update after the plan's last run");
    if (ord != PKD_OK) return ord;
  }
  pkd::HostPlan h;
  pkd_status st = pkd::build_host_plan(p, indptr, last_page_len, plan->slots, &h);
  if (st != PKD_OK) return st;
  const int32_t stride = 1 + (h.max_units + pkd::kMergeGroup - 1) / pkd::kMergeGroup;
  if (h.info.num_items > plan->cap_items || h.info.num_partials > plan->cap_partials ||
      stride > plan->cap_merge_stride)
    return pkd::fail(PKD_EUNSUPPORTED, "the page table needs more units than the graph "
                                       "plan's capacity (an internal bound was exceeded)");
  h.info.num_workgroups = plan->slots;
  h.info.workgroups_per_cu = plan->host.info.workgroups_per_cu;
  h.info.workspace_bytes = plan->host.info.workspace_bytes;
  plan->host = std::move(h);
  st = upload(plan, stream);
  if (st != PKD_OK) return st;
  pkd::clear_error();
  return PKD_OK;
}

pkd_status pkd_plan_get_info(const pkd_plan* plan, pkd_plan_info* info) {
  if (plan == nullptr || info == nullptr)
    return pkd::fail(PKD_EINVAL, "plan and info must not be NULL");
  *info = plan->host.info;
  return PKD_OK;
}

pkd_status pkd_plan_workspace_bytes(const pkd_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr)
    return pkd::fail(PKD_EINVAL, "plan and bytes must not be NULL");
  *bytes = plan->host.info.workspace_bytes;
  return PKD_OK;
}

void pkd_plan_destroy(pkd_plan* plan) { free_plan(plan); }

}  // extern "C"

namespace {

// `shared`: the order of a device state beyond the plan's that the run uses
// (the static workspace), or NULL.
pkd_status run_impl(const pkd_plan* plan, const void* q, const void* k_cache,
                    const void* v_cache, int64_t page_stride, float q_scale,
                    float k_scale, float v_scale, const float* sinks, void* o,
                    float* lse, void* workspace, size_t workspace_bytes,
                    void* stream, RunOrder* shared = nullptr) {
  pkd_status st = check_run(plan, q, k_cache, v_cache, page_stride, o, workspace,
                            workspace_bytes);
  if (st != PKD_OK) return st;
  const pkd_plan_params& p = plan->host.params;
  if (plan->item_capacity() == 0) return PKD_OK;
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale))
    return pkd::fail(PKD_EINVAL, "q_scale, k_scale and v_scale must be finite");
  {
    // the kernel runs on the stream's device (the current one for the null
    // stream) and reads the plan's memory, which lives on the plan's device
    int dev = -1;
    const hipError_t e = stream != nullptr
                             ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev)
                             : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "querying the stream's device");
    if (dev != plan->device)
      return pkd::fail(PKD_EINVAL, "the run's stream is on device " + std::to_string(dev) +
                                       ", the plan on device " + std::to_string(plan->device));
  }
  pkd::DecodeArgs a{};
  a.counters = plan->d_counters();
  a.reserve = plan->d_reserve();
  a.merge_counters = plan->d_merge_counters();
  a.merge_stride = plan->merge_stride();
  a.num_items = plan->host.info.num_items;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.indices = plan->indices;
  a.items = plan->d_items();
  a.o = o;
  a.lse = lse;
  const int32_t parts = plan->ws_partials();
  a.ws_o = reinterpret_cast<float*>(workspace);
  const int32_t Q = pkd::q_len_of(p);
  a.ws_o_bytes = (size_t)parts * Q * p.num_qo_heads * p.head_dim * 4;
  a.ws_lse = parts > 0 ? reinterpret_cast<float*>(
                             reinterpret_cast<char*>(workspace) +
                             pkd::workspace_lse_offset(parts, Q * p.num_qo_heads, p.head_dim))
                       : nullptr;
  a.page_stride = page_stride;
  if (p.layout == PKD_NHD) {
    a.slot_stride = p.num_kv_heads * p.head_dim;
    a.head_stride = p.head_dim;
  } else {
    a.slot_stride = p.head_dim;
    a.head_stride = p.page_size * p.head_dim;
  }
  a.num_qo_heads = p.num_qo_heads;
  a.kv_div = plan->host.kv_blocks;
  a.num_kv_heads = p.num_kv_heads * a.kv_div;
  a.group = p.num_qo_heads / a.num_kv_heads;
  a.q_len = Q;
  a.cols = a.group * Q;
  a.window_left = p.window_left;
  a.alibi = p.pos_encoding_mode == PKD_POS_ALIBI;
  a.rope_freq = plan->d_rope();
  int lg = 0;
  while ((1 << lg) < p.page_size) ++lg;
  a.log2_page = lg;
  a.o_bf16 = p.o_dtype == PKD_BF16;
  const float scale = p.sm_scale * q_scale * k_scale;
  const bool cap = p.logits_soft_cap > 0.0f;
  a.logit_scale = cap ? scale : scale * 1.4426950408889634f;
  a.cap = cap ? p.logits_soft_cap : 0.0f;
  a.inv_cap = cap ? 1.0f / p.logits_soft_cap : 0.0f;
  a.v_scale = v_scale;
  a.steal_limit = plan->host.steal_limit;
  a.plan_header = plan->graph ? plan->d_counters() + pkd_plan::kHeaderWord : nullptr;
  if (sinks != nullptr && reinterpret_cast<uintptr_t>(sinks) % 4 != 0)
    return pkd::fail(PKD_EINVAL, "sinks must be 4-byte aligned");
  a.sinks = sinks;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (capturing(hs)) {
    // recorded into a graph: its replays are not tracked
    int e = pkd::launch_decode(p, a, plan->host.info.num_workgroups, stream);
    if (e != hipSuccess) return hip_fail((hipError_t)e, "decode launch");
    return PKD_OK;
  }
  // (locks in a fixed order: the plan's, then the shared state's)
  std::lock_guard<std::mutex> lock(plan->order.mu);
  pkd_status ord = order_after(plan->order, hs, "ordering the run after the plan's last run");
  if (ord != PKD_OK) return ord;
  std::unique_lock<std::mutex> lock_shared;
  if (shared != nullptr) {
    lock_shared = std::unique_lock<std::mutex>(shared->mu);
    ord = order_after(*shared, hs, "ordering the run after the last use of the static workspace");
    if (ord != PKD_OK) return ord;
  }
  int e = pkd::launch_decode(p, a, plan->host.info.num_workgroups, stream);
  if (e != hipSuccess) return hip_fail((hipError_t)e, "decode launch");
  note_launch(plan->order, hs);
  if (shared != nullptr) note_launch(*shared, hs);
  return PKD_OK;
}

}  // namespace

extern "C" {

pkd_status pkd_run(const pkd_plan* plan, const void* q, const void* k_cache,
                   const void* v_cache, int64_t page_stride, float q_scale,
                   float k_scale, float v_scale, const float* sinks, void* o,
                   float* lse, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return run_impl(plan, q, k_cache, v_cache, page_stride, q_scale, k_scale, v_scale, sinks,
                  o, lse, workspace, workspace_bytes, stream);
}

pkd_status pkd_run_static_workspace(const pkd_plan* plan, const void* q, const void* k_cache,
                                    const void* v_cache, int64_t page_stride, float q_scale,
                                    float k_scale, float v_scale, const float* sinks,
                                    void* o, float* lse, void* stream) {
  if (plan == nullptr) return pkd::fail(PKD_EINVAL, "plan is NULL (run before plan)");
  const size_t need = plan->host.info.workspace_bytes;
  if (need > pkd::kStaticScratchBytes)
    return pkd::fail(PKD_EWORKSPACE,
                     "the plan needs a workspace of " + std::to_string(need) +
                         " bytes, more than the static workspace's " +
                         std::to_string(pkd::kStaticScratchBytes) +
                         "; use pkd_run with a workspace of that size");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return pkd::fail(PKD_EINVAL, "the current device (" + std::to_string(dev) +
                                     ") is not the plan's (" + std::to_string(plan->device) +
                                     ")");
  void* ws = pkd::static_scratch_address(dev);
  if (ws == nullptr)
    return pkd::fail(PKD_EHIP, "the static workspace's device address could not be "
                               "looked up on device " + std::to_string(dev));
  RunOrder* shared = dev < kMaxDevices ? &g_static_order[dev] : nullptr;
  return run_impl(plan, q, k_cache, v_cache, page_stride, q_scale, k_scale, v_scale, sinks,
                  o, lse, ws, pkd::kStaticScratchBytes, stream, shared);
}

pkd_status pkd_merge_states(const float* v, const float* s, int32_t rows,
                            int32_t num_states, int32_t head_dim, void* v_out,
                            int32_t out_dtype, float* s_out, void* stream) {
  if (rows < 0 || num_states < 0)
    return pkd::fail(PKD_EINVAL, "rows and num_states must be >= 0");
  if (head_dim < 1 || head_dim > 1024)
    return pkd::fail(PKD_EUNSUPPORTED, "head_dim " + std::to_string(head_dim) +
                                           " outside [1, 1024]");
  if (out_dtype != PKD_F16 && out_dtype != PKD_BF16 && out_dtype != PKD_F32)
    return pkd::fail(PKD_EUNSUPPORTED, "out_dtype must be F16, BF16 or F32");
  if (rows == 0) return PKD_OK;
  if (v_out == nullptr || (num_states > 0 && (v == nullptr || s == nullptr)))
    return pkd::fail(PKD_EINVAL, "v, s and v_out must not be NULL");
  pkd::MergeArgs m{};
  m.v = v;
  m.s = s;
  m.v_out = v_out;
  m.s_out = s_out;
  m.num_rows = rows;
  m.num_states = num_states;
  m.head_dim = head_dim;
  m.out_dtype = out_dtype;
  int e = pkd::launch_merge(m, stream);
  if (e != hipSuccess) return hip_fail((hipError_t)e, "merge launch");
  return PKD_OK;
}

}  // extern "C"
