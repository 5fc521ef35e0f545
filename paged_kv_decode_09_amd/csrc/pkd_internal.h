// Internal declarations shared by the planner, the C-ABI layer and the HIP
// kernels of the paged-KV decode library. Not installed; callers use pkd.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "pkd.h"

namespace pkd {

// Workgroup geometry of the decode kernel: kWaves wavefronts of 64 lanes work
// on one work item; each wavefront takes kStepTokens tokens per step.
constexpr int kWaves = 4;
constexpr int kStepTokens = 32;
constexpr int kMaxGroup = 16;       // query rows per kv head: G * Q (one MFMA tile)
constexpr int kMergeRowsPerBlock = 4;
// Units the planner sizes itself are multiples of kUnitQuantumTokens tokens
// (two 32-token steps for each wavefront) and never shorter, unless the batch
// is too small to give every workgroup such a unit (then multiples of one
// step for each wavefront); under a fixed split, chunks are processed as
// units of at most kFixedUnitMaxTokens tokens.
constexpr int kUnitQuantumTokens = 2 * kWaves * kStepTokens;
constexpr int kFixedUnitMaxTokens = 3072;
// Units of a split request are merged in two levels: each run of
// kMergeGroup consecutive units of a (request, kv head) first, then the runs.
constexpr int kMergeGroup = 8;

// Reserve slots: the unit a decode workgroup holds beyond its current one is
// published in one of its two slots (by unit parity) so that a workgroup
// with no work left can take it. A slot value (unsigned) below kMaxItems is
// a published unit, free to take. The owner claims it by adding kClaimStep
// near the end of its current unit; a thief replaces the published value by
// kStolen with a compare-and-swap. The owner sees kStolen in the value its
// addition returns iff the thief came first. 0xFFFFFFFF: never published.
// Only units of at least kStealMinBytes of K/V are published: a stolen unit
// starts without prefetch and its owner spends a few microseconds dropping
// it, which a short unit does not repay.
constexpr uint32_t kMaxItems = 1u << 24;
constexpr uint32_t kClaimStep = 1u << 25;
constexpr uint32_t kStolen = 1u << 28;
constexpr int64_t kStealMinBytes = 512 << 10;

// Wavefronts per SIMD (= decode workgroups per compute unit) each decode
// kernel instance is built for: its launch bounds cap its registers to fit,
// and the planner sizes the launch for it. Two steps of K/V rows, the next
// unit's page ids and the running state stay in registers without spilling
// (a spill reload would wait for every load in flight). One workgroup per
// compute unit already keeps several times the loads in flight that HBM
// needs to stream at full rate; more only lengthens the queues, and with
// them every dependent load at a unit boundary. Head_dim 64 (a quarter of
// the bytes per step) uses three, or two with 16-bit K/V and the rotary
// embedding, whose rotation needs more registers than a third of the file.
// An instance with one step of K/V rows in registers (`single`) runs two
// workgroups per compute unit at head_dim 128.
constexpr int decode_waves_per_simd(int head_dim, bool kv8, bool rope, bool single = false) {
  return head_dim >= 128 ? (single && head_dim == 128 ? 2 : 1) : (rope && !kv8 ? 2 : 3);
}

// Plans whose kernel holds one step of K/V rows in registers per wavefront
// instead of two (its next loads leave as soon as a step is staged in LDS):
// RoPE at head_dim 128, or at 256 with 16-bit K/V, under the planner's own
// split. The rotation keeps such a kernel busy issuing: at head_dim 128 a
// second workgroup per compute unit fills the stalls of the first (the
// serving batch with RoPE 119.5 -> 115.5 us, E4M3 KV with RoPE 550 -> 498),
// at 256 the freed registers end its spills (Gemma-2-style with RoPE 772 ->
// 751). Under a fixed split or with one unit per request the units can be
// long, and a workgroup alone on its compute unit at the end streams at half
// rate with one buffer (long context with RoPE 233 -> 268): those plans keep
// two buffers.
inline bool decode_single(const pkd_plan_params& p) {
  return p.pos_encoding_mode == PKD_POS_ROPE_LLAMA && p.fixed_split_size <= 0 &&
         !p.disable_split_kv &&
         (p.head_dim == 128 || (p.head_dim == 256 && p.kv_dtype != PKD_E4M3));
}

// One split request: its workspace slots are partial_base ..
// partial_base + num_chunks - 1, in chunk order.
struct MergeRow {
  int32_t request;
  int32_t partial_base;
  int32_t num_chunks;
  int32_t reserved;
};

// The plan's host copy. The decode workgroups take items in this order from
// a shared counter.
struct HostPlan {
  pkd_plan_params params{};
  pkd_plan_info info{};
  // Blocks of query heads per kv head (kv_blocks(params)): the items count
  // params.num_kv_heads * kv_blocks heads, and an item's kv_head is a block.
  int32_t kv_blocks = 1;
  int32_t max_units = 0;   // most units of one request (per kv head)
  // items [0, steal_limit) have at least kStealMinBytes of K/V (the items
  // are sorted longest first): only these are published for stealing
  int32_t steal_limit = 0;
  std::vector<pkd_work_item> items;
  std::vector<MergeRow> merges;
};

// Query tokens per request of a plan (0 in the parameters means 1).
inline int32_t q_len_of(const pkd_plan_params& p) {
  return p.q_len_per_req > 1 ? p.q_len_per_req : 1;
}

// Records `msg` as this thread's last error and returns `st`.
pkd_status fail(pkd_status st, const std::string& msg);
void clear_error();

// Validation of the parameters alone (no page table).
pkd_status check_params(const pkd_plan_params& p);

// Blocks of query heads per kv head. A unit carries at most kMaxGroup query
// rows (G * Q, one MFMA tile); a group with more is split into the fewest
// equal blocks of G / kv_blocks heads that fit, and each block is planned
// and run as a kv head of its own: block b of kv head h is head
// h * kv_blocks + b, its q heads (h * kv_blocks + b) * (G / kv_blocks) + ...,
// and it reads kv head h's K/V (once per block). 1 when G * Q <= kMaxGroup.
int32_t kv_blocks(const pkd_plan_params& p);

// The planner: validates the page table, picks the chunk size, builds the
// work units and spreads them over `num_slots` workgroups (the decode
// workgroups that fit on the GPU at once). Pure host code.
// `page_base` (may be NULL) gives each request's offset into the page index
// array when it is not indptr[i] (a block table: i * max_blocks_per_seq).
pkd_status build_host_plan(const pkd_plan_params& p, const int32_t* indptr,
                           const int32_t* last_page_len, int32_t num_slots,
                           HostPlan* out, const int32_t* page_base = nullptr);

// CSR page counts of a block-table batch: indptr [B+1] (running page counts),
// last_page_len [B] and page_base [B] = i * max_blocks, from seq_lens [B].
pkd_status block_table_csr(const pkd_plan_params& p, const int32_t* seq_lens,
                           int32_t max_blocks, std::vector<int32_t>* indptr,
                           std::vector<int32_t>* last_page_len,
                           std::vector<int32_t>* page_base);

// Capacities of a graph plan for p.batch_size requests holding at most
// max_pages pages in all, on a launch of `slots` workgroups: the most units
// per item head (kv head and block of its q heads) the planner can make (all
// requests, and one request).
void graph_capacities(const pkd_plan_params& p, int32_t max_pages, int64_t slots,
                      int64_t* units_total, int64_t* units_one);

// Decode workgroups per compute unit the kernel instance of `p` is built for.
int32_t decode_wgs_per_cu_table(const pkd_plan_params& p);

// Byte offset of the LSE part of the workspace.
size_t workspace_lse_offset(int32_t num_partials, int32_t num_qo_heads,
                            int32_t head_dim);

// ----------------------------------------------------------------- kernels

struct DecodeArgs {
  // counters[0]: tickets taken (items beyond each workgroup's first two).
  // Zero when a launch starts; the workgroup that takes the launch's last
  // ticket resets it.
  int32_t* counters;
  // [2 * gridDim.x] reserve slots, two per workgroup (by unit parity): the
  // unit a workgroup holds beyond its current one, for workgroups whose own
  // units have run out (encoding at kMaxItems). 0xFFFFFFFF after planning.
  int32_t* reserve;
  // [B][num_kv_heads][merge_stride] per (request, kv head) of a split
  // request: [0] runs merged, [1 + r] units of run r finished. Zero when a
  // launch starts; each is reset by the workgroup that completes it.
  int32_t* merge_counters;
  int32_t merge_stride;
  int32_t num_items;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* indices;
  const pkd_work_item* items;
  void* o;
  float* lse;
  float* ws_o;          // [num_partials][q_len][num_qo_heads][head_dim]
  size_t ws_o_bytes;
  float* ws_lse;        // [num_partials][q_len][num_qo_heads], base-2
  int64_t page_stride;  // elements between pages
  int32_t slot_stride;  // elements between tokens of a page
  int32_t head_stride;  // elements between kv heads of a page
  int32_t num_qo_heads;
  int32_t num_kv_heads; // heads of the items: kv heads times kv_div
  int32_t kv_div;       // blocks of q heads per kv head: an item's kv_head / kv_div is the cache's
  int32_t group;        // q heads per item head: G / kv_div
  int32_t q_len;        // Q, query tokens per request
  int32_t cols;         // group * Q <= kMaxGroup: query rows of a unit
  int32_t window_left;  // -1, or the left window of each query token
  int32_t alibi;        // nonzero: ALiBi bias on the logits
  // ROPE_LLAMA: [head_dim/2][2] rotary frequencies in revolutions per token
  // (hi, lo), else NULL
  const float* rope_freq;
  int32_t log2_page;
  int32_t o_bf16;       // output dtype: 0 = f16, 1 = bf16
  float logit_scale;    // sm_scale*q_scale*k_scale (times log2 e if no cap)
  float cap;            // soft cap (> 0 only in the capped kernels)
  float inv_cap;
  float v_scale;
  int32_t steal_limit;  // items below it may be published for stealing
  const float* sinks;   // NULL, or one sink logit per q head (natural units)
  // NULL, or (a graph plan) the device words {num_items, steal_limit,
  // merge_stride} of the current page table, read in place of the above
  const int32_t* plan_header;
};

struct MergeArgs {
  const float* v;       // [num_rows][num_states][head_dim] per-state outputs
  const float* s;       // [num_rows][num_states] per-state natural-log LSE
  void* v_out;
  float* s_out;
  int32_t num_rows;
  int32_t num_states;
  int32_t head_dim;
  int32_t out_dtype;    // pkd_dtype of v_out
};

// Launch wrappers (decode.hip). Return a hipError_t value as int.
int launch_decode(const pkd_plan_params& p, const DecodeArgs& a,
                  int32_t num_workgroups, void* stream);
// Decode workgroups per compute unit reported by the HIP runtime for the
// kernel instance of `p` (0 on failure).
int32_t decode_wgs_per_cu(const pkd_plan_params& p);
int launch_merge(const MergeArgs& a, void* stream);

// The library's static workspace (decode.hip): a file-scope device array of
// kStaticScratchBytes that pkd_run_static_workspace uses in place of a
// caller's workspace. static_scratch_resolve looks up its device address on
// the current device (once per device; the array's host-side name is not a
// device address); static_scratch_address returns what was resolved for
// `device` (NULL if never resolved or the lookup failed). Returns a
// hipError_t value as int.
constexpr size_t kStaticScratchBytes = PKD_STATIC_WORKSPACE_BYTES;
int static_scratch_resolve(int device);
void* static_scratch_address(int device);

}  // namespace pkd
