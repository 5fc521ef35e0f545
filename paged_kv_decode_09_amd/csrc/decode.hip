// HIP kernels for gfx950 (CDNA4): paged-KV batch decode and the log-sum-exp
// merge of split-KV partial states.
//
// What is computed is the run() of flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper
// ("FlashInfer attention kernels" page): for every work item (request, kv head,
// chunk of tokens) the G query rows of that kv head attend the chunk's keys and
// values, found through the CSR page table, with sm_scale, the optional
// logits_soft_cap (cap*tanh(x/cap)) and the window already folded into the
// item's token range by the planner. Split requests leave per-unit partial
// states, which the workgroup finishing a (request, kv head)'s last unit
// folds by log-sum-exp (the merge_states step named with plan()'s
// fixed_split_size); merge_kernel is the same step as a standalone call.
//
// Design (MI355X-first, not the page's):
//  * A persistent grid of workgroups of 4 wavefronts, one per compute unit
//    (three at head_dim 64, two for the one-buffer RoPE instances at 128),
//    that pipeline work items taken from a counter.
//    Wavefront w takes the 32-token steps w, w+4, ... of an item; the four
//    partial states are merged in LDS in wavefront order at the end, so the
//    result depends only on the item's token range (bitwise batch invariance
//    under a fixed split).
//  * K and V rows arrive as whole 128-byte lines (non-temporal 16-byte loads,
//    8 rows per load instruction) into registers, one step ahead, and go to
//    the wave's LDS copies of the step. The RoPE instances under the
//    planner's own split hold one step in registers (SINGLE): its rows go to
//    LDS and the next step's loads leave before the step is attended.
//  * q.K^T on MFMA 16x16x32: K rows, read back from LDS in the operand
//    layout, are the A operand; the item's G*Q <= 16 query rows are the B
//    operand (columns past them repeat row 0 and are never written). A kv
//    head with more query rows is planned as blocks of its q heads, each an
//    item head of its own over the same K/V.
//    Result lane l holds the logits of tokens 8*(l/16)+4*tile+i for row l%16.
//  * P.V on MFMA as O^T = V^T P^T. P^T is what each lane holds after the
//    softmax, so it needs no data movement; it enters as a hi + lo pair in
//    the operand type (two MFMAs; hi alone in the RoPE instances, whose
//    rounded operands already move p as much). V^T comes from the LDS copy of the step's
//    V rows read with ds_read_b64_tr_b16 (16-bit V) or ds_read_b64_tr_b8
//    (E4M3 V, converted after the read).
//  * Online softmax in base 2 (v_exp_f32): one running max per head, made
//    uniform across the four lane groups with two cross-lane maxima per step
//    (gfx950 row exchanges); the running sum stays per lane and is reduced
//    once at the end.
//  * Tokens outside [token_begin, token_end) are masked by a select, and their
//    loads are clamped onto the chunk's own tokens, so stale or NaN slots of a
//    page are never read.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "pkd_internal.h"

namespace pkd {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __fp16 trf16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
#define PKD_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// tanh from its exponential form: tanh(y) = 1 - 2 / (e^{2y} + 1).
// Saturates to +-1 for large |y|; absolute error a few fp32 ulps.
__device__ __forceinline__ float tanh_from_exp(float y) {
  float e = fast_exp2(y * (2.0f * kLog2e));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// cos and sin of the rotary angle of position t for a frequency given in
// revolutions per token as an unevaluated sum f.x + f.y: t * f.x is split
// into its rounded product and exact residual (an fma), the whole
// revolutions are dropped exactly, and the hardware sine and cosine (which
// take revolutions) see an argument in [-1, 2].
__device__ __forceinline__ void rope_cos_sin(int t, f32x2 f, float& c, float& sn) {
  const float tf = (float)t;                          // exact below 2^24
  const float p = tf * f[0];
  const float e = __builtin_fmaf(tf, f[0], -p);
  const float r = (p - __builtin_floorf(p)) + __builtin_fmaf(tf, f[1], e);
  c = __builtin_amdgcn_cosf(r);
  sn = __builtin_amdgcn_sinf(r);
}

// Operand type of the MFMA: the q dtype (fp8 K/V are converted to it).
template <bool BF16>
struct Op;

template <>
struct Op<false> {
  using v8 = f16x8;
  using et = _Float16;
  __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static unsigned pack(float a, float b) {
    f16x2 h = __builtin_convertvector((f32x2){a, b}, f16x2);
    return __builtin_bit_cast(unsigned, h);
  }
};

template <>
struct Op<true> {
  using v8 = bf16x8;
  using et = __bf16;
  __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static unsigned pack(float a, float b) {
    bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(unsigned, h);
  }
};

// Eight E4M3 codes (little-endian in two dwords) -> eight operand values,
// two per instruction with gfx950's scaled packed conversion (scale 1). Every
// OCP E4M3 value is exact in fp16 and bf16, so nothing rounds: the results
// equal a decode to fp32 followed by a pack.
template <bool BF16>
__device__ __forceinline__ typename Op<BF16>::v8 e4m3x8(unsigned lo, unsigned hi) {
  u32x4 r;
  if constexpr (BF16) {
    r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  } else {
    r[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
    r[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
    r[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
    r[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
  }
  return __builtin_bit_cast(typename Op<BF16>::v8, r);
}

// Eight E4M3 codes (words 0 and 1 of a piece, or 2 and 3 if `upper`) as
// fp32, in order, two per scaled conversion (scale 1: exact).
__device__ __forceinline__ void e4m3_f32x8(const u32x4& w, bool upper, float (&x)[8]) {
  const unsigned lo = upper ? w[2] : w[0], hi = upper ? w[3] : w[1];
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, false);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, 1.0f, true);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true);
  x[0] = a[0]; x[1] = a[1]; x[2] = b[0]; x[3] = b[1];
  x[4] = c[0]; x[5] = c[1]; x[6] = d[0]; x[7] = d[1];
}

// The values of x in a lane and in the lane 16 (or 32) away, from gfx950's
// row exchanges on two copies of x. v_permlane16_swap swaps the odd 16-lane rows
// of its first operand with the even rows of its second, v_permlane32_swap
// the upper half of the first with the lower half of the second; on two
// copies of x, lane l of the two results then holds {x[l], x[l ^ 16]} (or
// {x[l], x[l ^ 32]}), in some order. No lane index, no LDS round trip. The
// copies are made opaque first: the compiler would otherwise take the
// exchange of two equal operands for a no-op.
template <bool kHalves>
__device__ __forceinline__ f32x2 lane_pair(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("" : "+v"(a));
  asm volatile("" : "+v"(b));
  // (the elements are copied out before any bit cast: a bit cast applied to
  // an element of the returned vector reads element 0)
  unsigned lo, hi;
  if constexpr (kHalves) {
    auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    lo = r[0];
    hi = r[1];
  }
  return (f32x2){__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi)};
}
// Reductions over the four 16-lane groups; max and + are commutative, so
// every lane gets the same bits as from x op x[l ^ 16], then op x[l ^ 32].
__device__ __forceinline__ float wave_max_over_groups(float x) {
  f32x2 p = lane_pair<false>(x);
  x = fmaxf(p[0], p[1]);
  p = lane_pair<true>(x);
  return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float wave_sum_over_groups(float x) {
  f32x2 p = lane_pair<false>(x);
  x = p[0] + p[1];
  p = lane_pair<true>(x);
  return p[0] + p[1];
}

// Both results of gfx950's v_permlane32_swap on two copies of x: one lane's
// pair holds x[l] and x[l ^ 32] (which is which depends on the lane's half;
// swap_other() below picks the partner's). The copies are made opaque as in
// lane_pair.
__device__ __forceinline__ u32x2 swap_halves(unsigned x) {
  unsigned a = x, b = x;
  asm volatile("" : "+v"(a));
  asm volatile("" : "+v"(b));
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return (u32x2){r0, r1};
}
// x of lane l ^ 32. `second` (from partner_slot) says which result of the
// exchange holds it in this lane.
__device__ __forceinline__ unsigned swap_other(unsigned x, bool second) {
  const u32x2 r = swap_halves(x);
  return second ? r[1] : r[0];
}
// Whether the second result of the exchange holds lane l ^ 32's value in
// lane l: found by exchanging the lane index itself (once per kernel).
__device__ __forceinline__ bool partner_slot(unsigned lane) {
  return swap_halves(lane)[1] == (lane ^ 32u);
}

// Device-scope (agent) relaxed atomic store: it bypasses the caches that are
// not coherent across the XCDs, so a workgroup on any XCD that loads with
// the sc1 policy (load_coherent4/1 below) sees the value once the storing
// wave's store has completed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Workgroup barrier that orders LDS accesses only. (__syncthreads() also
// orders global memory, which on this GPU makes every wave first wait for
// all its loads in flight, including prefetches meant to cross the barrier.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(0): this wave's vector memory operations have completed.
__device__ __forceinline__ void wait_vector_memory() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Four consecutive outputs (idx a multiple of 4) in one 8-byte store.
__device__ __forceinline__ void store_out4(void* base, size_t idx, f32x4 v, int bf16) {
  u32x2 w;
  if (bf16) {
    w[0] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2));
    w[1] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2));
  } else {
    w[0] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){v[0], v[1]}, f16x2));
    w[1] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){v[2], v[3]}, f16x2));
  }
  *reinterpret_cast<u32x2*>(reinterpret_cast<char*>(base) + idx * 2) = w;
}

__device__ __forceinline__ void store_out(void* base, size_t idx, float v, int bf16) {
  if (bf16)
    reinterpret_cast<__bf16*>(base)[idx] = (__bf16)v;
  else
    reinterpret_cast<_Float16*>(base)[idx] = (_Float16)v;
}

// Geometry of one kernel instance.
template <int HD, bool KV8>
struct Geo {
  static constexpr int kKvBytes = KV8 ? 1 : 2;
  static constexpr int kRowBytes = HD * kKvBytes;
  // 16-byte pieces a lane loads per row: the four lane groups of a wave cover
  // 64 contiguous bytes of the row per piece.
  static constexpr int kPieces = kRowBytes / 64;
  static constexpr int kQkMfma = HD / 32;   // MFMAs per 16-token tile
  static constexpr int kPvMfma = HD / 16;   // MFMAs per 32-token step
  // LDS row pitch of the K and V copies; the pad staggers rows across banks.
  static constexpr int kVPitch = kRowBytes + (KV8 ? 16 : 32);
  static constexpr int kVBytes = kStepTokens * kVPitch;
  // K rows are staged in a region of their own, after the V rows
  static constexpr int kStageBytes = 2 * kVBytes;
  static constexpr int kMergeBytes = kMaxGroup * HD * 4;
  static constexpr int kWaveLds = kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes;
};

// Page ids of the item are staged in LDS, a window at a time, so that the
// per-step page lookups do not queue behind the K/V loads in flight.
constexpr int kPageWin = 1024;

// hd index of the first of the 8 operand elements that lane group g feeds to
// QK MFMA j. The hd order inside the dot product is free as long as q uses
// the same one; this one makes each load instruction of a wave cover 64
// contiguous bytes of a row.
template <bool KV8>
__device__ __forceinline__ int qk_hd(int j, int g) {
  return KV8 ? 64 * (j >> 1) + 16 * g + 8 * (j & 1) : 32 * j + 8 * g;
}

template <int NP>
struct StepRegs {
  u32x4 k[2][NP];
  u32x4 v[2][NP];
};

// Buffer resource over `bytes` bytes at `base` for the loads below (raw
// buffer, dword 3 as for every gfx9 raw buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// 16- and 4-byte loads with the sc1 cache policy (device-coherent, the
// policy of an agent-scope atomic load), up to 16 bytes per instruction.
constexpr int kCoherentPolicy = 16;   // sc1
// (The builtins return raw bits as unsigned integers.)
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherentPolicy));
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherentPolicy));
}
// 16-byte store with the same policy as store_coherent.
__device__ __forceinline__ void store_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherentPolicy);
}

// merge_states for one (request, item head) of a split request: fold the G
// heads' states of `count` workspace slots first, first + stride, ...
// (normalised outputs, base-2 LSE) by log-sum-exp, in slot order. The
// result goes to o and the natural-log lse (out_slot < 0), or, as a state
// of the same form, to workspace slot out_slot (then one of the inputs, and
// count <= kBatch: every thread has its inputs before any thread writes).
//
// Each thread owns one float4 column of one head and loads the outputs and
// LSEs of kBatch slots at once; a later batch rescales the running sums to
// the new maximum.
template <int HD>
__device__ void merge_partials(const DecodeArgs& a, int request, int qh0, int first, int stride,
                               int count, int out_slot) {
  constexpr int kBatch = HD == 128 ? 16 : 8;
  constexpr int cols4 = HD / 4;
  const int n = count;
  const int G = a.group;
  const int nq = a.num_qo_heads;
  const int R = a.q_len * nq;                          // query rows of a slot
  const size_t span = (size_t)(n - 1) * stride + 1;   // slots covered
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(a.ws_o + (size_t)first * R * HD, (uint32_t)(span * R * HD * 4));
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(a.ws_lse + (size_t)first * R, (uint32_t)(span * R * 4));
  for (int e0 = 0; e0 < a.cols * cols4; e0 += kWaves * 64) {
    const int e = e0 + (int)threadIdx.x;
    const bool active = e < a.cols * cols4;
    // row h of the unit: query token qj, q head qh0 + gh
    const int h = active ? e / cols4 : 0, c4 = active ? e - h * cols4 : 0;
    const int qj = h / G, gh = h - qj * G;
    const int row = qj * nq + qh0 + gh;                 // within a slot
    float M = -INFINITY, den = 0.0f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n; k0 += kBatch) {
      f32x4 x[kBatch];
      float l[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int k = min(k0 + j, n - 1) * stride;
        x[j] = load_coherent4(ro, (uint32_t)((k * R + row) * HD + 4 * c4) * 4);
        l[j] = load_coherent1(rl, (uint32_t)(k * R + row) * 4);
      }
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (k0 + j < n) bm = fmaxf(bm, l[j]);
      const float Mn = fmaxf(M, bm);
      if (Mn != -INFINITY) {
        const float sc = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
        den *= sc;
        num *= sc;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (k0 + j < n) {
            const float wk = l[j] == -INFINITY ? 0.0f : fast_exp2(l[j] - Mn);
            den += wk;
            num += wk * x[j];
          }
        }
        M = Mn;
      }
    }
    if (out_slot >= 0) {
      // in place: every thread holds its inputs before any thread writes
      wait_vector_memory();
      lds_barrier();
    }
    if (!active) continue;
    if (out_slot < 0 && a.sinks != nullptr) {
      // the q head's sink joins the final softmax (one more logit, no value)
      const float s2 = a.sinks[qh0 + gh] * kLog2e;
      const float Mn = fmaxf(M, s2);
      if (Mn != -INFINITY) {
        const float r = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
        den = den * r + (s2 == -INFINITY ? 0.0f : fast_exp2(s2 - Mn));
        num *= r;
        M = Mn;
      }
    }
    const float lse2 = den > 0.0f ? M + __builtin_amdgcn_logf(den) : -INFINITY;
    if (out_slot < 0) {
      const size_t orow = ((size_t)request * a.q_len + qj) * nq + qh0 + gh;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out(a.o, orow * HD + 4 * c4 + i, den > 0.0f ? num[i] / den : 0.0f, a.o_bf16);
      if (a.lse != nullptr && c4 == 0) a.lse[orow] = lse2 * kLn2;
    } else {
      float* orow = a.ws_o + ((size_t)out_slot * R + row) * HD + 4 * c4;
#pragma unroll
      for (int i = 0; i < 4; ++i) store_coherent(orow + i, den > 0.0f ? num[i] / den : 0.0f);
      if (c4 == 0) store_coherent(a.ws_lse + (size_t)out_slot * R + row, lse2);
    }
  }
}

// Wave-uniform description of one work item (a pkd_work_item in SGPRs).
struct Unit {
  int request, kv_head, tb, te, page_base, partial, chunk, num_chunks, qpos;
};

// Lane l < 9 loads dword l of item k (lanes past it load the last one
// again): the whole item is then in lanes 0..8 of one VGPR, in flight like
// any other vector load.
constexpr int kItemWords = sizeof(pkd_work_item) / 4;
__device__ __forceinline__ unsigned load_item_lanes(const pkd_work_item* items, int k, int lane) {
  return reinterpret_cast<const unsigned*>(items + k)[lane < kItemWords ? lane : kItemWords - 1];
}
__device__ __forceinline__ Unit unit_from_lanes(unsigned v) {
  Unit u;
  u.request = __builtin_amdgcn_readlane((int)v, 0);
  u.kv_head = __builtin_amdgcn_readlane((int)v, 1);
  u.tb = __builtin_amdgcn_readlane((int)v, 2);
  u.te = __builtin_amdgcn_readlane((int)v, 3);
  u.page_base = __builtin_amdgcn_readlane((int)v, 4);
  u.partial = __builtin_amdgcn_readlane((int)v, 5);
  u.chunk = __builtin_amdgcn_readlane((int)v, 6);
  u.num_chunks = __builtin_amdgcn_readlane((int)v, 7);
  u.qpos = __builtin_amdgcn_readlane((int)v, 8);
  return u;
}

// One window of a unit's steps: the tokens [wlo, whi] whose pages are in
// sp[0 ..] (page wpage0 onwards), read for kv head offset head_off.
struct Win {
  int base, wlo, whi, wpage0;
  const int* sp;
  int64_t head_off;
};

template <int HD, bool QBF16, bool KV8, bool CAP, bool ROPE, bool SINGLE>
__global__ __launch_bounds__(kWaves * 64, decode_waves_per_simd(HD, KV8, ROPE, SINGLE)) void decode_kernel(DecodeArgs args) {
  DecodeArgs a = args;
  if (args.plan_header != nullptr) {
    // a graph plan: the launch was recorded once; the current page table's
    // counts are in the plan's device header
    a.num_items = __builtin_amdgcn_readfirstlane(args.plan_header[0]);
    a.steal_limit = __builtin_amdgcn_readfirstlane(args.plan_header[1]);
    a.merge_stride = __builtin_amdgcn_readfirstlane(args.plan_header[2]);
  }
  using G_ = Geo<HD, KV8>;
  using O = Op<QBF16>;
  // SINGLE: one register buffer of K/V rows per wavefront, whose next loads
  // leave as soon as a step is staged in LDS (decode_single tells which
  // plans run such an instance). At head_dim 128 two workgroups share a
  // compute unit, which keeps the loads in flight per SIMD of two buffers
  // at one workgroup, and the rotation of one wavefront's keys fills the
  // stalls of the other's.
  constexpr bool kSingle = SINGLE;
  static_assert(!SINGLE || (ROPE && (HD == 128 || (HD == 256 && !KV8))), "no such instance");
  // (two workgroups' LDS must fit a compute unit at head_dim 128)
  constexpr int kPageWinOf = kSingle && HD == 128 ? kPageWin / 2 : kPageWin;
  using v8 = typename O::v8;
  __shared__ __attribute__((aligned(16))) char smem[kWaves * G_::kWaveLds];
  __shared__ int s_pages[2][kPageWinOf]; // first window of this unit / of the next
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_d[kWaves][kMaxGroup];
  __shared__ int s_ticket[2];
  __shared__ int s_last;
  __shared__ unsigned long long s_steal;
  __shared__ int s_drop;
  // rotary frequencies [HD/2] (revolutions per token, hi + lo), and the
  // cosine and sine of the angle of a 4-token advance; ROPE only
  __shared__ f32x2 s_rope[ROPE ? HD / 2 : 1];
  __shared__ f32x2 s_rope4[ROPE ? HD / 2 : 1];

  if constexpr (ROPE) {
    for (int i = threadIdx.x; i < HD / 2; i += kWaves * 64) {
      const f32x2 f = reinterpret_cast<const f32x2*>(a.rope_freq)[i];
      float c, sn;
      rope_cos_sin(4, f, c, sn);
      s_rope[i] = f;
      s_rope4[i] = (f32x2){c, sn};
    }
    lds_barrier();
  }
  const int lane = threadIdx.x & 63;
  // wave-uniform (an SGPR), so that the step loop branches on scalars
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;        // MFMA row (tile token) / column (q head)
  const int g = lane >> 4;        // lane group
  const int group = a.group;
  // the cache's kv head of an item head (a block of its q heads when the
  // group is split; the division is skipped otherwise)
  auto cache_head = [&](int h) { return a.kv_div > 1 ? h / a.kv_div : h; };
  const int lp = a.log2_page;
  const int page_mask = (1 << lp) - 1;
  const int last_item = a.num_items - 1;
  // steps per window of pages held in LDS
  const int win_steps = max(1, ((kPageWinOf - 1) << lp) >> 5);
  // Token (within a step) whose K row lane n loads for tiles 0 and 1: tile
  // rows 4g'+i then map to tokens 8g'+4*tile+i.
  const int tau0 = 8 * (n >> 2) + (n & 3);
  const int tau1 = tau0 + 4;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  char* vl = smem + wave * G_::kWaveLds;

  // The first window of a unit: its first win_steps steps.
  auto first_window = [&](const Unit& u, const int* sp) {
    Win W;
    W.base = u.tb & ~(kStepTokens - 1);
    W.wlo = u.tb;
    W.whi = min(u.te, W.base + win_steps * kStepTokens) - 1;
    W.wpage0 = u.tb >> lp;
    W.sp = sp;
    W.head_off = (int64_t)cache_head(u.kv_head) * a.head_stride;
    return W;
  };

  // Tokens (clamped onto [wlo, whi]) whose rows lane n loads in step s of
  // window W, for tiles 0 and 1. Tokens outside the window (masked ones, and
  // the surplus prefetch past its last step) are clamped onto it, so every
  // load reads a valid row of the unit.
  auto token = [&](const Win& W, int s, int tau) {
    return min(max(W.base + s * kStepTokens + tau, W.wlo), W.whi);
  };
  // Whole-line loads. Lane l loads 16-byte chunk (l % kLr) of step row
  // l / kLr + kRowsPer * b: one load instruction covers kLr * 16 contiguous
  // bytes of each of its rows, whole 128-byte lines when a row holds one.
  // (Loads of 64 bytes from each of 16 rows, the layout the MFMA operand
  // wants, stream about 15 % slower from HBM.) The rows reach the MFMA
  // layout through this wave's LDS copy (consume).
  constexpr int kChunks = G_::kRowBytes / 16;
  constexpr int kLr = kChunks < 8 ? kChunks : 8;
  constexpr int kRowsPer = 64 / kLr;
  constexpr int kRowBlocks = kStepTokens / kRowsPer;   // rows per lane and step
  constexpr int kChunkBlocks = kChunks / kLr;
  constexpr int kNP = G_::kPieces;
  static_assert(kRowBlocks * kChunkBlocks == 2 * kNP, "one register per load");
  const int lrow = lane / kLr, lchunk = lane % kLr;
  // Issue the K/V loads of this lane's rows: tokens c[b] in pages pg[b].
  auto issue_rows = [&](const Win& W, const int (&c)[kRowBlocks], const int (&pg)[kRowBlocks],
                        StepRegs<kNP>& st) {
    // K and V rows are read once per launch: non-temporal loads (each one a
    // whole 128-byte line) keep them from displacing other lines in the caches
    int64_t rb[kRowBlocks];
#pragma unroll
    for (int b = 0; b < kRowBlocks; ++b)
      rb[b] = ((int64_t)pg[b] * a.page_stride + (int64_t)(c[b] & page_mask) * a.slot_stride +
               W.head_off) * G_::kKvBytes;
#pragma unroll
    for (int q = 0; q < kChunkBlocks; ++q)
#pragma unroll
      for (int b = 0; b < kRowBlocks; ++b) {
        const int i = q * kRowBlocks + b;
        st.k[i / kNP][i % kNP] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + rb[b] + 16 * (q * kLr + lchunk)));
      }
#pragma unroll
    for (int q = 0; q < kChunkBlocks; ++q)
#pragma unroll
      for (int b = 0; b < kRowBlocks; ++b) {
        const int i = q * kRowBlocks + b;
        st.v[i / kNP][i % kNP] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + rb[b] + 16 * (q * kLr + lchunk)));
      }
  };
  // Issue the K/V loads of step s of window W (page ids from its LDS window).
  auto issue = [&](const Win& W, int s, StepRegs<kNP>& st) {
    int c[kRowBlocks], pg[kRowBlocks];
#pragma unroll
    for (int b = 0; b < kRowBlocks; ++b) {
      c[b] = token(W, s, lrow + kRowsPer * b);
      pg[b] = W.sp[(c[b] >> lp) - W.wpage0];
    }
    issue_rows(W, c, pg, st);
  };

  // q operand: column n is query row n of the unit (query token n / G, q
  // head n % G of the kv head). Columns n >= G*Q load row 0 again: they
  // produce a duplicate of row 0's softmax that stays in its own columns (no
  // step mixes columns) and is never written out. Every lane loads, so that
  // the number of loads in flight is the same on every path.
  const int cols = a.cols;
  const int col_tok = (n < cols ? n : 0) / group;   // query token of column n
  const int col_head = (n < cols ? n : 0) - col_tok * group;
  v8 bq[G_::kQkMfma];
  auto load_q = [&](const Unit& u) {
    const _Float16* qrow = reinterpret_cast<const _Float16*>(a.q) +
                           (((size_t)u.request * a.q_len + col_tok) * a.num_qo_heads +
                            u.kv_head * group + col_head) * HD;
#pragma unroll
    for (int j = 0; j < G_::kQkMfma; ++j)
      bq[j] = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(qrow + qk_hd<KV8>(j, g)));
  };

  float m_run, d_run;     // running max (base-2 logits) / this lane's sum, column n
  f32x4 acc[G_::kPvMfma];
  // Tokens column n may see in the current unit: up to its query token's
  // position, and from its window start (set per unit).
  int col_lo = 0, col_hi = 0;
  // Tokens every column sees (wave-uniform, set per unit): from the last
  // query token's window start to the first query token's position.
  int vis_lo = 0, vis_hi = -1;
  // per-step work trimmed where it leaves the bits unchanged (see consume)
  constexpr bool kTrimStep = ROPE && HD <= 128;
  // ALiBi slope of column n's q head, in the units the logits are in before
  // the cap (base 2 without a cap); 0 without ALiBi, which leaves every
  // logit's bits unchanged.
  float col_slope = 0.0f;

  // ROPE_LLAMA: operand pieces j and j + kQkMfma/2 of a lane hold the two
  // halves (d, d + HD/2) of the same rotary pairs, so each lane turns its
  // own elements. Element e of piece j is hd index qk_hd(j, g) + e.
  constexpr int kHalf = G_::kQkMfma / 2;
  // Head_dim 64 with E4M3 keys: lane group g holds dims 16g..16g+15 of its
  // row (both operand pieces), so the partner d +- 32 of each of its dims
  // sits in lane l ^ 32 (group g ^ 2). The lanes exchange their pieces with
  // gfx950's half-wave swap and each turns its own 16 elements: with c, s of
  // pair d mod 32, a first-half element becomes own * c - partner * s, a
  // second-half one own * c + partner * s.
  constexpr bool kRopeCross = ROPE && KV8 && HD == 64;
  [[maybe_unused]] const bool swap_second = kRopeCross ? partner_slot((unsigned)lane) : false;
  [[maybe_unused]] const float rope_sgn = g >= 2 ? 1.0f : -1.0f;
  // q of this column at its query position (kRopeCross)
  auto rope_q_cross = [&](int pos) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4 w = __builtin_bit_cast(u32x4, bq[j]);
      u32x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = swap_other(w[i], swap_second);
      const v8 par = __builtin_bit_cast(v8, pw);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, sn;
        rope_cos_sin(pos, s_rope[16 * (g & 1) + 8 * j + e], c, sn);
        bq[j][e] = (typename O::et)((float)bq[j][e] * c + rope_sgn * (float)par[e] * sn);
      }
    }
  };
  auto rope_pair = [&](v8& lo_op, v8& hi_op, int j, int pos) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, sn;
      rope_cos_sin(pos, s_rope[qk_hd<KV8>(j, g) + e], c, sn);
      const float lo = (float)lo_op[e], hi = (float)hi_op[e];
      lo_op[e] = (typename O::et)(lo * c - hi * sn);
      hi_op[e] = (typename O::et)(hi * c + lo * sn);
    }
  };
  // the K operand of piece j of tile `tile` (kr: K in the MFMA layout)
  auto k_operand = [&](const u32x4 (&kr)[2][kNP], int tile, int j) {
    if constexpr (KV8) {
      const u32x4 w = kr[tile][j >> 1];
      return (j & 1) ? e4m3x8<QBF16>(w[2], w[3]) : e4m3x8<QBF16>(w[0], w[1]);
    } else {
      return __builtin_bit_cast(v8, kr[tile][j]);
    }
  };
  bool q_turned = false;   // this unit's q has been rotated (ROPE only)

  // Attend step s of window W whose K/V rows are in st. A step wholly past
  // the window (the padding step of an odd count) changes nothing.
  // ---- the step's K and V rows to this wave's LDS copies (row = token
  // within the step) as loaded. A wave's LDS accesses run in order, so the
  // previous step's reads are done before these writes land.
  auto stage = [&](const Win& W, int s, const StepRegs<kNP>& st) {
    const int t0 = W.base + s * kStepTokens;
    if (t0 > W.whi) return;
    char* kl = vl + G_::kVBytes;
#pragma unroll
    for (int q = 0; q < kChunkBlocks; ++q)
#pragma unroll
      for (int b = 0; b < kRowBlocks; ++b) {
        const int i = q * kRowBlocks + b;
        const int off = (lrow + kRowsPer * b) * G_::kVPitch + 16 * (q * kLr + lchunk);
        *reinterpret_cast<u32x4*>(kl + off) = st.k[i / kNP][i % kNP];
        *reinterpret_cast<u32x4*>(vl + off) = st.v[i / kNP][i % kNP];
      }
  };
  // ---- attend the step staged in LDS: K read back in the MFMA layout (lane
  // (n, g) of tile t: 64-byte piece p of row tau_t from byte 16 g)
  auto attend = [&](const Win& W, int s) {
    const int t0 = W.base + s * kStepTokens;
    if (t0 > W.whi) return;
    char* kl = vl + G_::kVBytes;
    // (With the rotary embedding at head_dim 256 and 16-bit K the pieces are
    // read pair by pair inside the rotation below: all sixteen at once would
    // not leave the registers the rotation needs.)
    constexpr bool kPieceByPiece = ROPE && HD == 256 && !KV8;
    u32x4 kr[2][kNP];
    auto read_piece = [&](int tile, int p) {
      return *reinterpret_cast<const u32x4*>(kl + (tile ? tau1 : tau0) * G_::kVPitch + 64 * p + 16 * g);
    };
    if constexpr (!kPieceByPiece) {
#pragma unroll
      for (int p = 0; p < kNP; ++p) {
        kr[0][p] = read_piece(0, p);
        kr[1][p] = read_piece(1, p);
      }
    }
    if constexpr (ROPE) {
      // q at its query position, once per unit (its loads have landed by
      // the unit's first step)
      if (!q_turned) {
        if constexpr (kRopeCross) {
          rope_q_cross(col_hi);
        } else {
#pragma unroll
          for (int j = 0; j < kHalf; ++j) rope_pair(bq[j], bq[j + kHalf], j, col_hi);
        }
        q_turned = true;
      }
    }
    // ---- logits: S[tile] rows = tokens, columns = heads
    f32x4 sc[2];
    if constexpr (ROPE) {
      // each key at its token index t0 + tau, a rotary pair of pieces at a
      // time. Rows outside the window hold a clamped token's key and are
      // masked below, so the unclamped index serves every row. Tile 1's rows
      // are 4 tokens after tile 0's: their angles follow from tile 0's by
      // the angle-addition formulas.
      const int tok = t0 + tau0;
      sc[0] = (f32x4){0.f, 0.f, 0.f, 0.f};
      sc[1] = sc[0];
      if constexpr (kRopeCross) {
        // the partner lane's 16 E4M3 codes of the same row, then each own
        // element turned with its pair's angle (tile 1's from tile 0's)
        u32x4 own[2], par[2];
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          own[tile] = kr[tile][0];
#pragma unroll
          for (int i = 0; i < 4; ++i) par[tile][i] = swap_other(own[tile][i], swap_second);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          u32x4 k0, k1;   // the rotated pieces j of tiles 0 and 1, packed
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // elements 8j + 2q, 8j + 2q + 1: word 2j + q / 2, half q % 2
            const int wi = 2 * j + (q >> 1);
            f32x2 o0, p0, o1, p1;
            if (q & 1) {
              o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(own[0][wi], 1.0f, true);
              p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(par[0][wi], 1.0f, true);
              o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(own[1][wi], 1.0f, true);
              p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(par[1][wi], 1.0f, true);
            } else {
              o0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(own[0][wi], 1.0f, false);
              p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(par[0][wi], 1.0f, false);
              o1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(own[1][wi], 1.0f, false);
              p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(par[1][wi], 1.0f, false);
            }
            float r0[2], r1[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int i = 16 * (g & 1) + 8 * j + 2 * q + u;   // pair index
              float c0, s0;
              rope_cos_sin(tok, s_rope[i], c0, s0);
              const f32x2 r4 = s_rope4[i];
              const float c1 = c0 * r4[0] - s0 * r4[1], s1 = s0 * r4[0] + c0 * r4[1];
              r0[u] = o0[u] * c0 + rope_sgn * p0[u] * s0;
              r1[u] = o1[u] * c1 + rope_sgn * p1[u] * s1;
            }
            k0[q] = O::pack(r0[0], r0[1]);
            k1[q] = O::pack(r1[0], r1[1]);
          }
          sc[0] = O::mfma(__builtin_bit_cast(v8, k0), bq[j], sc[0]);
          sc[1] = O::mfma(__builtin_bit_cast(v8, k1), bq[j], sc[1]);
        }
      } else {
#pragma unroll
      for (int j = 0; j < kHalf; ++j) {
        if constexpr (kPieceByPiece) {
          // 16-bit K at head_dim 256: piece j and j + kHalf of both tiles
          kr[0][j] = read_piece(0, j);
          kr[0][j + kHalf] = read_piece(0, j + kHalf);
          kr[1][j] = read_piece(1, j);
          kr[1][j + kHalf] = read_piece(1, j + kHalf);
        }
        v8 lo0, hi0, lo1, hi1;
        if constexpr (KV8) {
          // E4M3 codes straight to fp32 (two per exact conversion), turned,
          // then rounded once to the operand type
          float fl0[8], fh0[8], fl1[8], fh1[8];
          e4m3_f32x8(kr[0][j >> 1], (j & 1) != 0, fl0);
          e4m3_f32x8(kr[0][(j + kHalf) >> 1], ((j + kHalf) & 1) != 0, fh0);
          e4m3_f32x8(kr[1][j >> 1], (j & 1) != 0, fl1);
          e4m3_f32x8(kr[1][(j + kHalf) >> 1], ((j + kHalf) & 1) != 0, fh1);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = qk_hd<KV8>(j, g) + e;
            float c0, s0;
            rope_cos_sin(tok, s_rope[d], c0, s0);
            const f32x2 r4 = s_rope4[d];
            const float c1 = c0 * r4[0] - s0 * r4[1], s1 = s0 * r4[0] + c0 * r4[1];
            lo0[e] = (typename O::et)(fl0[e] * c0 - fh0[e] * s0);
            hi0[e] = (typename O::et)(fh0[e] * c0 + fl0[e] * s0);
            lo1[e] = (typename O::et)(fl1[e] * c1 - fh1[e] * s1);
            hi1[e] = (typename O::et)(fh1[e] * c1 + fl1[e] * s1);
          }
        } else {
          lo0 = k_operand(kr, 0, j);
          hi0 = k_operand(kr, 0, j + kHalf);
          lo1 = k_operand(kr, 1, j);
          hi1 = k_operand(kr, 1, j + kHalf);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = qk_hd<KV8>(j, g) + e;
            float c0, s0;
            rope_cos_sin(tok, s_rope[d], c0, s0);
            const f32x2 r4 = s_rope4[d];
            const float c1 = c0 * r4[0] - s0 * r4[1], s1 = s0 * r4[0] + c0 * r4[1];
            float l = (float)lo0[e], h = (float)hi0[e];
            lo0[e] = (typename O::et)(l * c0 - h * s0);
            hi0[e] = (typename O::et)(h * c0 + l * s0);
            l = (float)lo1[e];
            h = (float)hi1[e];
            lo1[e] = (typename O::et)(l * c1 - h * s1);
            hi1[e] = (typename O::et)(h * c1 + l * s1);
          }
        }
        sc[0] = O::mfma(lo0, bq[j], sc[0]);
        sc[0] = O::mfma(hi0, bq[j + kHalf], sc[0]);
        sc[1] = O::mfma(lo1, bq[j], sc[1]);
        sc[1] = O::mfma(hi1, bq[j + kHalf], sc[1]);
      }
      }
    } else {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        f32x4 acc_s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < G_::kQkMfma; ++j) acc_s = O::mfma(k_operand(kr, tile, j), bq[j], acc_s);
        sc[tile] = acc_s;
      }
    }
    // ---- online softmax (base 2)
    const int lo = max(W.wlo, col_lo), hi = min(W.whi, col_hi);
    float x[8];
    float mx = -INFINITY;
    // A step wholly inside every column's visible range (all of them contain
    // [max(wlo, vis_lo), min(whi, vis_hi)]) needs no mask, and without ALiBi
    // no bias: the same bits, fewer instructions. Only the RoPE instances up
    // to head_dim 128, whose steps are bound by instruction issue, take this
    // path (serving_rope -1.7 us); elsewhere the second path costs more than
    // it saves (gemma2_decode +5, fp8_kv +2 us).
    if (kTrimStep && !a.alibi && t0 >= max(W.wlo, vis_lo) &&
        t0 + kStepTokens - 1 <= min(W.whi, vis_hi)) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sc[tile][i] * a.logit_scale;
          if constexpr (CAP) v = a.cap * tanh_from_exp(v * a.inv_cap) * kLog2e;
          x[4 * tile + i] = v;
          mx = fmaxf(mx, v);
        }
      }
    } else {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 8 * g + 4 * tile + i;
          float v = sc[tile][i] * a.logit_scale;
          v = __builtin_fmaf(col_slope, (float)(t - col_hi), v);   // ALiBi
          if constexpr (CAP) v = a.cap * tanh_from_exp(v * a.inv_cap) * kLog2e;
          v = (t >= lo && t <= hi) ? v : -INFINITY;
          x[4 * tile + i] = v;
          mx = fmaxf(mx, v);
        }
      }
    }
    mx = wave_max_over_groups(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = fast_exp2(x[e] - m_use);
      psum += x[e];
    }
    d_run = d_run * alpha + psum;
    // P^T in the operand type as an unevaluated sum hi + lo: hi = p rounded,
    // lo = the rest rounded. P.V then errs by about 2^-16 of |p| (bf16) rather
    // than the 2^-9 of hi alone, which, with one or two dominant tokens, would
    // be as large as the output's own rounding. With RoPE the rotated q and
    // keys are rounded to the operand type already, which moves each p by as
    // much; hi alone serves there (the second MFMA and its operand would cost
    // that VALU-bound instance 2 % and buy no accuracy).
    constexpr bool kPLo = !ROPE;
    u32x4 pw, pwl;
#pragma unroll
    for (int i = 0; i < 4; ++i) pw[i] = O::pack(x[2 * i], x[2 * i + 1]);
    const v8 pop = __builtin_bit_cast(v8, pw);
    if constexpr (kPLo) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pwl[i] = O::pack(x[2 * i] - (float)pop[2 * i], x[2 * i + 1] - (float)pop[2 * i + 1]);
    }
    const v8 pop_lo = __builtin_bit_cast(v8, pwl);
    // the output sums to the new maximum: with kTrimStep here and only when
    // some column's maximum moved (alpha 1 everywhere gives the same bits),
    // else with each MFMA below
    if constexpr (kTrimStep) {
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int b = 0; b < G_::kPvMfma; ++b) acc[b] *= alpha;
      }
    }
    // ---- O^T += V^T P^T, two MFMAs (hi, lo) per 16 hd columns
#pragma unroll
    for (int b = 0; b < G_::kPvMfma; ++b) {
      v8 vop;
      if constexpr (KV8) {
        // lane (n, g): column 16b+n of rows 8g..8g+7 from one 8-bit transpose read
        const char* src = vl + (8 * g + (n >> 1)) * G_::kVPitch + 16 * b + 8 * (n & 1);
        i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((PKD_LDS i32x2*)(src));
        vop = e4m3x8<QBF16>((unsigned)r[0], (unsigned)r[1]);
      } else {
        const char* src0 = vl + (8 * g + (n >> 2)) * G_::kVPitch + 2 * (16 * b + 4 * (n & 3));
        trf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PKD_LDS trf16x4*)(src0));
        trf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((PKD_LDS trf16x4*)(src0 + 4 * G_::kVPitch));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        vop = __builtin_bit_cast(v8, (u32x4){l2[0], l2[1], h2[0], h2[1]});
      }
      f32x4 c = acc[b];
      if constexpr (!kTrimStep) {
        c[0] *= alpha; c[1] *= alpha; c[2] *= alpha; c[3] *= alpha;
      }
      if constexpr (kPLo) c = O::mfma(vop, pop_lo, c);
      acc[b] = O::mfma(vop, pop, c);
    }
  };
  auto consume = [&](const Win& W, int s, const StepRegs<kNP>& st) {
    stage(W, s, st);
    attend(W, s);
  };

  // the partial outputs, for 16-byte device-coherent stores
  const __amdgpu_buffer_rsrc_t ws_o_rsrc =
      make_rsrc(a.ws_o, (uint32_t)min<size_t>(a.ws_o_bytes, 0xFFFFFFF0u));

  // reserve slots of all workgroups, two each (by unit parity)
  const int nslots = 2 * (int)gridDim.x;
  // the ticket counter (4 bytes)
  const __amdgpu_buffer_rsrc_t cnt_rsrc = make_rsrc(a.counters, 4);
  const __amdgpu_buffer_rsrc_t res_rsrc = make_rsrc(a.reserve, (uint32_t)nslots * 4);

  // ---- Units form a pipeline per workgroup. While unit `cur` is attended,
  // the item and the page ids of the next unit `nxt` are loaded, and the
  // last load issue of cur's step loop is nxt's first step, so that cur's
  // end-of-unit work (wavefront merge, outputs, merge of split requests)
  // overlaps with those loads. A workgroup holds at most one unit beyond
  // the current one. It takes the ticket for the unit after that in the
  // last pass of the current unit's steps, early enough for the ticket to
  // return by the unit's end, late enough that near the end of the queue
  // the last units go to the workgroups about to need them.
  // Its first two units are items blockIdx.x and blockIdx.x + gridDim.x
  // (a graph plan's grid may exceed the item count); later ones are tickets
  // from the plan's counter, offset by twice the grid size. A workgroup
  // takes tickets while it holds a unit nxt, so each workgroup whose second
  // unit exists takes the valid tickets it gets and then exactly one past
  // the end: a launch takes max(0, N - 2 grid) + max(0, min(grid, N - grid))
  // tickets (N items), and the workgroup that takes the last one resets the
  // counter for the next launch.
  //
  // A long enough held unit nxt (an item below a.steal_limit) is published
  // in a reserve slot from the time its ticket is known until cur's last
  // issue, when thread 0 claims it. A workgroup whose own chain has run out
  // takes published units of others (a "steal"); an owner that finds its
  // claimed unit stolen (told at the unit's first step) masks the rest of
  // it (no arithmetic, no outputs), which keeps its pipeline going. Every
  // unit is processed by exactly one workgroup. Thread 0 alone publishes
  // and claims, so its claim is ordered after its publication, and its
  // publication after its previous claim of the slot (whose result it has
  // read).
  int cur = blockIdx.x;
  int nxt = cur + (int)gridDim.x;
  if (threadIdx.x == 0 && nxt < a.steal_limit)
    __hip_atomic_store(a.reserve + 2 * blockIdx.x + 1, nxt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  StepRegs<kNP> A, B;
  Unit cu;
  unsigned itemv;
  unsigned claim = 0;     // what thread 0's claim of cur returned
  bool claimed = false;   // cur was published and claimed by this workgroup
  int buf = 0, par = 0;

  // A published unit of another workgroup, or -1 when none is left. Slots
  // are scanned from this workgroup's right neighbour on, so that thieves
  // spread over the owners; a lost compare-and-swap scans again.
  auto steal = [&]() {
    // an opaque copy of the thread index, so that the scan's addresses are
    // computed here and not kept in registers through the decode loop
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));
    for (int tries = 0; tries < 4; ++tries) {
      // (scan position << 32 | unit) of the first published slot, by an LDS
      // minimum over the workgroup
      if (tid == 0) s_steal = ~0ull;
      lds_barrier();
      unsigned long long best = ~0ull;
      for (int i0 = 0; i0 < nslots; i0 += 8 * kWaves * 64) {
        // all eight loads in flight at once (positions past the end load
        // the last slot again and are ignored)
        unsigned v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = min(i0 + k * kWaves * 64 + tid, nslots - 1);
          int slot = 2 * (int)blockIdx.x + 2 + i;
          slot = slot >= nslots ? slot - nslots : slot;
          v[k] = __builtin_amdgcn_raw_buffer_load_b32(res_rsrc, (uint32_t)slot * 4u, 0, kCoherentPolicy);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int i = i0 + k * kWaves * 64 + tid;
          const unsigned long long key = ((unsigned long long)i << 32) | v[k];
          best = i < nslots && v[k] < kMaxItems && key < best ? key : best;
        }
      }
      if (best != ~0ull) atomicMin(&s_steal, best);
      lds_barrier();
      best = s_steal;
      lds_barrier();
      const int i = __builtin_amdgcn_readfirstlane((int)(best >> 32));
      const int v = __builtin_amdgcn_readfirstlane((int)(unsigned)best);
      if (i < 0) return -1;                 // nothing published
      int slot = 2 * (int)blockIdx.x + 2 + i;
      slot = slot >= nslots ? slot - nslots : slot;
      if (tid == 0) s_steal = atomicCAS(a.reserve + slot, v, (int)kStolen) == v;
      lds_barrier();
      const bool won = __builtin_amdgcn_readfirstlane((int)s_steal) != 0;
      lds_barrier();
      if (won) return v;
    }
    return -1;
  };

  for (;;) {
    // (a graph plan's launch may hold more workgroups than units)
    if (cur >= a.num_items) break;
    // ---- chain start: cur's item, first page window and first step, its q,
    // and the item of nxt
    cu = unit_from_lanes(load_item_lanes(a.items, cur, lane));
    {
      const Win W = first_window(cu, s_pages[buf]);
      const int wpages = (W.whi >> lp) - W.wpage0 + 1;
      const int32_t* pidx = a.indices + cu.page_base;
      for (int i = threadIdx.x; i < wpages; i += kWaves * 64) s_pages[buf][i] = pidx[W.wpage0 + i];
    }
    lds_barrier();
    issue(first_window(cu, s_pages[buf]), wave, A);
    load_q(cu);
    itemv = load_item_lanes(a.items, min(nxt, last_item), lane);   // item of nxt

    while (cur < a.num_items) {
      // ---- unit start: cur's first step is in flight in A, its q in bq, the
      // item of nxt in itemv
      // the ticket for the unit after nxt, taken by thread 0 in the last
      // pass of cur's steps (none once the tickets are spent)
      unsigned tk = 0;
      // nxt (read after cur's first step): its first page window (the first
      // kWaves*64 pages now, to LDS at cur's end; more, rarely, then), and the
      // pages of this wave's first step of nxt (for the hand-over issue)
      Unit nu;
      Win Wn;
      int nwpages, pgn, hpg[kRowBlocks];
      const int32_t* npidx;
      auto load_next = [&]() {
        nu = unit_from_lanes(itemv);
        Wn = first_window(nu, s_pages[buf ^ 1]);
        nwpages = (Wn.whi >> lp) - Wn.wpage0 + 1;
        npidx = a.indices + nu.page_base;
        pgn = npidx[Wn.wpage0 + min((int)threadIdx.x, nwpages - 1)];
#pragma unroll
        for (int b = 0; b < kRowBlocks; ++b) hpg[b] = npidx[token(Wn, wave, lrow + kRowsPer * b) >> lp];
      };

      m_run = -INFINITY;
      d_run = 0.0f;
      q_turned = false;
      col_hi = cu.qpos + col_tok;
      col_lo = a.window_left < 0 ? 0 : col_hi - a.window_left;
      vis_hi = cu.qpos;
      vis_lo = a.window_left < 0 ? 0 : cu.qpos + a.q_len - 1 - a.window_left;
      if (a.alibi) {
        // the ALiBi paper's slopes over the q heads (n2: the power of two
        // at or below num_qo_heads; the heads past it take odd powers of
        // 2^(-4/n2))
        const int hq = cu.kv_head * group + col_head;
        const int lg2 = 31 - __builtin_clz(a.num_qo_heads);
        const int n2 = 1 << lg2;
        // (dividing by the power of two n2 is the exact product with 2^-lg2)
        const float inv_n2 = __builtin_ldexpf(1.0f, -lg2);
        const float ex = hq < n2 ? -8.0f * (float)(hq + 1) * inv_n2
                                 : -4.0f * (float)(2 * (hq - n2) + 1) * inv_n2;
        col_slope = fast_exp2(ex) * (CAP ? 1.0f : kLog2e);
      }
#pragma unroll
      for (int b = 0; b < G_::kPvMfma; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      const int base = cu.tb & ~(kStepTokens - 1);
      const int nsteps = (cu.te - base + kStepTokens - 1) / kStepTokens;
      const int qh0 = cu.kv_head * group;

      // Steps are processed in windows whose pages fit the LDS page table. A
      // wave takes every kWaves-th step of a window, one step ahead of the
      // loads (buffers A and B alternate); the count is padded to an even
      // number >= 2 with steps past the window, which read clamped rows and
      // whose tokens are all masked (no effect on the state). The first and
      // the last step are peeled, and each pass of the loop between them
      // issues and consumes two steps, so that the compiler's wait before a
      // step covers that step's loads only. The last issue of the last
      // window is the next unit's first step when there is a next unit.
      bool drop = false;      // cur was taken by another workgroup: no outputs
      int w0 = 0;
      do {
        int w1 = min(nsteps, w0 + win_steps);
        Win W;
        W.base = base;
        W.wlo = max(cu.tb, base + w0 * kStepTokens);
        W.whi = min(cu.te, base + w1 * kStepTokens) - 1;
        W.wpage0 = W.wlo >> lp;
        W.sp = s_pages[buf];
        W.head_off = (int64_t)cache_head(cu.kv_head) * a.head_stride;
        const int s0 = w0 + ((wave - w0) % kWaves + kWaves) % kWaves;
        const int mine = s0 < w1 ? (w1 - s0 + kWaves - 1) / kWaves : 0;
        int m2 = max(2, (mine + 1) & ~1);
        if (w0 > 0) {
          // a later window: its pages replace the previous window's
          lds_barrier();
          const int wpages = (W.whi >> lp) - W.wpage0 + 1;
          const int32_t* pidx = a.indices + cu.page_base;
          for (int i = threadIdx.x; i < wpages; i += kWaves * 64) s_pages[buf][i] = pidx[W.wpage0 + i];
          lds_barrier();
          issue(W, s0, A);
        }
        if constexpr (kSingle) {
          // one buffer: step s is staged, the next step's loads leave, then
          // s is attended; a wave with no step here runs one padding step
          int n1 = max(1, mine);
          for (int k = 0; k < n1; ++k) {
            const int s = s0 + k * kWaves;
            stage(W, s, A);
            __builtin_amdgcn_sched_barrier(0);
            if (k == 0) {
              load_next();
              if (w0 == 0 && claimed) {
                // the claim of cur returned with its first step (as in the
                // two-buffer loop below): stolen means no outputs
                if (threadIdx.x == 0) s_drop = (claim & kStolen) != 0;
                lds_barrier();
                drop = __builtin_amdgcn_readfirstlane(s_drop) != 0;
                if (drop) {
                  W.whi = W.wlo;
                  n1 = 1;
                  w1 = nsteps;
                }
              }
            }
            if (k + 1 < n1) {
              issue(W, s + kWaves, A);
            } else {
              // the last step: thread 0 claims nxt and takes the ticket (in
              // range only after the last window, as below), then the next
              // unit's first step, or a clamped padding step, is issued
              const bool hand = w1 == nsteps && nxt < a.num_items;
              const uint32_t coff = hand && nxt < a.steal_limit && threadIdx.x == 0
                                        ? (uint32_t)(2 * blockIdx.x + (par ^ 1)) * 4u
                                        : 0x80000000u;
              claim = (unsigned)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32((int)kClaimStep, res_rsrc,
                                                                               coff, 0, 0);
              const uint32_t toff = hand && threadIdx.x == 0 ? 0u : 0x80000000u;
              tk = (unsigned)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, cnt_rsrc, toff, 0, 0);
              int cc[kRowBlocks], pp[kRowBlocks];
#pragma unroll
              for (int b = 0; b < kRowBlocks; ++b) {
                const int cw = token(W, s + kWaves, lrow + kRowsPer * b);
                const int pw = W.sp[(cw >> lp) - W.wpage0];
                cc[b] = hand ? token(Wn, wave, lrow + kRowsPer * b) : cw;
                pp[b] = hand ? hpg[b] : pw;
              }
              issue_rows(hand ? Wn : W, cc, pp, A);
            }
            __builtin_amdgcn_sched_barrier(0);
            attend(W, s);
            __builtin_amdgcn_sched_barrier(0);
          }
          w0 = w1;
          continue;
        }
        // The scheduling barriers keep each issue ahead of the step it overlaps:
        // the loads must leave before the wait for the previous step's rows.
        issue(W, s0 + kWaves, B);
        __builtin_amdgcn_sched_barrier(0);
        consume(W, s0, A);
        __builtin_amdgcn_sched_barrier(0);
        load_next();                       // again (same loads) in a later window
        if (w0 == 0 && claimed) {
          // The claim of cur, made before its first step was issued, has
          // returned with that step: tell the wavefronts whether cur was
          // stolen. Then every later row is clamped to the first token (the
          // only unmasked one), the step count is the minimum and the unit
          // ends with this window.
          if (threadIdx.x == 0) s_drop = (claim & kStolen) != 0;
          lds_barrier();
          drop = __builtin_amdgcn_readfirstlane(s_drop) != 0;
          if (drop) {
            W.whi = W.wlo;
            m2 = 2;
            w1 = nsteps;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        int j = 1;
        // (a guarded do-while: as a plain while loop the compiler keeps more
        // registers live across it)
        if (m2 > 2) do {
          issue(W, s0 + (j + 1) * kWaves, A);
          {
            // the ticket: in range for thread 0 in the last pass of the last
            // window only (the other lanes and passes do nothing)
            const uint32_t toff = j + 3 >= m2 && w1 == nsteps && nxt < a.num_items && threadIdx.x == 0
                                      ? 0u : 0x80000000u;
            tk = (unsigned)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, cnt_rsrc, toff, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          consume(W, s0 + j * kWaves, B);
          __builtin_amdgcn_sched_barrier(0);
          issue(W, s0 + (j + 2) * kWaves, B);
          __builtin_amdgcn_sched_barrier(0);
          consume(W, s0 + (j + 1) * kWaves, A);
          __builtin_amdgcn_sched_barrier(0);
          j += 2;
        } while (j + 1 < m2);
        {
          // last issue: the next unit's first step after the last window if
          // there is a next unit, else a clamped padding step of this window
          const bool hand = w1 == nsteps && nxt < a.num_items;
          // Thread 0 claims nxt if it was published (after the last window);
          // the other lanes, and earlier windows, fall outside the buffer and
          // do nothing. The result is read with nxt's first step.
          const uint32_t coff = hand && nxt < a.steal_limit && threadIdx.x == 0
                                    ? (uint32_t)(2 * blockIdx.x + (par ^ 1)) * 4u
                                    : 0x80000000u;
          claim = (unsigned)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32((int)kClaimStep, res_rsrc,
                                                                           coff, 0, 0);
          {
            // the ticket of a last window of two steps, whose loop above has
            // no pass (out of range, and so nothing, in every other case)
            const uint32_t toff = m2 == 2 && hand && threadIdx.x == 0 ? 0u : 0x80000000u;
            const unsigned t2 = (unsigned)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, cnt_rsrc, toff, 0, 0);
            tk = m2 == 2 ? t2 : tk;
          }
          int cc[kRowBlocks], pp[kRowBlocks];
#pragma unroll
          for (int b = 0; b < kRowBlocks; ++b) {
            const int cw = token(W, s0 + m2 * kWaves, lrow + kRowsPer * b);
            const int pw = W.sp[(cw >> lp) - W.wpage0];
            cc[b] = hand ? token(Wn, wave, lrow + kRowsPer * b) : cw;
            pp[b] = hand ? hpg[b] : pw;
          }
          issue_rows(hand ? Wn : W, cc, pp, A);
        }
        __builtin_amdgcn_sched_barrier(0);
        consume(W, s0 + (m2 - 1) * kWaves, B);
        __builtin_amdgcn_sched_barrier(0);
        w0 = w1;
      } while (w0 < nsteps);

      // ---- end of cur: nxt's pages and the ticket, this wave's state to LDS
      if ((int)threadIdx.x < nwpages) s_pages[buf ^ 1][threadIdx.x] = pgn;
      for (int i = threadIdx.x + kWaves * 64; i < nwpages; i += kWaves * 64)
        s_pages[buf ^ 1][i] = npidx[Wn.wpage0 + i];
      if (threadIdx.x == 0) {
        s_ticket[par] = nxt < a.num_items ? 2 * (int)gridDim.x + (int)tk : a.num_items;
        // the last ticket of the launch: every ticket has been taken, so the
        // counter can be reset for the next launch
        const int grid = (int)gridDim.x;
        const int last_ticket =
            max(0, a.num_items - 2 * grid) + max(0, min(grid, a.num_items - grid)) - 1;
        if (nxt < a.num_items && (int)tk == last_ticket)
          __hip_atomic_store(a.counters, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      d_run = wave_sum_over_groups(d_run);
      float* sacc = reinterpret_cast<float*>(vl);   // [16 rows][HD], own region
      if (n < cols) {
#pragma unroll
        for (int b = 0; b < G_::kPvMfma; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[n * HD + 16 * b + 4 * g + i] = acc[b][i];
        if (g == 0) {
          // (the row index, n, is taken from the hardware lane id here, so
          // that neither it nor these two addresses are kept in registers
          // through the step loop)
          unsigned id;
          asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(id));
          const int row = (int)(id & 15);
          s_m[wave][row] = m_run;
          s_d[wave][row] = d_run;
        }
      }
      lds_barrier();
      // the unit after nxt: its item, to be read during nxt
      const int nxt2 = __builtin_amdgcn_readfirstlane(s_ticket[par]);
      if (threadIdx.x == 0 && nxt2 < a.steal_limit)
        __hip_atomic_store(a.reserve + 2 * blockIdx.x + par, nxt2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // ---- merge the wavefronts' states, in wavefront order: one float4
      // column of one head per thread
      constexpr int cols4 = HD / 4;
      for (int e = threadIdx.x; !drop && e < cols * cols4; e += kWaves * 64) {
        const int h = e / cols4, c = 4 * (e - h * cols4);
        const int qj = h / group, gh = h - qj * group;   // query token, head of row h
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        float den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float mw = s_m[w][h];
          const float sw = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
          num += sw * *reinterpret_cast<const f32x4*>(smem + w * G_::kWaveLds + (h * HD + c) * 4);
          den += sw * s_d[w][h];
        }
        const int qh = qh0 + gh;
        if (cu.partial < 0 && a.sinks != nullptr) {
          // the q head's sink joins the softmax (one more logit, no value)
          const float s2 = a.sinks[qh] * kLog2e;
          const float Mn = fmaxf(M, s2);
          if (Mn != -INFINITY) {
            const float r = M == -INFINITY ? 0.0f : fast_exp2(M - Mn);
            den = den * r + (s2 == -INFINITY ? 0.0f : fast_exp2(s2 - Mn));
            num *= r;
            M = Mn;
          }
        }
        // (a row with no visible token in this unit, possible only for an
        // early query token of a split request, is an empty state)
        f32x4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = den > 0.0f ? num[i] / den * a.v_scale : 0.0f;
        const float lse2 = den > 0.0f ? M + __builtin_amdgcn_logf(den) : -INFINITY;
        if (cu.partial < 0) {
          const size_t orow = ((size_t)cu.request * a.q_len + qj) * a.num_qo_heads + qh;
          store_out4(a.o, orow * HD + c, ov, a.o_bf16);
          if (a.lse != nullptr && c == 0) a.lse[orow] = lse2 * kLn2;
        } else {
          // device-coherent stores: the merging workgroup may sit on another XCD
          const size_t wrow = ((size_t)cu.partial * a.q_len + qj) * a.num_qo_heads + qh;
          store_coherent4(ws_o_rsrc, (uint32_t)(wrow * HD + c) * 4, ov);
          if (c == 0) store_coherent(a.ws_lse + wrow, lse2);
        }
      }
      if (!drop && cu.partial >= 0) {
        // Count this unit once its partial state has reached the device-coherent
        // level. Units are merged in runs of kMergeGroup consecutive units, then
        // the runs: the workgroup that counts the last unit of a run merges the
        // run into the run's first slot (or straight into o if the request has
        // a single run), and the one that counts the last run merges the runs.
        // Which workgroups these are does not change the result.
        wait_vector_memory();
        lds_barrier();
        const int n = cu.num_chunks;
        const int run = cu.chunk / kMergeGroup;
        const int runs = (n + kMergeGroup - 1) / kMergeGroup;
        const int run_len = min(kMergeGroup, n - run * kMergeGroup);
        const int slot0 = cu.partial - cu.chunk;
        int32_t* cnt = a.merge_counters +
                       ((size_t)cu.request * a.num_kv_heads + cu.kv_head) * a.merge_stride;
        if (threadIdx.x == 0) s_last = atomicAdd(cnt + 1 + run, 1) == run_len - 1;
        lds_barrier();
        if (__builtin_amdgcn_readfirstlane(s_last)) {
          const int rslot = slot0 + run * kMergeGroup;
          merge_partials<HD>(a, cu.request, qh0, rslot, 1, run_len, runs == 1 ? -1 : rslot);
          if (threadIdx.x == 0) atomicExch(cnt + 1 + run, 0);   // ready for the next launch
          if (runs > 1) {
            wait_vector_memory();
            lds_barrier();
            if (threadIdx.x == 0) s_last = atomicAdd(cnt, 1) == runs - 1;
            lds_barrier();
            if (__builtin_amdgcn_readfirstlane(s_last)) {
              merge_partials<HD>(a, cu.request, qh0, slot0, kMergeGroup, runs, -1);
              if (threadIdx.x == 0) atomicExch(cnt, 0);
            }
          }
        }
      }
      load_q(nu);
      itemv = load_item_lanes(a.items, min(nxt2, last_item), lane);
      lds_barrier();                       // LDS free for the next unit
      claimed = nxt < a.steal_limit;
      cur = nxt;
      cu = nu;
      nxt = nxt2;
      par ^= 1;
      buf ^= 1;
    }
    // ---- the chain has run out: go on with a unit taken from another one
    if (a.steal_limit == 0) break;
    cur = steal();
    if (cur < 0) break;
    nxt = a.num_items;
    claimed = false;
  }
}

// merge_states: one wavefront per row folds the row's num_states states
// (v[row][k][:], s[row][k], natural-log LSE).
//
// Lanes are split into `cl` chunk lanes x (hd/4) column lanes (float4 each);
// chunk lane kk folds states kk, kk+cl, ... in ascending order, then the cl
// partial sums are added in a fixed butterfly. The sum order depends only on
// num_states, so the result is deterministic.
__global__ __launch_bounds__(kMergeRowsPerBlock * 64) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.num_rows) return;
  const int hd = a.head_dim;
  const int nst = a.num_states;
  const float* vs = a.v + (size_t)row * nst * hd;
  const float* ss = a.s + (size_t)row * nst;
  float M = -INFINITY;
  for (int k = lane; k < nst; k += 64) M = fmaxf(M, ss[k] * kLog2e);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  auto weight = [&](int k) {
    const float sk = ss[k] * kLog2e;
    return sk == -INFINITY ? 0.0f : fast_exp2(sk - M);
  };
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int k = lane; k < nst; k += 64) den += weight(k);
    for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off);
  }
  auto put = [&](size_t idx, float ov) {
    if (a.out_dtype == PKD_F32)
      reinterpret_cast<float*>(a.v_out)[idx] = ov;
    else
      store_out(a.v_out, idx, ov, a.out_dtype == PKD_BF16);
  };
  const int ng = hd >> 2;                    // float4 columns
  const bool vec = (hd & 3) == 0 && hd <= 256 && (ng & (ng - 1)) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.v) & 15) == 0;
  if (vec) {
    const int cl = 64 / ng;                  // chunk lanes (>= 1)
    const int cg = lane % ng, kk = lane / ng;
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY && kk < cl) {
#pragma unroll 8
      for (int k = kk; k < nst; k += cl) {
        const float wk = weight(k);
        const f32x4 x = *reinterpret_cast<const f32x4*>(vs + (size_t)k * hd + 4 * cg);
        acc4 += wk * x;
      }
    }
    for (int off = ng; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc4[e] += __shfl_xor(acc4[e], off);
    }
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        put((size_t)row * hd + 4 * cg + e, M == -INFINITY ? 0.0f : acc4[e] / den);
    }
  } else {
    for (int c = lane; c < hd; c += 64) {
      float num = 0.0f;
      if (M != -INFINITY)
        for (int k = 0; k < nst; ++k) num += weight(k) * vs[(size_t)k * hd + c];
      put((size_t)row * hd + c, M == -INFINITY ? 0.0f : num / den);
    }
  }
  if (a.s_out != nullptr && lane == 0)
    a.s_out[row] = M == -INFINITY ? -INFINITY : (M + __builtin_amdgcn_logf(den)) * kLn2;
}

// The kernel instance for (head_dim, q type, KV type, soft cap, RoPE, one
// K/V buffer).
using DecodeFn = void (*)(DecodeArgs);

template <bool QBF16, bool KV8, bool CAP, bool ROPE>
DecodeFn pick_hd(int hd, bool single) {
  switch (hd) {
    case 64: return decode_kernel<64, QBF16, KV8, CAP, ROPE, false>;
    case 128:
      if constexpr (ROPE) {
        if (single) return decode_kernel<128, QBF16, KV8, CAP, true, true>;
      }
      return decode_kernel<128, QBF16, KV8, CAP, ROPE, false>;
    default:
      if constexpr (ROPE && !KV8) {
        if (single) return decode_kernel<256, QBF16, KV8, CAP, true, true>;
      }
      return decode_kernel<256, QBF16, KV8, CAP, ROPE, false>;
  }
}

template <bool ROPE>
DecodeFn pick_types(const pkd_plan_params& p) {
  const bool cap = p.logits_soft_cap > 0.0f;
  const bool qbf = p.q_dtype == PKD_BF16;
  const bool kv8 = p.kv_dtype == PKD_E4M3;
  const bool one = decode_single(p);
  const int hd = p.head_dim;
  if (qbf) {
    if (kv8) return cap ? pick_hd<true, true, true, ROPE>(hd, one) : pick_hd<true, true, false, ROPE>(hd, one);
    return cap ? pick_hd<true, false, true, ROPE>(hd, one) : pick_hd<true, false, false, ROPE>(hd, one);
  }
  if (kv8) return cap ? pick_hd<false, true, true, ROPE>(hd, one) : pick_hd<false, true, false, ROPE>(hd, one);
  return cap ? pick_hd<false, false, true, ROPE>(hd, one) : pick_hd<false, false, false, ROPE>(hd, one);
}

DecodeFn pick_kernel(const pkd_plan_params& p) {
  return p.pos_encoding_mode == PKD_POS_ROPE_LLAMA ? pick_types<true>(p) : pick_types<false>(p);
}

}  // namespace

// Launches return the status of their own launch call (hipLaunchKernel),
// so an earlier, unrelated error pending on the thread is neither reported
// as theirs nor cleared.
int launch_decode(const pkd_plan_params& p, const DecodeArgs& a, int32_t num_workgroups,
                  void* stream) {
  if (num_workgroups <= 0) return hipSuccess;
  DecodeArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(pick_kernel(p)), dim3(num_workgroups),
                         dim3(kWaves * 64), params, 0, reinterpret_cast<hipStream_t>(stream));
}

int32_t decode_wgs_per_cu(const pkd_plan_params& p) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, reinterpret_cast<const void*>(pick_kernel(p)), kWaves * 64, 0) != hipSuccess)
    return 0;
  return blocks;
}

// ---------------------------------------------------------------------------
// Static workspace of pkd_run_static_workspace: split-KV partial states of
// one run at a time per GPU. Each GPU the library runs on holds its own
// copy, at its own device address, until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: only the
// address hipGetSymbolAddress returns is passed to kernels.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

int static_scratch_resolve(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device] != nullptr) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch[device] = ptr;
  return hipSuccess;
}

void* static_scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.num_rows <= 0) return hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((a.num_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock);
  MergeArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(merge_kernel), grid,
                         dim3(kMergeRowsPerBlock * 64), params, 0, s);
}

}  // namespace pkd

