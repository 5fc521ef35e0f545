// HIP kernels for gfx950 (CDNA4): paged-KV batch decode and the log-sum-exp
// merge of split-KV partial states.
//
// What is computed is the run() of flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper
// ("FlashInfer attention kernels" page): for every work item (request, kv head,
// chunk of tokens) the G query rows of that kv head attend the chunk's keys and
// values, found through the CSR page table, with sm_scale, the optional
// logits_soft_cap (cap*tanh(x/cap)) and the window already folded into the
// item's token range by the planner. The merge folds per-chunk states by
// log-sum-exp (the merge_states step named with plan()'s fixed_split_size).
//
// Design (MI355X-first, not the page's):
//  * One workgroup of 4 wavefronts per work item. Wavefront w takes the
//    32-token steps w, w+4, ... of the item; the four partial states are
//    merged in LDS in wavefront order at the end, so the result depends only
//    on the item's token range (bitwise batch invariance under a fixed split).
//  * q.K^T on MFMA 16x16x32: K rows are the A operand and arrive straight
//    from HBM in 16-byte loads (one row segment per lane); the G <= 16 query
//    rows of the kv head are the B operand (columns past G are zero).
//    Result lane l holds the logits of tokens 8*(l/16)+4*tile+i for head l%16.
//  * P.V on MFMA as O^T = V^T P^T. P^T is exactly what each lane holds after
//    the softmax, so it needs no data movement; V^T comes from a per-wave LDS
//    copy of the step's V rows read with ds_read_b64_tr_b16 (16-bit V) or
//    ds_read_b64_tr_b8 (E4M3 V, converted after the read).
//  * Online softmax in base 2 (v_exp_f32): one running max per head, made
//    uniform across the four lane groups with two cross-lane maxima per step;
//    the running sum stays per lane and is reduced once at the end.
//  * Tokens outside [token_begin, token_end) are masked by a select, and their
//    loads are clamped onto the chunk's own tokens, so stale or NaN slots of a
//    page are never read.
#include <hip/hip_runtime.h>

#include <cmath>

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

// Operand type of the MFMA: the q dtype (fp8 K/V are converted to it).
template <bool BF16>
struct Op;

template <>
struct Op<false> {
  using v8 = f16x8;
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
  __device__ static f32x4 mfma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static unsigned pack(float a, float b) {
    bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(unsigned, h);
  }
};

// Eight E4M3 codes (little-endian in two dwords) -> eight operand values.
// v_cvt_pk_f32_fp8 decodes OCP E4M3 exactly; the values are exact in fp16 and
// bf16 too, so the second conversion does not round.
template <bool BF16>
__device__ __forceinline__ typename Op<BF16>::v8 e4m3x8(unsigned lo, unsigned hi) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  u32x4 r;
  r[0] = Op<BF16>::pack(a[0], a[1]);
  r[1] = Op<BF16>::pack(b[0], b[1]);
  r[2] = Op<BF16>::pack(c[0], c[1]);
  r[3] = Op<BF16>::pack(d[0], d[1]);
  return __builtin_bit_cast(typename Op<BF16>::v8, r);
}

__device__ __forceinline__ float wave_max_over_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
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
  // Steps of K/V rows held in registers: the next step's loads are issued
  // before the current step is computed.
  static constexpr int kStages = 2;
  // LDS row pitch of the V copy; the pad staggers rows across banks.
  static constexpr int kVPitch = kRowBytes + (KV8 ? 16 : 32);
  static constexpr int kVBytes = kStepTokens * kVPitch;
  static constexpr int kMergeBytes = kMaxGroup * HD * 4;
  static constexpr int kWaveLds = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
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

// The item list is read-only for the whole launch: read it through the
// constant address space so that it arrives in scalar registers.
__device__ __forceinline__ pkd_work_item load_item(const pkd_work_item* items, int k) {
  const __attribute__((address_space(4))) int32_t* w =
      (const __attribute__((address_space(4))) int32_t*)(items + k);
  pkd_work_item it;
  it.request = w[0];
  it.kv_head = w[1];
  it.token_begin = w[2];
  it.token_end = w[3];
  it.page_base = w[4];
  it.partial = w[5];
  it.chunk = w[6];
  it.reserved = w[7];
  return it;
}

template <int NP>
struct StepRegs {
  u32x4 k[2][NP];
  u32x4 v[2][NP];
};

template <int HD, bool QBF16, bool KV8, bool CAP>
__global__ __launch_bounds__(kWaves * 64, decode_waves_per_simd(HD, KV8)) void decode_kernel(DecodeArgs a) {
  using G_ = Geo<HD, KV8>;
  using O = Op<QBF16>;
  using v8 = typename O::v8;
  __shared__ __attribute__((aligned(16))) char smem[kWaves * G_::kWaveLds];
  __shared__ int s_pages[kPageWin];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_d[kWaves][kMaxGroup];

  const int lane = threadIdx.x & 63;
  // wave-uniform (an SGPR), so that the step loop branches on scalars
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;        // MFMA row (tile token) / column (q head)
  const int g = lane >> 4;        // lane group
  const int group = a.group;
  // Work items are taken in order from the plan's counter, one at a time per
  // workgroup; the next one is requested when the current one starts.
  __shared__ int s_item;
  if (threadIdx.x == 0) s_item = atomicAdd(&a.counters[0], 1);
  __syncthreads();
  int item = __builtin_amdgcn_readfirstlane(s_item);   // uniform: scalar loads, scalar branches
  while (item < a.num_items) {
  // the item list is read-only for the whole launch: scalar loads
  const pkd_work_item it = load_item(a.items, item);
  int next = 0;
  if (threadIdx.x == 0) next = atomicAdd(&a.counters[0], 1);
  const int tb = it.token_begin, te = it.token_end;
  const int qh0 = it.kv_head * group;
  const int lp = a.log2_page;

  // ---- q operand: head n of this kv head (zero past G)
  v8 bq[G_::kQkMfma];
  {
    const _Float16* qrow = reinterpret_cast<const _Float16*>(a.q) +
                           ((size_t)it.request * a.num_qo_heads + qh0 + n) * HD;
#pragma unroll
    for (int j = 0; j < G_::kQkMfma; ++j) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (n < group) x = *reinterpret_cast<const u32x4*>(qrow + qk_hd<KV8>(j, g));
      bq[j] = __builtin_bit_cast(v8, x);
    }
  }

  const int base = tb & ~(kStepTokens - 1);
  const int nsteps = (te - base + kStepTokens - 1) / kStepTokens;
  // Token (within a step) whose K row lane n loads for tiles 0 and 1: tile
  // rows 4g'+i then map to tokens 8g'+4*tile+i.
  const int tau0 = 8 * (n >> 2) + (n & 3);
  const int tau1 = tau0 + 4;
  const int page_mask = (1 << lp) - 1;
  const int32_t* pidx = a.indices + it.page_base;
  const int64_t head_off = (int64_t)it.kv_head * a.head_stride;
  const char* kbase = reinterpret_cast<const char*>(a.k);
  const char* vbase = reinterpret_cast<const char*>(a.v);
  char* vl = smem + wave * G_::kWaveLds;

  float m_run = -INFINITY;   // running max (base-2 logits) of head n
  float d_run = 0.0f;        // this lane's share of the running sum
  f32x4 acc[G_::kPvMfma];
#pragma unroll
  for (int b = 0; b < G_::kPvMfma; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Tokens of the current LDS page window are [wlo, whi]; loads of tokens
  // outside it (masked ones, and the surplus prefetch past the last step) are
  // clamped onto it, so every load reads a valid row of the item.
  int wlo = tb, whi = te - 1;
  int wpage0 = 0;            // first page of the current LDS window
  auto clampw = [&](int t) { return min(max(t, wlo), whi); };

  // Issue the K/V loads of step s into st (page ids from the LDS window).
  auto issue = [&](int s, StepRegs<G_::kPieces>& st) {
    const int t0 = base + s * kStepTokens;
    const int c0 = clampw(t0 + tau0), c1 = clampw(t0 + tau1);
    const int pg0 = s_pages[(c0 >> lp) - wpage0];
    const int pg1 = s_pages[(c1 >> lp) - wpage0];
    const int64_t r0 = ((int64_t)pg0 * a.page_stride + (int64_t)(c0 & page_mask) * a.slot_stride + head_off) * G_::kKvBytes;
    const int64_t r1 = ((int64_t)pg1 * a.page_stride + (int64_t)(c1 & page_mask) * a.slot_stride + head_off) * G_::kKvBytes;
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      st.k[0][p] = *reinterpret_cast<const u32x4*>(kbase + r0 + 64 * p + 16 * g);
      st.k[1][p] = *reinterpret_cast<const u32x4*>(kbase + r1 + 64 * p + 16 * g);
    }
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      st.v[0][p] = *reinterpret_cast<const u32x4*>(vbase + r0 + 64 * p + 16 * g);
      st.v[1][p] = *reinterpret_cast<const u32x4*>(vbase + r1 + 64 * p + 16 * g);
    }
  };

  // Attend step s whose K/V rows are in st. A step wholly past the window
  // (the padding step of an odd count) changes nothing and is skipped.
  auto consume = [&](int s, const StepRegs<G_::kPieces>& st) {
    const int t0 = base + s * kStepTokens;
    if (t0 > whi) return;
    // ---- logits: S[tile] rows = tokens, columns = heads
    f32x4 sc[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      f32x4 acc_s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < G_::kQkMfma; ++j) {
        v8 kop;
        if constexpr (KV8) {
          const u32x4 w = st.k[tile][j >> 1];
          kop = (j & 1) ? e4m3x8<QBF16>(w[2], w[3]) : e4m3x8<QBF16>(w[0], w[1]);
        } else {
          kop = __builtin_bit_cast(v8, st.k[tile][j]);
        }
        acc_s = O::mfma(kop, bq[j], acc_s);
      }
      sc[tile] = acc_s;
    }
    // ---- V rows to this wave's LDS copy (row = token within the step)
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      *reinterpret_cast<u32x4*>(vl + tau0 * G_::kVPitch + 64 * p + 16 * g) = st.v[0][p];
      *reinterpret_cast<u32x4*>(vl + tau1 * G_::kVPitch + 64 * p + 16 * g) = st.v[1][p];
    }
    // ---- online softmax (base 2)
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sc[tile][i] * a.logit_scale;
        if constexpr (CAP) v = a.cap * tanh_from_exp(v * a.inv_cap) * kLog2e;
        const int t = t0 + 8 * g + 4 * tile + i;
        v = (t >= wlo && t <= whi) ? v : -INFINITY;
        x[4 * tile + i] = v;
        mx = fmaxf(mx, v);
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
    u32x4 pw;
    pw[0] = O::pack(x[0], x[1]);
    pw[1] = O::pack(x[2], x[3]);
    pw[2] = O::pack(x[4], x[5]);
    pw[3] = O::pack(x[6], x[7]);
    const v8 pop = __builtin_bit_cast(v8, pw);
    // ---- O^T += V^T P^T, one MFMA per 16 hd columns
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
      c[0] *= alpha; c[1] *= alpha; c[2] *= alpha; c[3] *= alpha;
      acc[b] = O::mfma(vop, pop, c);
    }
  };

  // Steps are processed in windows whose pages fit the LDS page table.
  // Loads are issued one step ahead and unconditionally (a surplus prefetch
  // past the window re-reads its last row), which keeps the number of loads
  // in flight the same on every path, so the compiler's wait before a step
  // covers that step's loads only.
  const int win_steps = max(1, ((kPageWin - 1) << lp) >> 5);
  for (int w0 = 0; w0 < nsteps; w0 += win_steps) {
    const int w1 = min(nsteps, w0 + win_steps);
    wlo = max(tb, base + w0 * kStepTokens);
    whi = min(te, base + w1 * kStepTokens) - 1;
    wpage0 = wlo >> lp;
    const int wpages = (whi >> lp) - wpage0 + 1;
    __syncthreads();                   // previous window fully consumed
    for (int i = threadIdx.x; i < wpages; i += kWaves * 64) s_pages[i] = pidx[wpage0 + i];
    __syncthreads();
    // This wave's steps in the window, taken two at a time; an odd count
    // gets one more step past the window, which reads clamped rows and whose
    // tokens are all masked (no effect on the state). The loop body has no
    // exit in the middle, so each half waits for its own loads only.
    const int s0 = w0 + ((wave - w0) % kWaves + kWaves) % kWaves;
    const int mine = s0 < w1 ? (w1 - s0 + kWaves - 1) / kWaves : 0;
    // The scheduling barriers keep each issue ahead of the step it overlaps:
    // the loads must leave before the wait for the previous step's rows.
    if constexpr (G_::kStages == 2) {
      StepRegs<G_::kPieces> A, B;
      issue(s0, A);
      for (int k = 0; k < (mine + 1) / 2; ++k) {
        const int s = s0 + 2 * k * kWaves;
        issue(s + kWaves, B);
        __builtin_amdgcn_sched_barrier(0);
        consume(s, A);
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 2 * kWaves, A);
        __builtin_amdgcn_sched_barrier(0);
        consume(s + kWaves, B);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      for (int k = 0; k < mine; ++k) {
        StepRegs<G_::kPieces> A;
        issue(s0 + k * kWaves, A);
        consume(s0 + k * kWaves, A);
      }
    }
  }

  // ---- merge the wavefronts' states in LDS, in wavefront order
  d_run = wave_sum_over_groups(d_run);
  __syncthreads();                       // all V copies consumed
  float* sacc = reinterpret_cast<float*>(vl);   // [16 heads][HD]
  if (n < group) {
#pragma unroll
    for (int b = 0; b < G_::kPvMfma; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[n * HD + 16 * b + 4 * g + i] = acc[b][i];
    if (g == 0) {
      s_m[wave][n] = m_run;
      s_d[wave][n] = d_run;
    }
  }
  __syncthreads();
  const int total = group * HD;
  for (int e = threadIdx.x; e < total; e += kWaves * 64) {
    const int h = e / HD, c = e - h * HD;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w][h];
      const float sw = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
      num += sw * reinterpret_cast<const float*>(smem + w * G_::kWaveLds)[h * HD + c];
      den += sw * s_d[w][h];
    }
    const float ov = num / den * a.v_scale;
    const float lse2 = M + __builtin_amdgcn_logf(den);
    const int qh = qh0 + h;
    if (it.partial < 0) {
      store_out(a.o, ((size_t)it.request * a.num_qo_heads + qh) * HD + c, ov, a.o_bf16);
      if (a.lse != nullptr && c == 0) a.lse[(size_t)it.request * a.num_qo_heads + qh] = lse2 * kLn2;
    } else {
      a.ws_o[((size_t)it.partial * a.num_qo_heads + qh) * HD + c] = ov;
      if (c == 0) a.ws_lse[(size_t)it.partial * a.num_qo_heads + qh] = lse2;
    }
  }
  if (threadIdx.x == 0) s_item = next;
  __syncthreads();                       // LDS free for the next item
  item = __builtin_amdgcn_readfirstlane(s_item);
  }
  // The last workgroup out resets the counters for the next launch: every
  // other workgroup has already taken its final item number by then.
  if (threadIdx.x == 0 && atomicAdd(&a.counters[1], 1) == (int)gridDim.x - 1) {
    atomicExch(&a.counters[0], 0);
    atomicExch(&a.counters[1], 0);
  }
}

// One wavefront per output row: fold the row's states in ascending order.
// Plan mode: row r is (merge entry r / num_qo_heads, head r % num_qo_heads),
// states are the entry's workspace slots. Flat mode: row r has num_states
// states at v[r][k][:], s[r][k].
//
// Lanes are split into `cl` chunk lanes x (hd/4) column lanes (float4 each);
// chunk lane kk folds states kk, kk+cl, ... in ascending order, then the cl
// partial sums are added in lane order. The sum order depends only on the
// number of states, so the result is deterministic and batch invariant.
__global__ __launch_bounds__(kMergeRowsPerBlock * 64) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.num_rows) return;
  const int hd = a.head_dim;
  const float* vs;
  const float* ss;
  int64_t v_stride, s_stride;   // between consecutive states
  int nst;
  size_t out_row;
  if (a.rows != nullptr) {
    const MergeRow mr = a.rows[row / a.num_qo_heads];
    const int qh = row % a.num_qo_heads;
    nst = mr.num_chunks;
    vs = a.v + ((size_t)mr.partial_base * a.num_qo_heads + qh) * hd;
    ss = a.s + (size_t)mr.partial_base * a.num_qo_heads + qh;
    v_stride = (int64_t)a.num_qo_heads * hd;
    s_stride = a.num_qo_heads;
    out_row = (size_t)mr.request * a.num_qo_heads + qh;
  } else {
    nst = a.num_states;
    vs = a.v + (size_t)row * nst * hd;
    ss = a.s + (size_t)row * nst;
    v_stride = hd;
    s_stride = 1;
    out_row = row;
  }
  const float to2 = a.s_base2 ? 1.0f : kLog2e;
  float M = -INFINITY;
  for (int k = lane; k < nst; k += 64) M = fmaxf(M, ss[k * s_stride] * to2);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  auto weight = [&](int k) {
    const float sk = ss[k * s_stride] * to2;
    return sk == -INFINITY ? 0.0f : fast_exp2(sk - M);
  };
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int k = lane; k < nst; k += 64) den += weight(k);
    for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off);
  }
  const int ngc = hd >> 2;
  const bool vec = (hd & 3) == 0 && hd <= 256 && (ngc & (ngc - 1)) == 0 &&
                   (reinterpret_cast<uintptr_t>(vs) & 15) == 0 && (v_stride & 3) == 0;
  if (vec) {
    const int ng = hd >> 2;                  // float4 columns
    const int cl = 64 / ng;                  // chunk lanes (>= 1)
    const int cg = lane % ng, kk = lane / ng;
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY && kk < cl) {
#pragma unroll 8
      for (int k = kk; k < nst; k += cl) {
        const float wk = weight(k);
        const f32x4 x = *reinterpret_cast<const f32x4*>(vs + k * v_stride + 4 * cg);
        acc4 += wk * x;
      }
    }
    // add the chunk lanes' partial sums in lane order
    for (int off = ng; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc4[e] += __shfl_xor(acc4[e], off);
    }
    if (kk == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ov = M == -INFINITY ? 0.0f : acc4[e] / den;
        const size_t idx = out_row * hd + 4 * cg + e;
        if (a.out_dtype == PKD_F32)
          reinterpret_cast<float*>(a.v_out)[idx] = ov;
        else
          store_out(a.v_out, idx, ov, a.out_dtype == PKD_BF16);
      }
    }
  } else {
    for (int c = lane; c < hd; c += 64) {
      float num = 0.0f;
      if (M != -INFINITY)
        for (int k = 0; k < nst; ++k) num += weight(k) * vs[k * v_stride + c];
      const float ov = M == -INFINITY ? 0.0f : num / den;
      const size_t idx = out_row * hd + c;
      if (a.out_dtype == PKD_F32)
        reinterpret_cast<float*>(a.v_out)[idx] = ov;
      else
        store_out(a.v_out, idx, ov, a.out_dtype == PKD_BF16);
    }
  }
  if (a.s_out != nullptr && lane == 0)
    a.s_out[out_row] = M == -INFINITY ? -INFINITY : (M + __builtin_amdgcn_logf(den)) * kLn2;
}

// The kernel instance for (head_dim, q type, KV type, soft cap).
using DecodeFn = void (*)(DecodeArgs);

template <bool QBF16, bool KV8, bool CAP>
DecodeFn pick_hd(int hd) {
  switch (hd) {
    case 64: return decode_kernel<64, QBF16, KV8, CAP>;
    case 128: return decode_kernel<128, QBF16, KV8, CAP>;
    default: return decode_kernel<256, QBF16, KV8, CAP>;
  }
}

DecodeFn pick_kernel(const pkd_plan_params& p) {
  const bool cap = p.logits_soft_cap > 0.0f;
  const bool qbf = p.q_dtype == PKD_BF16;
  const bool kv8 = p.kv_dtype == PKD_E4M3;
  if (qbf) {
    if (kv8) return cap ? pick_hd<true, true, true>(p.head_dim) : pick_hd<true, true, false>(p.head_dim);
    return cap ? pick_hd<true, false, true>(p.head_dim) : pick_hd<true, false, false>(p.head_dim);
  }
  if (kv8) return cap ? pick_hd<false, true, true>(p.head_dim) : pick_hd<false, true, false>(p.head_dim);
  return cap ? pick_hd<false, false, true>(p.head_dim) : pick_hd<false, false, false>(p.head_dim);
}

}  // namespace

int launch_decode(const pkd_plan_params& p, const DecodeArgs& a, int32_t num_workgroups,
                  void* stream) {
  if (num_workgroups <= 0) return hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(pick_kernel(p), dim3(num_workgroups), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

int32_t decode_wgs_per_cu(const pkd_plan_params& p) {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &blocks, reinterpret_cast<const void*>(pick_kernel(p)), kWaves * 64, 0) != hipSuccess)
    return 0;
  return blocks;
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.num_rows <= 0) return hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((a.num_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeRowsPerBlock * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkd

