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
  // LDS row pitch of the V copy; the pad staggers rows across banks.
  static constexpr int kVPitch = kRowBytes + (KV8 ? 16 : 32);
  static constexpr int kVBytes = kStepTokens * kVPitch;
  static constexpr int kMergeBytes = kMaxGroup * HD * 4;
  static constexpr int kWaveLds = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
};

// Byte offset, inside a K/V row, of the 8 operand elements that lane group g
// feeds to QK MFMA j. The hd order inside the dot product is free as long as
// q uses the same one.
template <bool KV8>
__device__ __forceinline__ int qk_hd(int j, int g) {
  return KV8 ? 64 * (j >> 1) + 16 * g + 8 * (j & 1) : 32 * j + 8 * g;
}

template <int HD, bool QBF16, bool KV8, bool CAP>
__global__ __launch_bounds__(kWaves * 64) void decode_kernel(DecodeArgs a) {
  using G_ = Geo<HD, KV8>;
  using O = Op<QBF16>;
  using v8 = typename O::v8;
  __shared__ __attribute__((aligned(16))) char smem[kWaves * G_::kWaveLds];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_d[kWaves][kMaxGroup];

  const pkd_work_item it = a.items[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;        // MFMA row (tile token) / column (q head)
  const int g = lane >> 4;        // lane group
  const int group = a.group;
  const int tb = it.token_begin, te = it.token_end;
  const int qh0 = it.kv_head * group;

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
  const int page_mask = (1 << a.log2_page) - 1;
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

  auto clampt = [&](int t) { return min(max(t, tb), te - 1); };
  int step = wave;
  int pg0 = 0, pg1 = 0;
  if (step < nsteps) {
    const int t0 = base + step * kStepTokens;
    pg0 = pidx[clampt(t0 + tau0) >> a.log2_page];
    pg1 = pidx[clampt(t0 + tau1) >> a.log2_page];
  }
  for (; step < nsteps; step += kWaves) {
    const int t0 = base + step * kStepTokens;
    const int c0 = clampt(t0 + tau0), c1 = clampt(t0 + tau1);
    const int64_t r0 = ((int64_t)pg0 * a.page_stride + (int64_t)(c0 & page_mask) * a.slot_stride + head_off) * G_::kKvBytes;
    const int64_t r1 = ((int64_t)pg1 * a.page_stride + (int64_t)(c1 & page_mask) * a.slot_stride + head_off) * G_::kKvBytes;
    // prefetch the page ids of this wave's next step
    if (step + kWaves < nsteps) {
      const int tn = t0 + kWaves * kStepTokens;
      pg0 = pidx[clampt(tn + tau0) >> a.log2_page];
      pg1 = pidx[clampt(tn + tau1) >> a.log2_page];
    }
    u32x4 kr[2][G_::kPieces], vr[2][G_::kPieces];
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      kr[0][p] = *reinterpret_cast<const u32x4*>(kbase + r0 + 64 * p + 16 * g);
      kr[1][p] = *reinterpret_cast<const u32x4*>(kbase + r1 + 64 * p + 16 * g);
    }
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      vr[0][p] = *reinterpret_cast<const u32x4*>(vbase + r0 + 64 * p + 16 * g);
      vr[1][p] = *reinterpret_cast<const u32x4*>(vbase + r1 + 64 * p + 16 * g);
    }

    // ---- logits: S[tile] rows = tokens, columns = heads
    f32x4 sc[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < G_::kQkMfma; ++j) {
        v8 kop;
        if constexpr (KV8) {
          const u32x4 w = kr[tile][j >> 1];
          kop = (j & 1) ? e4m3x8<QBF16>(w[2], w[3]) : e4m3x8<QBF16>(w[0], w[1]);
        } else {
          kop = __builtin_bit_cast(v8, kr[tile][j]);
        }
        s = O::mfma(kop, bq[j], s);
      }
      sc[tile] = s;
    }

    // ---- V rows to this wave's LDS copy (row = token within the step)
#pragma unroll
    for (int p = 0; p < G_::kPieces; ++p) {
      *reinterpret_cast<u32x4*>(vl + tau0 * G_::kVPitch + 64 * p + 16 * g) = vr[0][p];
      *reinterpret_cast<u32x4*>(vl + tau1 * G_::kVPitch + 64 * p + 16 * g) = vr[1][p];
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
        v = (t >= tb && t < te) ? v : -INFINITY;
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
}

// One wavefront per output row: fold the row's states in ascending order.
// Plan mode: row r is (merge entry r / num_qo_heads, head r % num_qo_heads),
// states are the entry's workspace slots. Flat mode: row r has num_states
// states at v[r][k][:], s[r][k].
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
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int k = 0; k < nst; ++k) {
      const float sk = ss[k * s_stride] * to2;
      den += sk == -INFINITY ? 0.0f : fast_exp2(sk - M);
    }
  }
  for (int c = lane; c < hd; c += 64) {
    float num = 0.0f;
    if (M != -INFINITY) {
      for (int k = 0; k < nst; ++k) {
        const float sk = ss[k * s_stride] * to2;
        const float w = sk == -INFINITY ? 0.0f : fast_exp2(sk - M);
        num += w * vs[k * v_stride + c];
      }
    }
    const float ov = M == -INFINITY ? 0.0f : num / den;
    const size_t idx = out_row * hd + c;
    if (a.out_dtype == PKD_F32)
      reinterpret_cast<float*>(a.v_out)[idx] = ov;
    else
      store_out(a.v_out, idx, ov, a.out_dtype == PKD_BF16);
  }
  if (a.s_out != nullptr && lane == 0)
    a.s_out[out_row] = M == -INFINITY ? -INFINITY : (M + __builtin_amdgcn_logf(den)) * kLn2;
}

template <int HD, bool QBF16, bool KV8>
hipError_t launch_hd(bool cap, const DecodeArgs& a, int32_t items, hipStream_t s) {
  dim3 grid(items), block(kWaves * 64);
  if (cap)
    hipLaunchKernelGGL((decode_kernel<HD, QBF16, KV8, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<HD, QBF16, KV8, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool QBF16, bool KV8>
hipError_t launch_types(int hd, bool cap, const DecodeArgs& a, int32_t items, hipStream_t s) {
  switch (hd) {
    case 64: return launch_hd<64, QBF16, KV8>(cap, a, items, s);
    case 128: return launch_hd<128, QBF16, KV8>(cap, a, items, s);
    default: return launch_hd<256, QBF16, KV8>(cap, a, items, s);
  }
}

}  // namespace

int launch_decode(const pkd_plan_params& p, const DecodeArgs& a, int32_t items,
                  void* stream) {
  if (items <= 0) return hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool cap = p.logits_soft_cap > 0.0f;
  const bool qbf = p.q_dtype == PKD_BF16;
  const bool kv8 = p.kv_dtype == PKD_E4M3;
  if (qbf)
    return kv8 ? launch_types<true, true>(p.head_dim, cap, a, items, s)
               : launch_types<true, false>(p.head_dim, cap, a, items, s);
  return kv8 ? launch_types<false, true>(p.head_dim, cap, a, items, s)
             : launch_types<false, false>(p.head_dim, cap, a, items, s);
}

int launch_merge(const MergeArgs& a, void* stream) {
  if (a.num_rows <= 0) return hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((a.num_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock);
  hipLaunchKernelGGL(merge_kernel, grid, dim3(kMergeRowsPerBlock * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkd
