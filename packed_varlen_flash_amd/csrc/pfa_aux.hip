// pfa_aux.hip -- HBM-bound companions of the attention kernels for gfx950, behind the C
// ABI: the (O, LSE) merge of two results over disjoint key sets (pfa_attn_merge) and the
// e4m3 quantiser of V for the FP8 P.V variant (pfa_quantize_v_fp8).
#include "pfa_common.h"

namespace {

// ---------------------------------------------------------------------------------
// (O, LSE) merge of two results for the same queries over disjoint key sets A and B.
// With Z_X = exp(LSE_X) the partition sum over X, the union has Z_A + Z_B and its output
// is the Z-weighted mean of O_A and O_B: the identity behind the blocked update of the
// GigaPath-Flash page (section 3.2), applied to two finished blocks.  One thread per
// 16-byte chunk (8 values) of one (token, head) row; a row's chunks are consecutive
// lanes of one wave, so every lane has read its row's LSE values before any lane
// stores, and the result may overwrite either input in place.  HBM-bound.
// ---------------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

struct MergeParams {
  const __bf16* o_a;
  const __bf16* o_b;
  const float* lse_a;
  const float* lse_b;
  __bf16* out;
  float* lse;
  int64_t total;
  int heads;
  int cpr;   // 16-byte chunks per row (head_dim / 8)
};

__global__ void __launch_bounds__(kMergeThreads) pfa_merge_kernel(MergeParams m) {
  const int64_t idx = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t row = idx / m.cpr;             // (token, head) row, head fastest
  const int ch = (int)(idx - row * m.cpr);
  if (row >= m.total * m.heads) return;
  const int64_t t = row / m.heads;
  const int h = (int)(row - t * m.heads);
  const float la = m.lse_a[(int64_t)h * m.total + t];
  const float lb = m.lse_b[(int64_t)h * m.total + t];
  const float mx = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (mx != -INFINITY) {                        // at least one side has keys
    wa = __builtin_amdgcn_exp2f((la - mx) * kLog2e);
    wb = __builtin_amdgcn_exp2f((lb - mx) * kLog2e);
    const float z = wa + wb;
    l = mx + __builtin_amdgcn_logf(z) * kLn2;
    const float inv = 1.0f / z;
    wa *= inv;
    wb *= inv;
  }
  const int64_t off = row * (int64_t)(m.cpr * 8) + ch * 8;
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(m.o_a + off);
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(m.o_b + off);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)(wa * (float)a[e] + wb * (float)b[e]);
  *reinterpret_cast<bf16x8*>(m.out + off) = r;
  if (m.lse != nullptr && ch == 0) m.lse[(int64_t)h * m.total + t] = l;
}

// ---------------------------------------------------------------------------------
// V quantiser of the FP8 P.V variant.  The FPS Attention slides (tool.lu deck on
// accelerating multimodal generation, slides 35-38) quantise V per channel.  Here every
// (segment, head, channel) gets the power-of-two scale 2^e, e the smallest integer with
// max|V| 2^-e <= 448 (not below -126), and the codes are V 2^-e rounded to e4m3 (nearest
// even).  Scaling by a power of two is exact, so the codes do not depend on the precision
// of the arithmetic, and a segment's scales depend on its own tokens only.  Four launches:
// zero the per-(segment, head, channel) maxima (held in v_scale as float bits), maxima
// (order-independent atomic max of non-negative floats, so the result is deterministic),
// codes, and finally the scales over the maxima.  All HBM-bound.
// ---------------------------------------------------------------------------------
constexpr int kQuantThreads = 256;
constexpr int kQuantUnroll = 8;    // loads in flight per thread; tokens per thread in the codes pass
constexpr int kAmaxBlock = 512;    // tokens per work unit of the maxima pass
constexpr int kAmaxWaves = 8;      // waves per maxima workgroup
constexpr int kAmaxThreads = 64 * kAmaxWaves;
static_assert(kAmaxThreads == 64 * 8, "the LDS reduction gives each thread one (chunk, element) pair");

struct QuantParams {
  const __bf16* v;
  const int32_t* cu;
  uint8_t* v8;
  float* v_scale;   // [num_seqs, heads, d]: maxima (float bits) during the call, then scales
  int num_seqs;
  int heads;
  int d;
};

// segment of row t: the last s with cu[s] <= t, skipping empty segments (cu[s+1] > t)
__device__ __forceinline__ int segment_of(const int32_t* cu, int n, int64_t t) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int v8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float m = __builtin_frexpf(amax, &E);   // amax = m 2^E, 0.5 <= m < 1
  const int e = m <= 0.875f ? E - 9 : E - 8;    // 448 = 0.875 * 2^9
  return e < -126 ? -126 : e;
}

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_zero_kernel(QuantParams q) {
  const int64_t n = (int64_t)q.num_seqs * q.heads * q.d;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kQuantThreads)
    reinterpret_cast<uint32_t*>(q.v_scale)[i] = 0u;
}

// Maxima over one work unit: a kAmaxBlock-token block of the packed rows times a group of
// 64 chunk columns (16 bytes each).  Lane l owns chunk column 64 g + l; wave w reads the
// block's tokens w, w + kAmaxWaves, ..., so each load instruction covers 1 KB of one row.
// Per segment run of the block the waves' maxima meet in LDS, and one atomic per
// (segment, channel) leaves the workgroup: the same-address atomics of a long segment are
// what bound this pass when every thread issued its own.
__global__ void __launch_bounds__(kAmaxThreads) pfa_v8_amax_kernel(QuantParams q) {
  __shared__ float part[kAmaxWaves][8][64];
  const int64_t T = q.cu[q.num_seqs];
  const int cpt = q.heads * q.d / 8;                      // 16-byte chunks per token
  const int ncg = (cpt + 63) / 64;
  const int64_t units = (T + kAmaxBlock - 1) / kAmaxBlock * ncg;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {   // uniform over the workgroup
    const int64_t t0 = u / ncg * kAmaxBlock;
    const int jg = (int)(u % ncg) * 64;
    const int j = jg + lane;
    const int64_t t1 = t0 + kAmaxBlock < T ? t0 + kAmaxBlock : T;
    const __bf16* src = q.v + 8 * j;
    int seg = segment_of(q.cu, q.num_seqs, t0);
    int64_t rs = t0;
    while (rs < t1) {                                       // one segment run per pass
      const int64_t seg_end = q.cu[seg + 1];
      const int64_t re = seg_end < t1 ? seg_end : t1;
      float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (j < cpt) {
        // this wave's first token at or after the run start
        int64_t t = t0 + w;
        if (rs - t0 > w) t += (rs - t0 - w + kAmaxWaves - 1) / kAmaxWaves * kAmaxWaves;
        for (; t + (int64_t)(kQuantUnroll - 1) * kAmaxWaves < re; t += (int64_t)kQuantUnroll * kAmaxWaves) {
          bf16x8 x[kQuantUnroll];
#pragma unroll
          for (int i = 0; i < kQuantUnroll; ++i)
            x[i] = *reinterpret_cast<const bf16x8*>(src + (t + (int64_t)i * kAmaxWaves) * cpt * 8);
#pragma unroll
          for (int i = 0; i < kQuantUnroll; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf((float)x[i][e]));
        }
        for (; t < re; t += kAmaxWaves) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(src + t * cpt * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf((float)x[e]));
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[w][e][lane] = mx[e];
      __syncthreads();
      {
        const int c = threadIdx.x & 63, e = threadIdx.x >> 6;   // one (chunk, element) per thread
        float m = 0.f;
#pragma unroll
        for (int ww = 0; ww < kAmaxWaves; ++ww) m = fmaxf(m, part[ww][e][c]);
        if (jg + c < cpt && m > 0.f)
          atomicMax(reinterpret_cast<uint32_t*>(q.v_scale) + ((int64_t)seg * q.heads) * q.d + 8 * (jg + c) + e,
                    __float_as_uint(m));
      }
      __syncthreads();
      rs = re;
      while (rs < t1 && q.cu[seg + 1] <= rs) ++seg;         // next non-empty segment
    }
  }
}

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_codes_kernel(QuantParams q) {
  const int64_t T = q.cu[q.num_seqs];
  const int cpt = q.heads * q.d / 8;
  const int64_t items = (T > 0 ? (T + kQuantUnroll - 1) / kQuantUnroll : 0) * cpt;
  for (int64_t it = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kQuantThreads) {
    const int64_t t0 = it / cpt * kQuantUnroll;        // kQuantUnroll tokens of one chunk column
    const int j = (int)(it % cpt);
    const int n = T - t0 < kQuantUnroll ? (int)(T - t0) : kQuantUnroll;
    bf16x8 x[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u)
      if (u < n) x[u] = *reinterpret_cast<const bf16x8*>(q.v + (t0 + u) * cpt * 8 + 8 * j);
    int seg = segment_of(q.cu, q.num_seqs, t0);
    int64_t seg_end = q.cu[seg + 1];
    int ex[8];
    auto exponents = [&]() {
      const uint32_t* am = reinterpret_cast<const uint32_t*>(q.v_scale) + ((int64_t)seg * q.heads) * q.d + 8 * j;
#pragma unroll
      for (int e = 0; e < 8; ++e) ex[e] = v8_exponent(__uint_as_float(am[e]));
    };
    exponents();
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      if (u >= n) break;
      const int64_t t = t0 + u;
      if (t >= seg_end) {                          // the run crosses into the next segment(s)
        while (q.cu[seg + 1] <= t) ++seg;
        seg_end = q.cu[seg + 1];
        exponents();
      }
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf((float)x[u][e], -ex[e]);
      int lo = 0, hi = 0;
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], lo, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], hi, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      *reinterpret_cast<u32x2*>(q.v8 + t * cpt * 8 + 8 * j) = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
  }
}

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_scale_kernel(QuantParams q) {
  const int64_t n = (int64_t)q.num_seqs * q.heads * q.d;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kQuantThreads)
    q.v_scale[i] = __builtin_ldexpf(1.0f, v8_exponent(q.v_scale[i]));
}

}  // namespace

extern "C" {

PFA_API int pfa_quantize_v_fp8(const void* v, const int32_t* cu_seqlens, int num_seqs, int heads,
                               int head_dim, void* v8, float* v_scale, hipStream_t stream) {
  if (v == nullptr || cu_seqlens == nullptr || v8 == nullptr || v_scale == nullptr) return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  const void* ins[2] = {v, cu_seqlens};
  for (const void* in : ins)
    if (in == v8 || in == static_cast<const void*>(v_scale)) return PFA_ERR_ALIAS;
  if (v8 == static_cast<const void*>(v_scale)) return PFA_ERR_ALIAS;
  if (misaligned16(v) || (reinterpret_cast<uintptr_t>(v8) & 7) != 0 || misaligned4(v_scale) ||
      misaligned4(cu_seqlens))
    return PFA_ERR_ALIGN;
  if ((int64_t)heads * head_dim > kMaxRowElems || (int64_t)num_seqs * heads * head_dim > INT32_MAX)
    return PFA_ERR_SIZE;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != PFA_OK) return rc;
  QuantParams qp;
  qp.v = static_cast<const __bf16*>(v);
  qp.cu = cu_seqlens;
  qp.v8 = static_cast<uint8_t*>(v8);
  qp.v_scale = v_scale;
  qp.num_seqs = num_seqs;
  qp.heads = heads;
  qp.d = head_dim;
  void* args[] = {&qp};
  const void* fns[4] = {reinterpret_cast<const void*>(&pfa_v8_zero_kernel),
                        reinterpret_cast<const void*>(&pfa_v8_amax_kernel),
                        reinterpret_cast<const void*>(&pfa_v8_codes_kernel),
                        reinterpret_cast<const void*>(&pfa_v8_scale_kernel)};
  const unsigned grids[4] = {(unsigned)cus, (unsigned)cus * 4, (unsigned)cus * 8, (unsigned)cus};
  const unsigned threads[4] = {kQuantThreads, kAmaxThreads, kQuantThreads, kQuantThreads};
  for (int i = 0; i < 4; ++i)
    if (hipLaunchKernel(fns[i], dim3(grids[i]), dim3(threads[i]), args, 0, stream) != hipSuccess)
      return PFA_ERR_LAUNCH;
  return PFA_OK;
}

PFA_API int pfa_attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                           int64_t total, int heads, int head_dim, void* out, float* lse,
                           hipStream_t stream) {
  if (o_a == nullptr || lse_a == nullptr || o_b == nullptr || lse_b == nullptr || out == nullptr)
    return PFA_ERR_NULL;
  if (total < 0) return PFA_ERR_SIZE;
  if (heads < 1) return PFA_ERR_HEADS;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  const void* ins[4] = {o_a, lse_a, o_b, lse_b};
  for (const void* in : ins)   // in place on one side is allowed; crossing o and lse is not
    if ((lse != nullptr && static_cast<const void*>(lse) == out) ||
        (in == static_cast<const void*>(out) && (in == lse_a || in == lse_b)) ||
        (lse != nullptr && in == static_cast<const void*>(lse) && (in == o_a || in == o_b)))
      return PFA_ERR_ALIAS;
  // O rows move in 16-byte chunks
  if (misaligned16(o_a) || misaligned16(o_b) || misaligned16(out) || misaligned4(lse_a) ||
      misaligned4(lse_b) || misaligned4(lse))
    return PFA_ERR_ALIGN;
  if (total == 0) return PFA_OK;
  const int64_t chunks = total * heads * (head_dim / 8);
  const int64_t blocks = (chunks + kMergeThreads - 1) / kMergeThreads;
  if (total > INT32_MAX || blocks > INT32_MAX) return PFA_ERR_SIZE;
  MergeParams mp;
  mp.o_a = static_cast<const __bf16*>(o_a);
  mp.o_b = static_cast<const __bf16*>(o_b);
  mp.lse_a = lse_a;
  mp.lse_b = lse_b;
  mp.out = static_cast<__bf16*>(out);
  mp.lse = lse;
  mp.total = total;
  mp.heads = heads;
  mp.cpr = head_dim / 8;
  void* args[] = {&mp};
  const hipError_t err = hipLaunchKernel(reinterpret_cast<const void*>(&pfa_merge_kernel),
                                         dim3((unsigned)blocks), dim3(kMergeThreads), args, 0, stream);
  return err == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

}  // extern "C"
