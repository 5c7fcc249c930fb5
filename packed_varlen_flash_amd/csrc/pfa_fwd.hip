// pfa_fwd.hip -- packed varlen attention forward for gfx950 (MI355X), behind a C ABI.
//
// The operation (Mage-Flow page, section on native-resolution sequence packing): image
// tokens are packed into one [T, heads, head_dim] sequence, cu_seqlens marks each
// image's rows, and attention is non-causal and block-diagonal, so a token only sees
// the keys of its own image.  The kernel is the blocked online-softmax scheme of the
// GigaPath-Flash page (section 3.2; its section 4.2 reference loop): split Q, K and V
// into blocks, compute the local scores of a Q block against one K block, update the
// running row maximum and normaliser, rescale and accumulate the output, and write only
// the final output (and here the log-sum-exp) back to HBM.
//
// gfx950 mapping (one workgroup = 4 wave64s, one wave per SIMD):
//   * work unit = (segment, head, BM-row query tile); a tile never spans two segments.
//     Tiles are listed longest segment first and handed out round-robin by a persistent
//     grid; each XCD receives contiguous runs of the list so the query tiles that share
//     one (segment, head) K/V stream sit behind the same L2.
//   * each wave owns QB blocks of 32 queries and keeps their Q fragments in VGPRs.
//   * K and V tiles of 64 keys are double-buffered in LDS, loaded with 16-byte global
//     loads; rows past the segment end are zero-filled, never read from a neighbour.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the accumulator gives every lane one
//     query column, so the row maximum and row sum are in-lane reductions plus a single
//     v_permlane32_swap between the two half-waves.
//   * P^T (bf16) is consumed straight from the accumulator registers as the B operand of
//     O^T += V^T P^T; the V^T operand comes from row-major V in LDS through
//     ds_read_b64_tr_b16 transposed loads.
//   * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA per score.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "pfa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kBN = 64;          // keys per LDS stage
constexpr int kSortMax = 1024;   // segment tables up to this size are sorted on device
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* cu;
  __bf16* out;
  float* lse;
  int num_seqs;
  int heads;
  int qt_max;      // ceil(max_seqlen / BM): slots per (segment, head) in unsorted mode
  float c;         // scale * log2(e)
};

template <int D, int QB>
struct Tile {
  static constexpr int BM = kWaves * QB * 32;       // query rows per workgroup tile
  static constexpr int KSTR = D + 8;                // K row stride in LDS (elements)
  static constexpr int VSTR = D + 16;               // V row stride in LDS (elements)
  static constexpr int KTILE = kBN * KSTR;
  static constexpr int VTILE = kBN * VSTR;
  static constexpr int CHUNKS_PER_ROW = D / 8;      // 16-byte chunks per row
  static constexpr int CPT = kBN * CHUNKS_PER_ROW / kThreads;  // chunks per thread per tile
  static constexpr int DT = D / 32;                 // 32-row output tiles along head_dim
  static constexpr int KSTEP = D / 16;              // 16-deep steps of the Q.K contraction
  static constexpr int SCHED_INTS = 2 * kSortMax + 8;
  static constexpr size_t LDS_BYTES =
      sizeof(__bf16) * (size_t)(2 * KTILE + 2 * VTILE) + sizeof(int) * SCHED_INTS;
  static_assert(CPT * kThreads == kBN * CHUNKS_PER_ROW, "tile must split evenly");
  static_assert(sizeof(int) * kSortMax <= sizeof(__bf16) * 2 * KTILE, "len scratch fits");
};

__device__ __forceinline__ float partner_max(float x) {
  // v_permlane32_swap pairs lane l with lane l^32: max of the pair on every lane.
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float partner_sum(float x) {
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// ---------------------------------------------------------------------------------
// Device-side scheduler: decode cu_seqlens into a longest-first list of work items.
// ---------------------------------------------------------------------------------
// Sorted mode (num_seqs <= kSortMax): s_order[r] = segment of rank r (length
// descending, ties by index), s_prefix[r] = first item of rank r; items of one segment
// are ordered head-major, query-tile-minor.  Returns the item count.
template <int BM>
__device__ int build_schedule(const Params& p, int* s_len, int* s_order, int* s_prefix) {
  const int n = p.num_seqs;
  const int tid = threadIdx.x;
  for (int s = tid; s < n; s += kThreads) {
    int L = p.cu[s + 1] - p.cu[s];
    s_len[s] = L > 0 ? L : 0;
  }
  __syncthreads();
  for (int s = tid; s < n; s += kThreads) {
    const int L = s_len[s];
    int rank = 0;
    for (int t = 0; t < n; ++t) {
      const int Lt = s_len[t];
      rank += (Lt > L) || (Lt == L && t < s);
    }
    s_order[rank] = s;
  }
  __syncthreads();
  // items per rank, then an inclusive Hillis-Steele scan in place (n <= kSortMax)
  for (int r = tid; r < n; r += kThreads) {
    const int L = s_len[s_order[r]];
    s_prefix[r + 1] = p.heads * ((L + BM - 1) / BM);
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
  for (int off = 1; off < n; off <<= 1) {
    int add[kSortMax / kThreads];
#pragma unroll
    for (int j = 0; j < kSortMax / kThreads; ++j) {
      const int r = tid + j * kThreads;
      add[j] = (r < n && r >= off) ? s_prefix[r + 1 - off] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortMax / kThreads; ++j) {
      const int r = tid + j * kThreads;
      if (r < n) s_prefix[r + 1] += add[j];
    }
    __syncthreads();
  }
  return s_prefix[n];
}

// ---------------------------------------------------------------------------------
// One query tile of one (segment, head).
// ---------------------------------------------------------------------------------
template <int D, int QB>
__device__ __forceinline__ void process_tile(const Params& p, __bf16* ks, __bf16* vs, int seg_a,
                                             int L, int h, int qt, int T) {
  using C = Tile<D, QB>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n32 = lane & 31;         // query column (S^T) / d row of V^T within a 32-tile
  const int g = lane >> 5;           // half-wave
  const int i16 = lane & 15;
  const int hh = (lane >> 4) & 1;
  const int64_t rs = (int64_t)p.heads * D;  // elements between consecutive tokens
  const int64_t head_off = (int64_t)h * D;
  const __bf16* qbase = p.q + (int64_t)seg_a * rs + head_off;
  const __bf16* kbase = p.k + (int64_t)seg_a * rs + head_off;
  const __bf16* vbase = p.v + (int64_t)seg_a * rs + head_off;
  const int q0 = qt * C::BM + wave * (QB * 32);
  const int nkb = (L + kBN - 1) / kBN;

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds q[row n32][16t + 8g .. +7]
  bf16x8 qr[QB][C::KSTEP];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int row = q0 + b * 32 + n32;
#pragma unroll
    for (int t = 0; t < C::KSTEP; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < L) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)row * rs + 16 * t + 8 * g);
      qr[b][t] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- K/V staging through registers
  u32x4 kst[C::CPT], vst[C::CPT];
  auto gload = [&](int kb) {
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int id = tid + r * kThreads;
      const int row = id / C::CHUNKS_PER_ROW;
      const int col = id % C::CHUNKS_PER_ROW;
      const int key = kb + row;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (key < L) {
        xk = *reinterpret_cast<const u32x4*>(kbase + (int64_t)key * rs + col * 8);
        xv = *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * rs + col * 8);
      }
      kst[r] = xk;
      vst[r] = xv;
    }
  };
  auto lstore = [&](int stage) {
#pragma unroll
    for (int r = 0; r < C::CPT; ++r) {
      const int id = tid + r * kThreads;
      const int row = id / C::CHUNKS_PER_ROW;
      const int col = id % C::CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(ks + stage * C::KTILE + row * C::KSTR + col * 8) = kst[r];
      *reinterpret_cast<u32x4*>(vs + stage * C::VTILE + row * C::VSTR + col * 8) = vst[r];
    }
  };

  f32x16 o[QB][C::DT];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m_run[b] = -INFINITY;
    l_run[b] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[b][dt][i] = 0.f;
  }

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < nkb; ++j) {
    const int cur = j & 1;
    const int kb = j * kBN;
    const bool more = j + 1 < nkb;
    if (more) gload(kb + kBN);

    const __bf16* kst_l = ks + cur * C::KTILE;
    const __bf16* vst_l = vs + cur * C::VTILE;

    // ---- S^T[key][query] = K Q^T for two 32-key sub-blocks
    f32x16 sacc[QB][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b][sb][i] = 0.f;
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(kst_l + (sb * 32 + n32) * C::KSTR + 16 * t + 8 * g);
#pragma unroll
        for (int b = 0; b < QB; ++b)
          sacc[b][sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[b][t], sacc[b][sb], 0, 0, 0);
      }
    }

    // ---- keys past the segment end never contribute
    if (kb + kBN > L) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + sb * 32 + (i >> 2) * 8 + 4 * g + (i & 3);
          if (key >= L) {
#pragma unroll
            for (int b = 0; b < QB; ++b) sacc[b][sb][i] = -INFINITY;
          }
        }
    }

    // ---- online softmax (base 2): running max, rescale, exponentiate, row sum
    bf16x8 pb[QB][2][2];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float mx = sacc[b][0][0];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[b][sb][i]);
      mx = partner_max(mx);
      const float m_new = fmaxf(m_run[b], mx * p.c);
      const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_new);
      m_run[b] = m_new;
      float rsum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[b][sb][i], p.c, -m_new));
          rsum += e;
          pb[b][sb][i >> 3][i & 7] = (__bf16)e;
        }
      l_run[b] = l_run[b] * alpha + rsum;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[b][dt][i] *= alpha;
    }

    // ---- O^T[d][query] += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int ch = 2 * sb + cc;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const __bf16* vp = vst_l + (16 * ch + 4 * g + (i16 >> 2)) * C::VSTR + 32 * dt + 16 * hh + 4 * (i16 & 3);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * C::VSTR));
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int b = 0; b < QB; ++b)
            o[b][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[b][sb][cc], o[b][dt], 0, 0, 0);
        }
      }

    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l in bf16 (round to nearest even), LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lt = partner_sum(l_run[b]);
    const int row = q0 + b * 32 + n32;
    if (row < L) {
      const float inv = 1.0f / lt;
      __bf16* orow = p.out + (int64_t)(seg_a + row) * rs + head_off;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[b][dt][4 * ii + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * ii + 4 * g) = w;
        }
      if (p.lse != nullptr && g == 0)
        p.lse[(int64_t)h * T + seg_a + row] = (m_run[b] + __builtin_amdgcn_logf(lt)) * kLn2;
    }
  }
}

template <int D, int QB>
__global__ void __launch_bounds__(kThreads) pfa_fwd_kernel(Params p) {
  using C = Tile<D, QB>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16* ks = reinterpret_cast<__bf16*>(smem);
  __bf16* vs = ks + 2 * C::KTILE;
  int* s_order = reinterpret_cast<int*>(vs + 2 * C::VTILE);
  int* s_prefix = s_order + kSortMax;
  int* s_len = reinterpret_cast<int*>(ks);  // scratch, dead before the first K tile lands

  const int T = p.cu[p.num_seqs];
  const bool sorted = p.num_seqs <= kSortMax;
  int total;
  if (sorted) {
    total = build_schedule<C::BM>(p, s_len, s_order, s_prefix);
  } else {
    total = p.num_seqs * p.heads * p.qt_max;
  }

  // XCD-aware placement: workgroup b runs on XCD b % 8; give each XCD a contiguous run
  // of the (longest-first) item list in every round.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int slot = (G % 8 == 0) ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  for (int base = 0; base < total; base += G) {
    const int u = base + slot;
    if (u >= total) break;
    int s, h, qt, a, L;
    if (sorted) {
      int lo = 0, hi = p.num_seqs - 1;   // last rank r with s_prefix[r] <= u
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= u) lo = mid; else hi = mid - 1;
      }
      s = s_order[lo];
      a = p.cu[s];
      L = p.cu[s + 1] - a;
      const int ntiles = (L + C::BM - 1) / C::BM;
      const int local = u - s_prefix[lo];
      h = local / ntiles;
      qt = local - h * ntiles;
    } else {
      const int per_seg = p.heads * p.qt_max;
      s = u / per_seg;
      const int rem = u - s * per_seg;
      h = rem / p.qt_max;
      qt = rem - h * p.qt_max;
      a = p.cu[s];
      L = p.cu[s + 1] - a;
    }
    // never touch rows outside [0, T), whatever the table says
    if (a < 0 || a >= T) continue;
    if (L > T - a) L = T - a;
    if (L <= 0 || qt * C::BM >= L) continue;
    process_tile<D, QB>(p, ks, vs, a, L, h, qt, T);
  }
}

// ---------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------
struct Variant {
  const void* fn;
  int bm;
  size_t lds;
};

template <int D, int QB>
Variant make_variant() {
  return Variant{reinterpret_cast<const void*>(&pfa_fwd_kernel<D, QB>), Tile<D, QB>::BM,
                 Tile<D, QB>::LDS_BYTES};
}

constexpr int kMaxDevices = 64;
constexpr int kVariants = 2;  // head_dim 64, 128
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kMaxDevices][kVariants];

int variant_index(int head_dim) { return head_dim == 64 ? 0 : 1; }

Variant variant_for(int head_dim) {
  if (head_dim == 64) return make_variant<64, 2>();
  return make_variant<128, 2>();
}

}  // namespace

extern "C" {

PFA_API const char* pfa_status_string(int status) {
  switch (status) {
    case PFA_OK: return "ok";
    case PFA_ERR_NULL: return "a required pointer is NULL";
    case PFA_ERR_NUM_SEQS: return "num_seqs must be >= 1";
    case PFA_ERR_HEADS: return "heads must be >= 1";
    case PFA_ERR_MAX_SEQLEN: return "max_seqlen must be >= 1";
    case PFA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case PFA_ERR_SCALE: return "scale must be finite and > 0";
    case PFA_ERR_ALIAS: return "out or lse aliases an input buffer";
    case PFA_ERR_CU_SEQLENS: return "cu_seqlens is malformed (must start at 0, be non-decreasing, lengths <= max_seqlen)";
    case PFA_ERR_DEVICE: return "no usable HIP device, or a device query failed";
    case PFA_ERR_LAUNCH: return "kernel launch failed";
    case PFA_ERR_SIZE: return "problem size exceeds the supported index range";
    default: return "unknown status";
  }
}

PFA_API int pfa_check_cu_seqlens(const int32_t* cu_host, int num_seqs, int max_seqlen,
                                 int64_t* total_out) {
  if (cu_host == nullptr) return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (cu_host[0] != 0) return PFA_ERR_CU_SEQLENS;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t len = (int64_t)cu_host[s + 1] - (int64_t)cu_host[s];
    if (len < 0 || len > max_seqlen) return PFA_ERR_CU_SEQLENS;
  }
  if (total_out != nullptr) *total_out = cu_host[num_seqs];
  return PFA_OK;
}

PFA_API int pfa_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* out, float* lse, hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens == nullptr || out == nullptr)
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[4] = {q, k, v, cu_seqlens};
  for (const void* in : ins)
    if (in == out || (lse != nullptr && in == static_cast<const void*>(lse))) return PFA_ERR_ALIAS;
  if (lse != nullptr && static_cast<const void*>(lse) == out) return PFA_ERR_ALIAS;
  const Variant var = variant_for(head_dim);
  const int64_t qt_max = ((int64_t)max_seqlen + var.bm - 1) / var.bm;
  const int64_t slots = (int64_t)num_seqs * heads * qt_max;
  if ((int64_t)heads * head_dim > INT32_MAX || slots > INT32_MAX) return PFA_ERR_SIZE;

  // ---- device limits (cached per device; a race only recomputes the same values)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PFA_ERR_DEVICE;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return PFA_ERR_DEVICE;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  const int vi = variant_index(head_dim);
  int occ = g_occ[dev][vi].load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (hipFuncSetAttribute(var.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)var.lds) != hipSuccess)
      return PFA_ERR_DEVICE;
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, var.fn, kThreads, var.lds) != hipSuccess || o <= 0)
      return PFA_ERR_DEVICE;
    occ = o;
    g_occ[dev][vi].store(occ, std::memory_order_relaxed);
  }

  int64_t grid = (int64_t)cus * occ;
  if (grid > slots) grid = slots;
  if (grid >= 8) grid -= grid % 8;   // keep whole rounds on every XCD

  Params prm;
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.cu = cu_seqlens;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.qt_max = (int)qt_max;
  prm.c = scale * kLog2e;
  void* args[] = {&prm};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)grid), dim3(kThreads), args, var.lds, stream);
  return err == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

}  // extern "C"
