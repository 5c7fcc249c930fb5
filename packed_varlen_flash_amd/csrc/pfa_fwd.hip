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
// gfx950 mapping (d = 128: one workgroup = 8 wave64s on one CU, two waves per SIMD;
// d = 64: 4 wave64s):
//   * work unit = (segment, head, BM-row query tile); a tile never spans two segments.
//     Tiles are listed longest segment first and handed out round-robin by a persistent
//     grid; each XCD receives contiguous runs of the list so the query tiles that share
//     one (segment, head) K/V stream sit behind the same L2.
//   * each wave owns QB blocks of 32 queries and keeps their Q fragments in VGPRs.
//   * K and V stages of 64 keys are double-buffered in LDS, loaded global -> LDS directly
//     by buffer loads bounded at the segment end, so rows past it read as zeros and no
//     neighbouring segment is ever touched.
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
#include <vector>

#include "pfa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kWave = 64;
constexpr int kHalf = 64;        // keys per softmax step (two 32-key sub-blocks)
constexpr int kStages = 2;       // LDS ring depth (stages)
constexpr int kRsrcFlags = 0x00020000;  // raw buffer resource word 3 (32-bit data format)
constexpr int kSortMax = 512;    // segment tables up to this size are sorted on device
constexpr int kWaitVmem = 0x0F70;   // s_waitcnt vmcnt(0), other counters unconstrained
// How far (base 2) a block max may exceed the running max before O and l are rescaled.
// 0 keeps the reference equal to the exact running max, so the largest weight of a row is
// exactly 1 and carries no bf16 rounding; a positive slack saves rescales (about 5% on
// 4096-token segments) but leaves that weight rounded, which on sharp softmax rows pushes
// the worst output error past 1e-2 of the exact result.
constexpr float kRescaleSlack = 0.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* cu_q;   // query segment table
  const int32_t* cu_k;   // key / value segment table (the same pointer for self-attention)
  __bf16* out;
  float* lse;
  int num_seqs;
  int heads;
  int qt_max;      // ceil(max_seqlen / BM): slots per (segment, head) in unsorted mode
  float c;         // scale * log2(e)
  // fused-projection variant only: row strides (elements) of q, k, v, and the rotary
  // angle tables [T, D/2] applied to q as it is loaded (nullptr: no rotation)
  int sq, sk, sv;
  const float* rope_cos;
  const float* rope_sin;
  // block-sparse variant only: key-block lists per (segment, layout head, query tile), CSR
  // row (s * layout_heads + hl) * qt_max + qt, entries kv_idx[kv_ptr[row] .. kv_ptr[row+1])
  const int32_t* kv_ptr;
  const int32_t* kv_idx;
  int nnz;
  int layout_heads;
  // FP8 P.V variant only: V as e4m3 codes [T, heads, D] and its dequantisation scales
  // [num_seqs, heads, D] (powers of two)
  const uint8_t* v8;
  const float* v_scale;
};

// Kernel variants: one segment table for queries and keys; separate query and key tables;
// one table with q, k, v read through row strides (views of one fused projection output)
// and q optionally rotated on load.
constexpr int kModeSelf = 0;
constexpr int kModeCross = 1;
constexpr int kModeQkv = 2;
constexpr int kModeSparse = 3;   // one table; each query tile reads only its listed key blocks
constexpr int kModeFp8 = 4;      // one table; P.V in FP8 (e4m3 weights and V)
constexpr int kModeSparseFp8 = 5;   // both: listed key blocks, P.V in FP8
constexpr bool mode_sparse(int mode) { return mode == kModeSparse || mode == kModeSparseFp8; }
constexpr bool mode_fp8(int mode) { return mode == kModeFp8 || mode == kModeSparseFp8; }
// FP8 weights: w = 2^8 p with p = 2^(s log2 e - m) in (0, 1], so w <= 256 < 448 (the
// largest e4m3 value) and the factor is folded into the exponent.
constexpr float kP8Log2 = 8.0f;
// Block-sparse variant: a compacted copy of the tile's key-block list lives in LDS after
// the schedule (count in the last slot), so segments are limited to this many key blocks.
constexpr int kSparseMaxBlocks = 1024;
constexpr int kSparseLdsBytes = (kSparseMaxBlocks + 4) * 4;
// Largest row stride (elements) of any input: 64 rows of it, in bytes, must stay within
// the 32-bit offsets of a buffer resource.
constexpr int64_t kMaxRowElems = int64_t(1) << 23;

// D: head_dim; QB: 32-query blocks per wave; NW: waves per workgroup; SK: keys per LDS
// stage (a multiple of 64).
template <int D, int QB, int NW = 4, int SK = 64>
struct Tile {
  static constexpr int THREADS = kWave * NW;
  static constexpr int BM = NW * QB * 32;           // query rows per workgroup tile
  static constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int TILE_BYTES = SK * D * 2;     // one K (or V) stage, unpadded
  static constexpr int CPT = SK * CPR / THREADS;    // chunks per thread per stage
  static constexpr int DT = D / 32;                 // 32-row output tiles along head_dim
  static constexpr int KSTEP = D / 16;              // 16-deep steps of the Q.K contraction
  static constexpr int SCHED_INTS = 2 * kSortMax + 8;
  static constexpr int CPR8 = D / 16;               // 16-byte chunks per e4m3 V row
  static constexpr int CPT8 = SK * CPR8 / THREADS;  // e4m3 V chunks per thread per stage
  static constexpr size_t LDS_BYTES = (size_t)kStages * 2 * TILE_BYTES + sizeof(int) * SCHED_INTS;
  static_assert(CPT * THREADS == SK * CPR, "stage must split evenly");
  static_assert(SK % kHalf == 0, "stages hold whole 64-key halves");
  static_assert(sizeof(int) * kSortMax <= (size_t)kStages * TILE_BYTES, "len scratch fits");
};

// LDS layout of a K or V stage: 16-byte chunks, row-major (row = key), with the chunk
// index XOR-swizzled inside each 256-byte line so the two read patterns are free of bank
// conflicts: K operand reads (16 lanes = 16 consecutive rows, one logical chunk) and
// transposed V reads (4 consecutive rows x 64 bytes per 32 lanes).
__device__ __forceinline__ int swz_k(int line) { return line & 15; }
__device__ __forceinline__ int swz_v(int line) { return (line & 3) << 2; }

// byte offset of logical (row, chunk) within a stage
template <int D, bool IS_K>
__device__ __forceinline__ int phys_off(int row, int chunk) {
  const int P = row * (D / 8) + chunk;
  const int line = P >> 4;
  const int sw = IS_K ? swz_k(line) : swz_v(line);
  return ((line << 4) | ((P & 15) ^ sw)) << 4;
}

// LDS layout of an e4m3 V stage: rows of D bytes (one key each), 16-byte chunks XORed
// with swz8(row) < D/16.  The transposed byte reads that build the P.V operand have 16
// lanes read 8 keys x 16 channels: keys 16q + {4g .. 4g+3, 8+4g .. 8+4g+3}, whose bits 1
// and 3 (d = 128) or bit 3 (d = 64) differ, so the swizzle spreads those 8 rows over
// distinct banks.
template <int D>
__device__ __forceinline__ int swz8(int row) {
  return D == 128 ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1)) : ((row >> 3) & 1);
}

// logical source offset (row * row_bytes + chunk * 16) of the e4m3 V chunk stored at
// physical chunk position P
template <int D>
__device__ __forceinline__ int logical_src8(int P, int row_bytes) {
  const int row = P / (D / 16);
  const int pc = P % (D / 16);
  return row * row_bytes + ((pc ^ swz8<D>(row)) << 4);
}

// logical byte offset (row * row_bytes + chunk * 16) of the chunk stored at physical
// chunk position P; the XOR swizzle is its own inverse
template <int D, bool IS_K>
__device__ __forceinline__ int logical_src(int P, int row_bytes) {
  const int line = P >> 4;
  const int sw = IS_K ? swz_k(line) : swz_v(line);
  const int Pl = (line << 4) | ((P & 15) ^ sw);
  return (Pl / (D / 8)) * row_bytes + (Pl % (D / 8)) * 16;
}

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
// Sorted mode (num_seqs <= kSortMax): s_order[r] = segment of rank r (key length, i.e.
// the work per query tile, descending; ties by index), s_prefix[r] = first item of rank
// r; a segment has heads * ceil(query length / BM) items, ordered head-major,
// query-tile-minor.  Returns the item count.
template <int BM, int THREADS>
__device__ int build_schedule(const int32_t* cu_q, const int32_t* cu_k, int n, int heads,
                              int* s_len, int* s_order, int* s_prefix) {
  const int tid = threadIdx.x;
  for (int s = tid; s < n; s += THREADS) {
    int L = cu_k[s + 1] - cu_k[s];
    s_len[s] = L > 0 ? L : 0;
  }
  __syncthreads();
  for (int s = tid; s < n; s += THREADS) {
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
  for (int r = tid; r < n; r += THREADS) {
    const int sg = s_order[r];
    int Lq = cu_q[sg + 1] - cu_q[sg];
    Lq = Lq > 0 ? Lq : 0;
    s_prefix[r + 1] = heads * ((Lq + BM - 1) / BM);
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
  for (int off = 1; off < n; off <<= 1) {
    int add[kSortMax / THREADS];
#pragma unroll
    for (int j = 0; j < kSortMax / THREADS; ++j) {
      const int r = tid + j * THREADS;
      add[j] = (r < n && r >= off) ? s_prefix[r + 1 - off] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kSortMax / THREADS; ++j) {
      const int r = tid + j * THREADS;
      if (r < n) s_prefix[r + 1] += add[j];
    }
    __syncthreads();
  }
  return s_prefix[n];
}

// ---------------------------------------------------------------------------------
// One query tile of one (segment, head).
//
// Keys are consumed in 64-key LDS stages held in a ring of kStages slots.  Per stage the
// wave computes both 32-key sub-blocks of S^T = K Q^T, runs one softmax head over the 64
// keys (mask, max, rescale decision), then the weights of sub-block 0, its PV product,
// the weights of sub-block 1 interleaved with that product's MFMAs, and the second PV.
// The loads of stage s+1 are issued right after the barrier that opens stage s, into the
// slot whose last readers that barrier retired.
// ---------------------------------------------------------------------------------
template <int D, int QB>
struct TileState {
  using C = Tile<D, QB>;
  bf16x8 qr[QB][C::KSTEP];       // Q fragments (B operand of K Q^T)
  f32x16 o[QB][C::DT];           // O^T accumulators
  float m_run[QB];               // running max (base-2 scaled)
  float l_run[QB];               // row sum of the fp32 weights (normalises O, gives the LSE)
};

// K operand fragments of one 32-key sub-block: kst points at the sub-block's first row;
// koff[t] is this lane's byte offset of (row n32, chunk 2t+g).
template <int D>
__device__ __forceinline__ void k_operands(const char* kst, const int (&koff)[D / 16],
                                           bf16x8 (&a)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a[t] = *reinterpret_cast<const bf16x8*>(kst + koff[t]);
}

// S^T (keys x queries) = K Q^T for both 32-key sub-blocks of a stage, the two accumulator
// chains interleaved so consecutive MFMAs never depend on each other.
template <int D, int QB>
__device__ __forceinline__ void qk_mfma(const bf16x8 (&ka)[D / 16], const bf16x8 (&kb)[D / 16],
                                        const bf16x8 (&qr)[QB][D / 16], f32x16 (&s0)[QB],
                                        f32x16 (&s1)[QB]) {
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[b][i] = 0.f;
      s1[b][i] = 0.f;
    }
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      s0[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t], qr[b][t], s0[b], 0, 0, 0);
      s1[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t], qr[b][t], s1[b], 0, 0, 0);
    }
}

// V^T operand fragments of one sub-block: vst points at its first row; voff[dt] is this
// lane's byte offset for the transposed read of rows 4g + i16/4 at d = 32dt + 16hh +
// 4(i16 & 3); the second read of each pair is 8 rows further.
template <int D>
__device__ __forceinline__ void v_operands(const char* vst, const int (&voff)[D / 32],
                                           bf16x8 (&va)[2][D / 32]) {
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* vp = vst + cc * 16 * D * 2 + voff[dt];
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 8 * D * 2));
      va[cc][dt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// O^T += V^T P^T for one sub-block, 16 keys per MFMA.
template <int D, int QB>
__device__ __forceinline__ void pv_mfma(TileState<D, QB>& st, const bf16x8 (&va)[2][D / 32],
                                        const bf16x8 (&pb)[QB][2]) {
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int b = 0; b < QB; ++b)
        st.o[b][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cc][dt], pb[b][cc], st.o[b][dt], 0, 0, 0);
}

// Online softmax head over a whole 64-key stage (both sub-blocks): one max, one rescale
// decision.  No weights are pending when it runs, so O is rescaled in place.
template <int D, int QB>
__device__ __forceinline__ void softmax_head64(TileState<D, QB>& st, f32x16 (&s0)[QB],
                                               f32x16 (&s1)[QB], int key0, int L, float c, int g) {
  using C = Tile<D, QB>;
  if (key0 + 64 > L) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + (i >> 2) * 8 + 4 * g + (i & 3);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        if (key >= L) s0[b][i] = -INFINITY;
        if (key + 32 >= L) s1[b][i] = -INFINITY;
      }
    }
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    float mx = fmaxf(s0[b][0], s0[b][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s0[b][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[b][i]);
    mx = partner_max(mx);
    const float mb = mx * c;
    if (__builtin_amdgcn_ballot_w64(mb > st.m_run[b] + kRescaleSlack) != 0) {
      const float m_new = fmaxf(st.m_run[b], mb);
      const float a = __builtin_amdgcn_exp2f(st.m_run[b] - m_new);
      st.m_run[b] = m_new;
      st.l_run[b] *= a;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][dt][i] *= a;
    }
  }
}

// Online softmax, second half (straight-line): P = 2^(s*c - m) as bf16 B operands and the
// row sum l_run of the fp32 weights, which normalises O and gives the LSE (a sum of the
// bf16-rounded weights could carry up to 2^-8 relative error, 3.9e-3, into the LSE of a
// sharp row).  With the exact running maximum each row's largest weight is 1 and exact in
// bf16, so normalising by the rounded weights' sum instead gains no accuracy; it cost 16
// dot products per stage in a loop bound by vector issue.  The sum chains straight into
// its running value, with no partial sums to seed or combine.
template <int D, int QB>
__device__ __forceinline__ void softmax_body(TileState<D, QB>& st, const f32x16 (&s)[QB],
                                             bf16x8 (&pb)[QB][2], float c) {
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float neg_m = -st.m_run[b];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[b][i], c, neg_m));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[b][i + 1], c, neg_m));
      st.l_run[b] += e0;
      st.l_run[b] += e1;
      const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
      pb[b][i >> 3][i & 7] = pr[0];
      pb[b][i >> 3][(i & 7) + 1] = pr[1];
    }
  }
}

// FP8 variant of softmax_body: weights w = 2^(s c - m + 8) rounded to e4m3 (nearest even)
// four to a register, sub-block `half` filling bytes 16 half .. 16 half + 15 of the P^T
// operand in the order of the accumulator elements; l_run adds the unrounded weights,
// which also normalise O.
template <int D, int QB>
__device__ __forceinline__ void softmax_body8(TileState<D, QB>& st, const f32x16 (&s)[QB],
                                              i32x8 (&pw)[QB], int half, float c) {
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float off = kP8Log2 - st.m_run[b];
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[b][i], c, off));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[b][i + 1], c, off));
      const float e2 = __builtin_amdgcn_exp2f(fmaf(s[b][i + 2], c, off));
      const float e3 = __builtin_amdgcn_exp2f(fmaf(s[b][i + 3], c, off));
      st.l_run[b] += e0;
      st.l_run[b] += e1;
      st.l_run[b] += e2;
      st.l_run[b] += e3;
      int w = 0;
      w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, w, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
      pw[b][half * 4 + (i >> 2)] = w;
    }
  }
}

// The V^T operand of one 32-channel output tile for all 64 keys of a stage (e4m3): byte
// 8q + r of lane (channel, g) is key 16q + 8(r/4) + 4g + r%4, matching the weight bytes
// of softmax_body8.  Four transposed 8-byte reads; voff8 is the lane's offset for q = 0.
template <int D>
__device__ __forceinline__ i32x8 v8_operand(const char* vst, int voff8) {
  i32x8 a;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vst + voff8 + q * 16 * D));
    a[2 * q] = x[0];
    a[2 * q + 1] = x[1];
  }
  return a;
}

// One 64-key stage of the FP8 variant: QK and the softmax head as in stage_body, then the
// weights of both sub-blocks (e4m3) and one 32x32x64 FP8 MFMA per output tile.
template <int D, int QB, int SK, typename IssueFn>
__device__ __forceinline__ void stage_body_fp8(TileState<D, QB>& st, char* __restrict__ knext,
                                               char* __restrict__ vnext, const char* __restrict__ kcur,
                                               const char* __restrict__ vcur, bool issue,
                                               const IssueFn& issue_fn, int s, int kbase, int L,
                                               const int (&koff)[D / 16], const int (&voff8)[D / 32],
                                               float c, int g) {
  static_assert(SK == kHalf, "one 64-key head per stage");
  if (issue) issue_fn(knext, vnext, s + 1);
  f32x16 s0[QB], s1[QB];
  i32x8 pw[QB];
  bf16x8 ka[D / 16], kb[D / 16];
  k_operands<D>(kcur, koff, ka);
  k_operands<D>(kcur + 32 * D * 2, koff, kb);
  qk_mfma<D, QB>(ka, kb, st.qr, s0, s1);
  softmax_head64<D, QB>(st, s0, s1, kbase, L, c, g);
  softmax_body8<D, QB>(st, s0, pw, 0, c);
  i32x8 va[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) va[dt] = v8_operand<D>(vcur, voff8[dt]);
  softmax_body8<D, QB>(st, s1, pw, 1, c);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int b = 0; b < QB; ++b)
      st.o[b][dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[dt], pw[b], st.o[b][dt], 0, 0, 0, 0,
                                                                   0, 0);
}

// Interleave n MFMAs with the VALU work around them, `valu` VALU instructions after each.
template <int N, int VALU>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VALU, 0);
  }
}

// One stage of keys kbase .. kbase + SK - 1: issue the next stage's loads into its slot,
// then QK, softmax and PV on the current slot.  The four LDS pointers are restrict-qualified: the next slot and
// the current slot never overlap, which lets the compiler keep the current slot's reads
// from waiting on the next slot's loads.  The straight-line half of each sub-block's
// softmax shares a basic block with the MFMAs of the neighbouring sub-block (QK of the
// next, PV of the previous), so the MFMA pipe and the VALU work side by side.
template <int D, int QB, int SK, typename IssueFn>
__device__ __forceinline__ void stage_body(TileState<D, QB>& st, char* __restrict__ knext,
                                           char* __restrict__ vnext, const char* __restrict__ kcur,
                                           const char* __restrict__ vcur, bool issue,
                                           const IssueFn& issue_fn, int s, int kbase, int L,
                                           const int (&koff)[D / 16], const int (&voff)[D / 32],
                                           float c, int g) {
  constexpr int NQK = QB * D / 16;   // MFMAs of one sub-block's QK (and of its PV)
  if (issue) issue_fn(knext, vnext, s + 1);
#pragma unroll
  for (int half = 0; half < SK / kHalf; ++half) {
    const int key0 = kbase + half * kHalf;     // first key of this half (kbase: of the stage)
    if (half > 0 && key0 >= L) break;            // nothing left in this stage
    const char* kh = kcur + half * kHalf * D * 2;
    const char* vh = vcur + half * kHalf * D * 2;
    f32x16 s0[QB], s1[QB];
    bf16x8 p0[QB][2], p1[QB][2];
    bf16x8 ka[D / 16], kb[D / 16];
    bf16x8 va[2][D / 32];
    k_operands<D>(kh, koff, ka);
    k_operands<D>(kh + 32 * D * 2, koff, kb);
    qk_mfma<D, QB>(ka, kb, st.qr, s0, s1);
    softmax_head64<D, QB>(st, s0, s1, key0, L, c, g);
    softmax_body<D, QB>(st, s0, p0, c);
    v_operands<D>(vh, voff, va);
    pv_mfma<D, QB>(st, va, p0);
    softmax_body<D, QB>(st, s1, p1, c);
    interleave_mfma_valu<NQK, 8 * 16 / NQK>();
    v_operands<D>(vh + 32 * D * 2, voff, va);
    pv_mfma<D, QB>(st, va, p1);
  }
}

// Rotary position embedding, rotate-half pairing, of one pair of 8-feature chunks: lo
// holds features i .. i+7 of a row and hi their partners i + D/2 .. i + D/2 + 7; cs and
// sn point at the cosines and sines of those 8 pairs' angles.  Each pair (a, b) turns to
// (a cos - b sin, b cos + a sin), evaluated in fp32 and rounded once to bf16 (nearest
// even).  The DiT block of the Mage-Flow page (section on its fusion opportunities)
// rotates q and k between the QKV projection and attention.
__device__ __forceinline__ void rope_rotate(bf16x8& lo, bf16x8& hi, const float* cs, const float* sn) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(sn);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(sn + 4);
  bf16x8 nlo, nhi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = e < 4 ? c0[e & 3] : c1[e & 3];
    const float sv = e < 4 ? s0[e & 3] : s1[e & 3];
    const float a = (float)lo[e];
    const float b = (float)hi[e];
    nlo[e] = (__bf16)(a * c - b * sv);
    nhi[e] = (__bf16)(b * c + a * sv);
  }
  lo = nlo;
  hi = nhi;
}

// MODE also keys the instantiation to its kernel variant (the HIP host pass rejects a
// device template specialisation shared by two kernel templates' instantiations).
template <int D, int QB, int NW, int SK, int MODE>
__device__ __forceinline__ void process_tile(const Params& p, __bf16* ks, __bf16* vs, int* s_blk,
                                             int seg, int qa, int Lq, int ka, int Lk, int h,
                                             int qt, int Tq) {
  using C = Tile<D, QB, NW, SK>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int n32 = lane & 31;         // query column (S^T) / key row of the K operand
  const int g = lane >> 5;           // half-wave
  const int i16 = lane & 15;
  const int hh = (lane >> 4) & 1;
  const int64_t rs = (int64_t)p.heads * D;  // elements between consecutive output tokens
  const int64_t q_rs = MODE == kModeQkv ? (int64_t)p.sq : rs;   // ... and input tokens
  const int64_t k_rs = MODE == kModeQkv ? (int64_t)p.sk : rs;
  const int64_t v_rs = MODE == kModeQkv ? (int64_t)p.sv : rs;
  const int64_t head_off = (int64_t)h * D;
  const __bf16* qbase = p.q + (int64_t)qa * q_rs + head_off;
  const __bf16* kbase = p.k + (int64_t)ka * k_rs + head_off;
  const __bf16* vbase = p.v + (int64_t)ka * v_rs + head_off;
  const uint8_t* v8base = mode_fp8(MODE) ? p.v8 + (int64_t)ka * rs + head_off : nullptr;
  const int q0 = qt * C::BM + wave * (QB * 32);
  int ns = (Lk + SK - 1) / SK;             // LDS stages (0 when the key segment is empty)
  const float c = p.c;
  if constexpr (mode_sparse(MODE)) {
    // The tile's list, compacted by wave 0 into LDS: entries outside the segment's key
    // blocks are dropped, the rest keep their order.  ns becomes the number kept.  (The
    // previous tile's last barrier retired every reader of the old list.)
    static_assert(SK == 64, "key blocks are 64-key stages");
    if (wave == 0) {
      const int64_t row = ((int64_t)seg * p.layout_heads + (p.layout_heads == 1 ? 0 : h)) * p.qt_max + qt;
      int e0 = 0, e1 = 0;
      if (qt < p.qt_max) {
        e0 = min(max(p.kv_ptr[row], 0), p.nnz);
        e1 = min(max(p.kv_ptr[row + 1], e0), p.nnz);
      }
      int cnt = 0;
      for (int base = e0; base < e1; base += kWave) {
        const int i = base + lane;
        const int b = i < e1 ? p.kv_idx[i] : -1;
        const bool ok = b >= 0 && b < ns;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (ok && pos < kSparseMaxBlocks) s_blk[pos] = b;
        cnt += __builtin_popcountll(m);
      }
      if (lane == 0) s_blk[kSparseMaxBlocks] = cnt < kSparseMaxBlocks ? cnt : kSparseMaxBlocks;
    }
    __syncthreads();
    ns = __builtin_amdgcn_readfirstlane(s_blk[kSparseMaxBlocks]);
  }
  // first key of stage i: consecutive 64-key stages, or the listed blocks in list order
  auto stage_key = [&](int i) {
    if constexpr (mode_sparse(MODE)) return __builtin_amdgcn_readfirstlane(s_blk[i]) * SK;
    else return i * SK;
  };

  TileState<D, QB> st;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int row = q0 + b * 32 + n32;
#pragma unroll
    for (int t = 0; t < C::KSTEP; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < Lq) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)row * q_rs + 16 * t + 8 * g);
      st.qr[b][t] = __builtin_bit_cast(bf16x8, x);
    }
    if constexpr (MODE == kModeQkv) {
      // rotate-half RoPE: the lane's chunk t holds features 16t + 8g + 0..7 and chunk
      // t + KSTEP/2 their partners D/2 further on, so each pair is rotated in registers
      if (p.rope_cos != nullptr && row < Lq) {
        const int64_t tab = (int64_t)(qa + row) * (D / 2);
#pragma unroll
        for (int t = 0; t < C::KSTEP / 2; ++t)
          rope_rotate(st.qr[b][t], st.qr[b][t + C::KSTEP / 2], p.rope_cos + tab + 16 * t + 8 * g,
                      p.rope_sin + tab + 16 * t + 8 * g);
      }
    }
    st.m_run[b] = -INFINITY;
    st.l_run[b] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[b][dt][i] = 0.f;
  }

  // ---- per-lane LDS offsets (fixed for the whole tile)
  int koff[C::KSTEP], voff[C::DT];
#pragma unroll
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, true>(n32, 2 * t + g);
  if constexpr (mode_fp8(MODE)) {
    // transposed e4m3 reads: lane i16 supplies row i16/2 (keys 4g + 0..3, then 8 + 4g +
    // 0..3) and half i16 & 1 of the 16 channels 32dt + 16hh ..; v8_operand adds 16q rows
    const int r = i16 >> 1;
    const int row = r < 4 ? 4 * g + r : 8 + 4 * g + (r - 4);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      voff[dt] = row * D + (((2 * dt + hh) ^ swz8<D>(row)) << 4) + 8 * (i16 & 1);
  } else {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      voff[dt] = phys_off<D, false>(4 * g + (i16 >> 2), 4 * dt + 2 * hh + ((i16 & 3) >> 1)) + 8 * (i16 & 1);
  }

  // ---- stage loads: global -> LDS directly (no registers).  Lane l of the wave's i-th
  // load writes physical chunk (wave*CPT + i)*64 + l, fetched from its logical source.
  // A buffer resource bounded at the segment end returns zeros for rows >= L, so no row
  // of a neighbouring segment is ever read.
  // the host keeps 64 rows of every stride within int range
  const int kbytes = (int)(k_rs * 2);
  const int vbytes = (int)(v_rs * 2);
  char* const kring = reinterpret_cast<char*>(ks);
  char* const vring = reinterpret_cast<char*>(vs);
  int src_k[C::CPT], src_v[C::CPT];      // logical source offsets of this lane's chunks
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int P = (wave * C::CPT + i) * 64 + lane;
    src_k[i] = logical_src<D, true>(P, kbytes);
    if constexpr (mode_fp8(MODE)) {
      if (i < C::CPT8) src_v[i] = logical_src8<D>((wave * C::CPT8 + i) * 64 + lane, (int)rs);
    } else {
      src_v[i] = logical_src<D, false>(P, vbytes);
    }
  }
  auto issue_fn = [&](char* kdst, char* vdst, int stage) {
    const int kb = stage_key(stage);
    const int rows = (Lk - kb < SK) ? (Lk - kb) : SK;
    __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)kb * k_rs), 0, rows * kbytes, kRsrcFlags);
    kdst += wave * C::CPT * 1024;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + i * 1024), 16, src_k[i], 0, 0, 0);
    if constexpr (mode_fp8(MODE)) {
      __amdgpu_buffer_rsrc_t r8 = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(v8base + (int64_t)kb * rs), 0, rows * (int)rs, kRsrcFlags);
      vdst += wave * C::CPT8 * 1024;
#pragma unroll
      for (int i = 0; i < C::CPT8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r8, (lds_void*)(vdst + i * 1024), 16, src_v[i], 0, 0, 0);
    } else {
      __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)kb * v_rs), 0, rows * vbytes, kRsrcFlags);
      vdst += wave * C::CPT * 1024;
#pragma unroll
      for (int i = 0; i < C::CPT; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + i * 1024), 16, src_v[i], 0, 0, 0);
    }
  };

  // ---- stage loop.  Stage s sits in slot s % 2; the loads of stage s+1 are issued
  // right after the barrier that retires every reader of its slot, and have the whole of
  // stage s to land.  Unrolled by two so both slot offsets are immediates.
  static_assert(kStages == 2, "the stage loop alternates two slots");
  // no keys, no loads: a zero-row stage would still zero-fill slot 0, which the epilogue
  // reuses for the output
  if (ns > 0) issue_fn(kring, vring, 0);
  for (int s = 0; s < ns; s += 2) {
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __syncthreads();
    if constexpr (mode_fp8(MODE))
      stage_body_fp8<D, QB, SK>(st, kring + C::TILE_BYTES, vring + C::TILE_BYTES, kring, vring, s + 1 < ns,
                                issue_fn, s, stage_key(s), Lk, koff, voff, c, g);
    else
      stage_body<D, QB, SK>(st, kring + C::TILE_BYTES, vring + C::TILE_BYTES, kring, vring, s + 1 < ns,
                            issue_fn, s, stage_key(s), Lk, koff, voff, c, g);
    if (s + 1 >= ns) break;
    __builtin_amdgcn_s_waitcnt(kWaitVmem);
    __syncthreads();
    if constexpr (mode_fp8(MODE))
      stage_body_fp8<D, QB, SK>(st, kring, vring, kring + C::TILE_BYTES, vring + C::TILE_BYTES, s + 2 < ns,
                                issue_fn, s + 1, stage_key(s + 1), Lk, koff, voff, c, g);
    else
      stage_body<D, QB, SK>(st, kring, vring, kring + C::TILE_BYTES, vring + C::TILE_BYTES, s + 2 < ns,
                            issue_fn, s + 1, stage_key(s + 1), Lk, koff, voff, c, g);
  }
  __syncthreads();   // every wave has left the ring

  // ---- epilogue: O = acc / l_run in bf16 (round to nearest even), LSE = ln2 * (m + log2
  // l_run).  O goes out through LDS: each wave writes its (QB*32) x D block into the free
  // ring in the swizzled K layout, then reads it back as whole 16-byte chunks of
  // consecutive rows, so 16 lanes store 256 contiguous bytes instead of every store
  // instruction touching 16-byte pieces of 32 different rows.
  static_assert(NW * QB * 32 * D * 2 <= 2 * kStages * C::TILE_BYTES, "O staging fits the ring");
  char* const ost = kring + wave * (QB * 32 * D * 2);
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lt = partner_sum(st.l_run[b]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;   // no keys: O = 0 (and LSE = -inf)
    const int r = b * 32 + n32;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        // this lane's channels 32dt + 8ii + 4g + e; FP8 dequantises V per channel here
        f32x4 sc = {inv, inv, inv, inv};
        if constexpr (mode_fp8(MODE))
          sc = inv * *reinterpret_cast<const f32x4*>(p.v_scale + ((int64_t)seg * p.heads + h) * D + 32 * dt +
                                                     8 * ii + 4 * g);
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[b][dt][4 * ii + e] * sc[e]);
        *reinterpret_cast<bf16x4*>(ost + phys_off<D, true>(r, 4 * dt + ii) + 8 * g) = w;
      }
    const float mfix = mode_fp8(MODE) ? st.m_run[b] - kP8Log2 : st.m_run[b];   // FP8 sums 2^8 p
    if (p.lse != nullptr && g == 0 && q0 + r < Lq)
      p.lse[(int64_t)h * Tq + qa + q0 + r] = (mfix + __builtin_amdgcn_logf(lt)) * kLn2;
  }
  __syncthreads();
  constexpr int OCH = QB * 32 * C::CPR;      // 16-byte chunks of the wave's block
  static_assert(OCH % kWave == 0, "whole chunk rows per lane");
#pragma unroll
  for (int k = 0; k < OCH / kWave; ++k) {
    const int P = k * kWave + lane;
    const int r = P / C::CPR;
    const int ch = P % C::CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(ost + phys_off<D, true>(r, ch));
    if (q0 + r < Lq)
      *reinterpret_cast<u32x4*>(p.out + (int64_t)(qa + q0 + r) * rs + head_off + ch * 8) = x;
  }
  __syncthreads();   // the next tile's first stage overwrites the ring
}

// kModeCross: separate query and key tables; otherwise the key table is the query table
// (known at compile time, so the key-side offsets and lengths fold into the query ones).
template <int D, int QB, int NW, int SK, int WPE, int MODE>
__global__ void __launch_bounds__(kWave * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
pfa_fwd_kernel(Params p) {
  const int32_t* const cu_k = MODE == kModeCross ? p.cu_k : p.cu_q;
  using C = Tile<D, QB, NW, SK>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __bf16* ks = reinterpret_cast<__bf16*>(smem);
  __bf16* vs = reinterpret_cast<__bf16*>(smem + kStages * C::TILE_BYTES);
  int* s_order = reinterpret_cast<int*>(smem + 2 * kStages * C::TILE_BYTES);
  int* s_prefix = s_order + kSortMax;
  int* s_blk = s_order + C::SCHED_INTS;     // block-sparse variant only (its LDS is larger)
  int* s_len = reinterpret_cast<int*>(ks);  // scratch, dead before the first K tile lands

  const int Tq = p.cu_q[p.num_seqs];
  const int Tk = cu_k[p.num_seqs];
  const bool sorted = p.num_seqs <= kSortMax;
  int total;
  if (sorted) {
    total = build_schedule<C::BM, C::THREADS>(p.cu_q, cu_k, p.num_seqs, p.heads, s_len, s_order,
                                              s_prefix);
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
    int s, h, qt;
    if (sorted) {
      int lo = 0, hi = p.num_seqs - 1;   // last rank r with s_prefix[r] <= u
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_prefix[mid] <= u) lo = mid; else hi = mid - 1;
      }
      s = s_order[lo];
      const int ntiles = (p.cu_q[s + 1] - p.cu_q[s] + C::BM - 1) / C::BM;
      const int local = u - s_prefix[lo];
      h = local / ntiles;
      qt = local - h * ntiles;
    } else {
      const int per_seg = p.heads * p.qt_max;
      s = u / per_seg;
      const int rem = u - s * per_seg;
      h = rem / p.qt_max;
      qt = rem - h * p.qt_max;
    }
    const int qa = p.cu_q[s];
    int Lq = p.cu_q[s + 1] - qa;
    // never touch rows outside [0, Tq) / [0, Tk), whatever the tables say
    if (qa < 0 || qa >= Tq) continue;
    if (Lq > Tq - qa) Lq = Tq - qa;
    if (Lq <= 0 || qt * C::BM >= Lq) continue;
    int ka = qa, Lk = Lq;
    if (MODE == kModeCross) {
      ka = cu_k[s];
      Lk = cu_k[s + 1] - ka;
      if (ka < 0 || ka > Tk) ka = Tk;
      if (Lk > Tk - ka) Lk = Tk - ka;
      if (Lk < 0) Lk = 0;
    }
    process_tile<D, QB, NW, SK, MODE>(p, ks, vs, s_blk, s, qa, Lq, ka, Lk, h, qt, Tq);
  }
}

// ---------------------------------------------------------------------------------
// Key rotation pass of the fused-projection forward: k_rot[t, h, :] = RoPE(k[t, h, :])
// with token t's angles, written contiguous [T, heads, D].  The forward kernel re-reads
// every key stage once per query tile of its segment, so the keys are rotated once here
// rather than at each load; queries are rotated in registers where they are loaded.
// One thread per pair of 16-byte chunks (features 8j .. 8j+7 and their partners D/2
// further on); consecutive threads cover consecutive chunks, then heads, then tokens,
// so a wave reads and writes whole contiguous rows.  HBM-bound.
// ---------------------------------------------------------------------------------
constexpr int kRopeThreads = 256;

struct RopeParams {
  const __bf16* src;     // row t, head h at src + t * stride + h * D
  __bf16* dst;           // [T, heads, D]
  const float* cos;      // [T, D/2]
  const float* sin;
  const int32_t* cu;     // T = cu[num_seqs], read on the device
  int num_seqs;
  int heads;
  int stride;
};

template <int D>
__global__ void __launch_bounds__(kRopeThreads) pfa_rope_k_kernel(RopeParams r) {
  constexpr int CPH = D / 16;                  // chunk pairs per (token, head) row
  const int64_t T = r.cu[r.num_seqs];
  const int64_t n = T * r.heads * CPH;         // <= 0 for a table that ends below zero
  for (int64_t idx = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * kRopeThreads) {
    const int64_t row = idx / CPH;
    const int j = (int)(idx - row * CPH);
    const int64_t t = row / r.heads;
    const int h = (int)(row - t * r.heads);
    const __bf16* src = r.src + t * r.stride + (int64_t)h * D + 8 * j;
    bf16x8 lo = *reinterpret_cast<const bf16x8*>(src);
    bf16x8 hi = *reinterpret_cast<const bf16x8*>(src + D / 2);
    rope_rotate(lo, hi, r.cos + t * (D / 2) + 8 * j, r.sin + t * (D / 2) + 8 * j);
    __bf16* dst = r.dst + row * D + 8 * j;
    *reinterpret_cast<bf16x8*>(dst) = lo;
    *reinterpret_cast<bf16x8*>(dst + D / 2) = hi;
  }
}

// ---------------------------------------------------------------------------------
// Backward.  For upstream gradient dO of O, with P the softmax of each query row over
// its segment (recomputed from the forward's LSE) and s = scale q.k, the chain rule of
// the forward definition gives (per segment and head)
//     dV = P^T dO,  dP = dO V^T,  delta_i = sum_j P_ij dP_ij = dO_i . O_i,
//     dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
// Three launches, no atomics and no scratch of the library's own:
//   * prep: ws[0] = -LSE * log2(e) and ws[1] = delta = rowsum(dO * O), fp32 [H, T] each,
//     in the caller's workspace;
//   * dK/dV: one work item = 128 keys of one (segment, head), stationary in VGPRs as the
//     B operands of S = Q K^T and dP = dO V^T (lanes hold keys); the segment's Q and dO
//     stream through LDS in 64-row stages; dV^T += dO^T P and dK^T += Q^T dS take their
//     A operands from transposed LDS reads of the same stages;
//   * dQ: one work item = 128 queries; the forward's shape: S^T = K Q^T, dP^T = V dO^T
//     (lanes hold queries), dQ^T += K^T dS^T with K^T from transposed LDS reads.
// Every stage tile is stored in the K swizzle (row reads conflict-free); the transposed
// reads take explicit per-lane offsets for each 16-row step and 8-row half, since that
// swizzle does not keep a constant pattern 8 rows apart.
// ---------------------------------------------------------------------------------
// waves per workgroup (one per SIMD).  dK/dV holds two accumulators and the stationary K
// and V fragments (419 registers at d = 128), so one workgroup fills a CU; dQ loads its
// two operand sets one after the other and fits 256 registers, so two workgroups share a
// CU (its few spills are per-item offsets, reloaded outside the stage loop).
constexpr int kBwdNW = 4;
constexpr int kBwdRows = kBwdNW * 32;      // keys (dK/dV) or queries (dQ) per work item
constexpr int kBwdStage = 64;              // rows per streamed stage

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* out;
  const __bf16* dout;
  const float* lse;
  float* ws;              // [2][heads][T]: -LSE*log2(e), then delta
  const int32_t* cu;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int num_seqs;
  int heads;
  int tiles_max;          // ceil(max_seqlen / kBwdRows): slots per (segment, head), unsorted mode
  float c;                // scale * log2(e)
  float scale;
};

template <int D>
struct BwdTile {
  static constexpr int THREADS = kWave * kBwdNW;
  static constexpr int CPR = D / 8;                          // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBwdStage * D * 2;       // one 64-row bf16 tile
  static constexpr int CPT = kBwdStage * CPR / THREADS;      // chunks per thread per tile
  static constexpr int DT = D / 32;
  static constexpr int KSTEP = D / 16;
  static constexpr int ROWF_BYTES = kBwdStage * 4;           // one 64-row fp32 vector
  // dK/dV: [Q ring][dO ring][row-vector ring: 2 x (neg_lse2, delta)] + schedule
  static constexpr size_t LDS_DKDV = (size_t)kStages * 2 * TILE_BYTES + kStages * 2 * ROWF_BYTES +
                                     sizeof(int) * (2 * kSortMax + 8);
  // dQ: [K ring][V ring] + schedule
  static constexpr size_t LDS_DQ = (size_t)kStages * 2 * TILE_BYTES + sizeof(int) * (2 * kSortMax + 8);
  static_assert(CPT * THREADS == kBwdStage * CPR, "stage must split evenly");
  static_assert(kBwdNW * 32 * D * 2 * 2 <= kStages * 2 * TILE_BYTES, "two output blocks fit the ring");
};

// Transposed A-operand reads of one 32-row sub-block (rows of the tile = the MFMA's k):
// off[cc][h][dt] is this lane's byte offset for 16-row step cc, 8-row half h.
template <int D>
__device__ __forceinline__ void t_operands(const char* base, const int (&off)[2][2][D / 32],
                                           bf16x8 (&va)[2][D / 32]) {
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off[cc][0][dt]));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off[cc][1][dt]));
      va[cc][dt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
}

// Offsets for t_operands over a K-swizzled tile: the same (row, chunk, half) pattern the
// forward uses for its V^T reads, resolved per row.
template <int D>
__device__ __forceinline__ void t_offsets(int lane, int (&off)[2][2][D / 32]) {
  const int g = lane >> 5, i16 = lane & 15, hh = (lane >> 4) & 1;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        off[cc][h][dt] = phys_off<D, true>(16 * cc + 8 * h + 4 * g + (i16 >> 2),
                                           4 * dt + 2 * hh + ((i16 & 3) >> 1)) + 8 * (i16 & 1);
}

// One 32-row block of an accumulator in the O^T layout (lane = row, values d = 32dt +
// 8(i/4) + 4g + i%4), times mul, stored as bf16 rows r < valid of dst (row stride rs)
// through the wave's LDS block ost (the forward's epilogue, factored).
template <int D>
__device__ __forceinline__ void stage_rows(const f32x16 (&acc)[D / 32], float mul, char* ost,
                                           int n32, int g) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[dt][4 * ii + e] * mul);
      *reinterpret_cast<bf16x4*>(ost + phys_off<D, true>(n32, 4 * dt + ii) + 8 * g) = w;
    }
}

template <int D>
__device__ __forceinline__ void store_rows(const char* ost, int lane, __bf16* dst, int64_t rs, int valid) {
  constexpr int CPR = D / 8;
  constexpr int OCH = 32 * CPR;
#pragma unroll
  for (int k = 0; k < OCH / kWave; ++k) {
    const int P = k * kWave + lane;
    const int r = P / CPR;
    const int ch = P % CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(ost + phys_off<D, true>(r, ch));
    if (r < valid) *reinterpret_cast<u32x4*>(dst + (int64_t)r * rs + ch * 8) = x;
  }
}

// prep: ws[0][h][t] = -LSE[h][t] * log2(e); ws[1][h][t] = sum_d dO[t,h,d] O[t,h,d].
// One thread per (token, head) row, grid-stride over T * heads rows.
template <int D>
__device__ __forceinline__ void bwd_prep_row(const BwdParams& p, int T, int64_t row) {
  const int64_t t = row / p.heads;
  const int h = (int)(row - t * p.heads);
  const bf16x8* o = reinterpret_cast<const bf16x8*>(p.out + row * D);
  const bf16x8* d = reinterpret_cast<const bf16x8*>(p.dout + row * D);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const bf16x8 a = o[c], b = d[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
  }
  const int64_t idx = (int64_t)h * T + t;
  p.ws[idx] = -p.lse[idx] * kLog2e;
  p.ws[(int64_t)p.heads * T + idx] = acc;
}

template <int D>
__global__ void __launch_bounds__(256) pfa_bwd_prep_kernel(BwdParams p) {
  const int T = p.cu[p.num_seqs];   // T is known only on the device
  for (int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x; row < (int64_t)T * p.heads;
       row += (int64_t)gridDim.x * 256)
    bwd_prep_row<D>(p, T, row);
}

// Decode work item u of a sorted or slot-enumerated schedule into (segment start, length,
// head, tile); false if the item is empty.
template <int BT>
__device__ __forceinline__ bool bwd_item(const BwdParams& p, int u, bool sorted, const int* s_order,
                                         const int* s_prefix, int T, int& a, int& L, int& h, int& tile) {
  int s;
  if (sorted) {
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= u) lo = mid; else hi = mid - 1;
    }
    s = s_order[lo];
    const int ntiles = (p.cu[s + 1] - p.cu[s] + BT - 1) / BT;
    const int local = u - s_prefix[lo];
    h = local / ntiles;
    tile = local - h * ntiles;
  } else {
    const int per_seg = p.heads * p.tiles_max;
    s = u / per_seg;
    const int rem = u - s * per_seg;
    h = rem / p.tiles_max;
    tile = rem - h * p.tiles_max;
  }
  a = p.cu[s];
  L = p.cu[s + 1] - a;
  if (a < 0 || a >= T) return false;
  if (L > T - a) L = T - a;
  return L > 0 && tile * BT < L;
}

// Loads of one 64-row bf16 stage (rows [r0, r0 + 64) of a segment starting at element
// base, bounded at L) into a K-swizzled LDS tile; rows >= L read as zeros.
// TAG keys the instantiation to its kernel (the HIP host pass rejects a specialisation
// holding buffer-to-LDS load builtins once two kernel templates have used it).
template <int D, int CPT, int TAG>
__device__ __forceinline__ void bwd_issue_tile(const __bf16* base, int r0, int L, int64_t rs,
                                               int row_bytes, char* dst, const int (&src)[CPT],
                                               int wave) {
  using C = BwdTile<D>;
  static_assert(CPT == C::CPT, "one source offset per chunk group");
  const int rows = (L - r0 < kBwdStage) ? (L - r0) : kBwdStage;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * rs), 0, rows * row_bytes, kRsrcFlags);
  dst += wave * C::CPT * 1024;
#pragma unroll
  for (int i = 0; i < C::CPT; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, src[i], 0, 0, 0);
}

// ---- dK / dV
template <int D>
__global__ void __launch_bounds__(kWave * kBwdNW) __attribute__((amdgpu_waves_per_eu(1, 1)))
pfa_bwd_dkdv_kernel(BwdParams p) {
  using C = BwdTile<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* const qring = reinterpret_cast<char*>(smem);
  char* const dring = qring + kStages * C::TILE_BYTES;
  char* const fring = dring + kStages * C::TILE_BYTES;            // [slot][neg_lse2 | delta]
  int* s_order = reinterpret_cast<int*>(fring + kStages * 2 * C::ROWF_BYTES);
  int* s_prefix = s_order + kSortMax;
  int* s_len = reinterpret_cast<int*>(qring);

  const int T = p.cu[p.num_seqs];
  const bool sorted = p.num_seqs <= kSortMax;
  const int total = sorted ? build_schedule<kBwdRows, C::THREADS>(p.cu, p.cu, p.num_seqs, p.heads,
                                                                   s_len, s_order, s_prefix)
                           : p.num_seqs * p.heads * p.tiles_max;
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int slot = (G % 8 == 0) ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  const int g = lane >> 5;
  const int64_t rs = (int64_t)p.heads * D;
  const int row_bytes = (int)(rs * 2);
  int koff[C::KSTEP];
#pragma unroll
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, true>(n32, 2 * t + g);
  int toff[2][2][C::DT];
  t_offsets<D>(lane, toff);
  int src[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) src[i] = logical_src<D, true>((wave * C::CPT + i) * 64 + lane, row_bytes);
  if (sorted) __syncthreads();   // s_len aliases the Q ring

  for (int u = slot; u < total; u += G) {
    int a, L, h, kt;
    if (!bwd_item<kBwdRows>(p, u, sorted, s_order, s_prefix, T, a, L, h, kt)) continue;
    const int64_t head_off = (int64_t)h * D;
    const int k0 = kt * kBwdRows + wave * 32;        // this wave's first key
    // stationary K^T and V^T fragments (B operands; lane n32 = key k0 + n32)
    bf16x8 kr[C::KSTEP], vr[C::KSTEP];
    {
      const int key = k0 + n32;
      const __bf16* kp = p.k + (int64_t)(a + key) * rs + head_off;
      const __bf16* vp = p.v + (int64_t)(a + key) * rs + head_off;
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (key < L) {
          x = *reinterpret_cast<const u32x4*>(kp + 16 * t + 8 * g);
          y = *reinterpret_cast<const u32x4*>(vp + 16 * t + 8 * g);
        }
        kr[t] = __builtin_bit_cast(bf16x8, x);
        vr[t] = __builtin_bit_cast(bf16x8, y);
      }
    }
    f32x16 dkt[C::DT], dvt[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dkt[dt][i] = dvt[dt][i] = 0.f;

    const __bf16* qbase = p.q + (int64_t)a * rs + head_off;
    const __bf16* dbase = p.dout + (int64_t)a * rs + head_off;
    const float* nl_base = p.ws + (int64_t)h * T + a;
    const float* dl_base = p.ws + (int64_t)p.heads * T + (int64_t)h * T + a;
    auto issue = [&](int slot_i, int stage) {
      const int r0 = stage * kBwdStage;
      bwd_issue_tile<D, C::CPT, 0>(qbase, r0, L, rs, row_bytes, qring + slot_i * C::TILE_BYTES, src, wave);
      bwd_issue_tile<D, C::CPT, 0>(dbase, r0, L, rs, row_bytes, dring + slot_i * C::TILE_BYTES, src, wave);
      if (wave < 2) {   // 64 fp32 row values: wave 0 -LSE*log2e, wave 1 delta
        const int rows = (L - r0 < kBwdStage) ? (L - r0) : kBwdStage;
        const float* fb = (wave == 0 ? nl_base : dl_base) + r0;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)fb, 0, rows * 4, kRsrcFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void*)(fring + (slot_i * 2 + wave) * C::ROWF_BYTES), 4, lane * 4, 0, 0, 0);
      }
    };
    const int ns = (L + kBwdStage - 1) / kBwdStage;
    issue(0, 0);
    for (int s = 0; s < ns; ++s) {
      const int cur = s & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      if (s + 1 < ns) issue(cur ^ 1, s + 1);
      const char* qst = qring + cur * C::TILE_BYTES;
      const char* dst = dring + cur * C::TILE_BYTES;
      const float* nls = reinterpret_cast<const float*>(fring + (cur * 2) * C::ROWF_BYTES);
      const float* dls = reinterpret_cast<const float*>(fring + (cur * 2 + 1) * C::ROWF_BYTES);
#pragma unroll
      for (int j = 0; j < kBwdStage / 32; ++j) {
        const char* qj = qst + j * 32 * D * 2;
        const char* dj = dst + j * 32 * D * 2;
        f32x16 sc, dp;
        {
          bf16x8 qa[C::KSTEP], da[C::KSTEP];
          k_operands<D>(qj, koff, qa);
          k_operands<D>(dj, koff, da);
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
          for (int t = 0; t < C::KSTEP; ++t) {
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], kr[t], sc, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[t], vr[t], dp, 0, 0, 0);
          }
        }
        // element i holds query row j*32 + 8(i/4) + 4g + i%4 of this key column
        bf16x8 pp[2], dsp[2];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int r = j * 32 + 8 * a4 + 4 * g;
          const float4 nl = *reinterpret_cast<const float4*>(nls + r);
          const float4 dl = *reinterpret_cast<const float4*>(dls + r);
          const float nlv[4] = {nl.x, nl.y, nl.z, nl.w};
          const float dlv[4] = {dl.x, dl.y, dl.z, dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * a4 + e;
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[i], p.c, nlv[e]));
            const float dsv = pv * (dp[i] - dlv[e]);
            pp[i >> 3][i & 7] = (__bf16)pv;
            dsp[i >> 3][i & 7] = (__bf16)dsv;
          }
        }
        bf16x8 ta[2][C::DT];
        t_operands<D>(dj, toff, ta);                 // dO^T
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            dvt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[cc][dt], pp[cc], dvt[dt], 0, 0, 0);
        t_operands<D>(qj, toff, ta);                 // Q^T
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            dkt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[cc][dt], dsp[cc], dkt[dt], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave has left the ring
    char* const ok = qring + wave * (32 * D * 2);
    char* const ov = qring + (kBwdNW + wave) * (32 * D * 2);
    stage_rows<D>(dkt, p.scale, ok, n32, g);
    stage_rows<D>(dvt, 1.0f, ov, n32, g);
    __syncthreads();
    const int valid = L - k0;
    store_rows<D>(ok, lane, p.dk + (int64_t)(a + k0) * rs + head_off, rs, valid);
    store_rows<D>(ov, lane, p.dv + (int64_t)(a + k0) * rs + head_off, rs, valid);
    __syncthreads();   // the next item's first stage overwrites the ring
  }
}

// ---- dQ
template <int D>
__global__ void __launch_bounds__(kWave * kBwdNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
pfa_bwd_dq_kernel(BwdParams p) {
  using C = BwdTile<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* const kring = reinterpret_cast<char*>(smem);
  char* const vring = kring + kStages * C::TILE_BYTES;
  int* s_order = reinterpret_cast<int*>(vring + kStages * C::TILE_BYTES);
  int* s_prefix = s_order + kSortMax;
  int* s_len = reinterpret_cast<int*>(kring);

  const int T = p.cu[p.num_seqs];
  const bool sorted = p.num_seqs <= kSortMax;
  const int total = sorted ? build_schedule<kBwdRows, C::THREADS>(p.cu, p.cu, p.num_seqs, p.heads,
                                                                   s_len, s_order, s_prefix)
                           : p.num_seqs * p.heads * p.tiles_max;
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int slot = (G % 8 == 0) ? (bid & 7) * (G >> 3) + (bid >> 3) : bid;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  const int g = lane >> 5;
  const int64_t rs = (int64_t)p.heads * D;
  const int row_bytes = (int)(rs * 2);
  int koff[C::KSTEP];
#pragma unroll
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, true>(n32, 2 * t + g);
  int toff[2][2][C::DT];
  t_offsets<D>(lane, toff);
  int src[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) src[i] = logical_src<D, true>((wave * C::CPT + i) * 64 + lane, row_bytes);
  if (sorted) __syncthreads();   // s_len aliases the K ring

  for (int u = slot; u < total; u += G) {
    int a, L, h, qt;
    if (!bwd_item<kBwdRows>(p, u, sorted, s_order, s_prefix, T, a, L, h, qt)) continue;
    const int64_t head_off = (int64_t)h * D;
    const int q0 = qt * kBwdRows + wave * 32;
    const int row = q0 + n32;                        // this lane's query
    // stationary Q^T and dO^T fragments (B operands; lane n32 = query)
    bf16x8 qr[C::KSTEP], dr[C::KSTEP];
    {
      const __bf16* qp = p.q + (int64_t)(a + row) * rs + head_off;
      const __bf16* dp = p.dout + (int64_t)(a + row) * rs + head_off;
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (row < L) {
          x = *reinterpret_cast<const u32x4*>(qp + 16 * t + 8 * g);
          y = *reinterpret_cast<const u32x4*>(dp + 16 * t + 8 * g);
        }
        qr[t] = __builtin_bit_cast(bf16x8, x);
        dr[t] = __builtin_bit_cast(bf16x8, y);
      }
    }
    const float nl = row < L ? p.ws[(int64_t)h * T + a + row] : 0.f;
    const float dl = row < L ? p.ws[(int64_t)p.heads * T + (int64_t)h * T + a + row] : 0.f;
    f32x16 dqt[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqt[dt][i] = 0.f;

    const __bf16* kbase = p.k + (int64_t)a * rs + head_off;
    const __bf16* vbase = p.v + (int64_t)a * rs + head_off;
    const int ns = (L + kBwdStage - 1) / kBwdStage;
    bwd_issue_tile<D, C::CPT, 1>(kbase, 0, L, rs, row_bytes, kring, src, wave);
    bwd_issue_tile<D, C::CPT, 1>(vbase, 0, L, rs, row_bytes, vring, src, wave);
    for (int s = 0; s < ns; ++s) {
      const int cur = s & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      if (s + 1 < ns) {
        bwd_issue_tile<D, C::CPT, 1>(kbase, (s + 1) * kBwdStage, L, rs, row_bytes, kring + (cur ^ 1) * C::TILE_BYTES, src, wave);
        bwd_issue_tile<D, C::CPT, 1>(vbase, (s + 1) * kBwdStage, L, rs, row_bytes, vring + (cur ^ 1) * C::TILE_BYTES, src, wave);
      }
      const char* kst = kring + cur * C::TILE_BYTES;
      const char* vst = vring + cur * C::TILE_BYTES;
#pragma unroll
      for (int j = 0; j < kBwdStage / 32; ++j) {
        const char* kj = kst + j * 32 * D * 2;
        const char* vj = vst + j * 32 * D * 2;
        f32x16 sc, dp;
        {
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
          {
            bf16x8 ka[C::KSTEP];
            k_operands<D>(kj, koff, ka);
#pragma unroll
            for (int t = 0; t < C::KSTEP; ++t)
              sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t], qr[t], sc, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);   // one operand set live at a time
          {
            bf16x8 va[C::KSTEP];
            k_operands<D>(vj, koff, va);
#pragma unroll
            for (int t = 0; t < C::KSTEP; ++t)
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t], dr[t], dp, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // element i holds key s*64 + j*32 + 8(i/4) + 4g + i%4 for this lane's query
        const int key0 = s * kBwdStage + j * 32;
        bf16x8 dsp[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + (i >> 2) * 8 + 4 * g + (i & 3);
          const float pv = key < L ? __builtin_amdgcn_exp2f(fmaf(sc[i], p.c, nl)) : 0.f;
          dsp[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - dl));
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {             // K^T, one 16-key half at a time
          bf16x8 ta[C::DT];
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(kj + toff[cc][0][dt]));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(kj + toff[cc][1][dt]));
            ta[dt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
            dqt[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[dt], dsp[cc], dqt[dt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __syncthreads();   // every wave has left the ring
    char* const oq = kring + wave * (32 * D * 2);
    stage_rows<D>(dqt, p.scale, oq, n32, g);
    __syncthreads();
    store_rows<D>(oq, lane, p.dq + (int64_t)(a + q0) * rs + head_off, rs, L - q0);
    __syncthreads();   // the next item's first stage overwrites the ring
  }
}

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
constexpr int kQuantTokens = 64;   // tokens per thread in the maxima pass

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

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_amax_kernel(QuantParams q) {
  const int64_t T = q.cu[q.num_seqs];
  const int cpt = q.heads * q.d / 8;                      // 16-byte chunks per token
  const int64_t items = (T > 0 ? (T + kQuantTokens - 1) / kQuantTokens : 0) * cpt;
  for (int64_t it = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kQuantThreads) {
    const int64_t t0 = it / cpt * kQuantTokens;
    const int j = (int)(it % cpt);
    const int64_t t1 = t0 + kQuantTokens < T ? t0 + kQuantTokens : T;
    int seg = segment_of(q.cu, q.num_seqs, t0);
    int64_t seg_end = q.cu[seg + 1];
    float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto flush = [&]() {
      uint32_t* dst = reinterpret_cast<uint32_t*>(q.v_scale) + ((int64_t)seg * q.heads) * q.d + 8 * j;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (mx[e] > 0.f) atomicMax(dst + e, __float_as_uint(mx[e]));
    };
    for (int64_t t = t0; t < t1; ++t) {
      if (t >= seg_end) {
        flush();
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[e] = 0.f;
        while (q.cu[seg + 1] <= t) ++seg;
        seg_end = q.cu[seg + 1];
      }
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(q.v + t * cpt * 8 + 8 * j);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[e] = fmaxf(mx[e], fabsf((float)x[e]));
    }
    flush();
  }
}

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_codes_kernel(QuantParams q) {
  const int64_t T = q.cu[q.num_seqs];
  const int cpt = q.heads * q.d / 8;
  const int64_t items = (T > 0 ? T : 0) * cpt;
  for (int64_t it = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kQuantThreads) {
    const int64_t t = it / cpt;
    const int j = (int)(it % cpt);
    const int seg = segment_of(q.cu, q.num_seqs, t);
    const uint32_t* am = reinterpret_cast<const uint32_t*>(q.v_scale) + ((int64_t)seg * q.heads) * q.d + 8 * j;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(q.v + t * cpt * 8 + 8 * j);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf((float)x[e], -v8_exponent(__uint_as_float(am[e])));
    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    *reinterpret_cast<u32x2*>(q.v8 + t * cpt * 8 + 8 * j) = u32x2{(uint32_t)lo, (uint32_t)hi};
  }
}

__global__ void __launch_bounds__(kQuantThreads) pfa_v8_scale_kernel(QuantParams q) {
  const int64_t n = (int64_t)q.num_seqs * q.heads * q.d;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kQuantThreads)
    q.v_scale[i] = __builtin_ldexpf(1.0f, v8_exponent(q.v_scale[i]));
}

// ---------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------
struct Variant {
  const void* fn;
  int bm;
  int threads;
  size_t lds;
};

template <int D, int QB, int NW, int SK, int WPE, int MODE>
Variant make_variant() {
  using C = Tile<D, QB, NW, SK>;
  static_assert(!mode_sparse(MODE) || (C::BM == PFA_SPARSE_BLOCK_Q && SK == PFA_SPARSE_BLOCK_K),
                "the block-sparse layout's blocks are the kernel's query tile and key stage");
  return Variant{reinterpret_cast<const void*>(&pfa_fwd_kernel<D, QB, NW, SK, WPE, MODE>), C::BM,
                 C::THREADS, C::LDS_BYTES + (mode_sparse(MODE) ? kSparseLdsBytes : 0)};
}

constexpr int kMaxDevices = 64;
constexpr int kVariants = 12;  // head_dim 64, 128 x the six kernel modes
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_occ[kMaxDevices][kVariants];
std::atomic<int> g_bwd_occ[kMaxDevices][2][2];   // [device][head_dim 64 / 128][dK-dV / dQ]

int variant_index(int head_dim, int mode) { return (head_dim == 64 ? 0 : 1) + 2 * mode; }

#ifndef PFA_D64_QB
#define PFA_D64_QB 2
#endif
#ifndef PFA_D64_WPE
#define PFA_D64_WPE 2
#endif
#ifndef PFA_D128_QB
#define PFA_D128_QB 1
#endif
#ifndef PFA_D128_WPE
#define PFA_D128_WPE 2
#endif
#ifndef PFA_D64_NW
#define PFA_D64_NW 4
#endif
#ifndef PFA_D128_NW
#define PFA_D128_NW 8
#endif
#ifndef PFA_D64_SK
#define PFA_D64_SK 64
#endif
#ifndef PFA_D128_SK
#define PFA_D128_SK 64
#endif

template <int MODE>
Variant variant_of(int head_dim) {
  if (head_dim == 64) return make_variant<64, PFA_D64_QB, PFA_D64_NW, PFA_D64_SK, PFA_D64_WPE, MODE>();
  return make_variant<128, PFA_D128_QB, PFA_D128_NW, PFA_D128_SK, PFA_D128_WPE, MODE>();
}

Variant variant_for(int head_dim, int mode) {
  return mode == kModeCross  ? variant_of<kModeCross>(head_dim)
       : mode == kModeQkv    ? variant_of<kModeQkv>(head_dim)
       : mode == kModeSparse ? variant_of<kModeSparse>(head_dim)
       : mode == kModeFp8    ? variant_of<kModeFp8>(head_dim)
       : mode == kModeSparseFp8 ? variant_of<kModeSparseFp8>(head_dim)
                             : variant_of<kModeSelf>(head_dim);
}

// compute units of the current device (cached; a race only recomputes the same value)
int device_cus(int* dev_out, int* cus_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PFA_ERR_DEVICE;
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return PFA_ERR_DEVICE;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  *dev_out = dev;
  *cus_out = cus;
  return PFA_OK;
}

// Size the persistent grid of one forward variant and launch it.  prm carries every
// field but qt_max; the caller has checked the arguments.
int launch_fwd(Params prm, int mode, int max_seqlen_q, int head_dim, hipStream_t stream) {
  const Variant var = variant_for(head_dim, mode);
  const int64_t qt_max = ((int64_t)max_seqlen_q + var.bm - 1) / var.bm;
  const int64_t slots = (int64_t)prm.num_seqs * prm.heads * qt_max;
  if (slots > INT32_MAX) return PFA_ERR_SIZE;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != PFA_OK) return rc;
  const int vi = variant_index(head_dim, mode);
  int occ = g_occ[dev][vi].load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (hipFuncSetAttribute(var.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)var.lds) != hipSuccess)
      return PFA_ERR_DEVICE;
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, var.fn, var.threads, var.lds) != hipSuccess || o <= 0)
      return PFA_ERR_DEVICE;
    occ = o;
    g_occ[dev][vi].store(occ, std::memory_order_relaxed);
  }
  int64_t grid = (int64_t)cus * occ;
  if (grid > slots) grid = slots;
  if (grid >= 8) grid -= grid % 8;   // keep whole rounds on every XCD
  prm.qt_max = (int)qt_max;
  void* args[] = {&prm};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)grid), dim3(var.threads), args, var.lds, stream);
  return err == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

bool misaligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }

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
    case PFA_ERR_ALIGN: return "a buffer is not 16-byte aligned";
    case PFA_ERR_LAYOUT: return "block-sparse layout is malformed (layout_heads, nnz, row pointers or block indices)";
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

PFA_API int pfa_varlen_fwd_qk(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int num_seqs, int max_seqlen_q,
                              int max_seqlen_k, int heads, int head_dim, float scale, void* out,
                              float* lse, hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens_q == nullptr ||
      cu_seqlens_k == nullptr || out == nullptr)
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen_q < 1 || max_seqlen_k < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  for (const void* in : ins)
    if (in == out || (lse != nullptr && in == static_cast<const void*>(lse))) return PFA_ERR_ALIAS;
  if (lse != nullptr && static_cast<const void*>(lse) == out) return PFA_ERR_ALIAS;
  if ((int64_t)heads * head_dim > kMaxRowElems) return PFA_ERR_SIZE;

  Params prm{};
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.cu_q = cu_seqlens_q;
  prm.cu_k = cu_seqlens_k;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.c = scale * kLog2e;
  const int mode = cu_seqlens_k != cu_seqlens_q ? kModeCross : kModeSelf;
  return launch_fwd(prm, mode, max_seqlen_q, head_dim, stream);
}

PFA_API int pfa_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* out, float* lse, hipStream_t stream) {
  return pfa_varlen_fwd_qk(q, k, v, cu_seqlens, cu_seqlens, num_seqs, max_seqlen, max_seqlen, heads,
                           head_dim, scale, out, lse, stream);
}

PFA_API int pfa_varlen_fwd_qkv(const void* qkv, const float* rope_cos, const float* rope_sin,
                               const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int heads,
                               int head_dim, float scale, void* out, float* lse, void* k_rot,
                               hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (qkv == nullptr || cu_seqlens == nullptr || out == nullptr) return PFA_ERR_NULL;
  const bool rope = rope_cos != nullptr || rope_sin != nullptr;
  if (rope && (rope_cos == nullptr || rope_sin == nullptr || k_rot == nullptr)) return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[4] = {qkv, cu_seqlens, rope_cos, rope_sin};
  const void* outs[3] = {out, lse, rope ? k_rot : nullptr};
  for (int a = 0; a < 3; ++a) {
    if (outs[a] == nullptr) continue;
    for (const void* in : ins)
      if (in == outs[a]) return PFA_ERR_ALIAS;
    for (int b = a + 1; b < 3; ++b)
      if (outs[a] == outs[b]) return PFA_ERR_ALIAS;
  }
  if (misaligned16(qkv) || misaligned16(out) ||
      (rope && (misaligned16(k_rot) || misaligned16(rope_cos) || misaligned16(rope_sin))))
    return PFA_ERR_ALIGN;
  const int64_t hd = (int64_t)heads * head_dim;
  if (3 * hd > kMaxRowElems) return PFA_ERR_SIZE;
  const int bm = variant_for(head_dim, kModeQkv).bm;   // launch_fwd repeats this check
  if ((int64_t)num_seqs * heads * (((int64_t)max_seqlen + bm - 1) / bm) > INT32_MAX) return PFA_ERR_SIZE;

  const __bf16* base = static_cast<const __bf16*>(qkv);
  Params prm{};
  prm.q = base;
  prm.k = rope ? static_cast<const __bf16*>(k_rot) : base + hd;
  prm.v = base + 2 * hd;
  prm.cu_q = cu_seqlens;
  prm.cu_k = cu_seqlens;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.c = scale * kLog2e;
  prm.sq = (int)(3 * hd);
  prm.sk = (int)(rope ? hd : 3 * hd);
  prm.sv = (int)(3 * hd);
  prm.rope_cos = rope_cos;
  prm.rope_sin = rope_sin;
  if (rope) {
    int dev = 0, cus = 0;
    const int rc = device_cus(&dev, &cus);
    if (rc != PFA_OK) return rc;
    RopeParams rp;
    rp.src = base + hd;
    rp.dst = static_cast<__bf16*>(k_rot);
    rp.cos = rope_cos;
    rp.sin = rope_sin;
    rp.cu = cu_seqlens;
    rp.num_seqs = num_seqs;
    rp.heads = heads;
    rp.stride = (int)(3 * hd);
    void* args[] = {&rp};
    const void* fn = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_rope_k_kernel<64>)
                                    : reinterpret_cast<const void*>(&pfa_rope_k_kernel<128>);
    if (hipLaunchKernel(fn, dim3((unsigned)cus * 8), dim3(kRopeThreads), args, 0, stream) != hipSuccess)
      return PFA_ERR_LAUNCH;
  }
  return launch_fwd(prm, kModeQkv, max_seqlen, head_dim, stream);
}

PFA_API int pfa_varlen_fwd_blocksparse(const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                       int heads, int head_dim, float scale, const int32_t* kv_ptr,
                                       const int32_t* kv_idx, int nnz, int layout_heads, void* out,
                                       float* lse, hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v == nullptr || cu_seqlens == nullptr || out == nullptr ||
      kv_ptr == nullptr || (kv_idx == nullptr && nnz > 0))
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  if (nnz < 0 || (layout_heads != 1 && layout_heads != heads)) return PFA_ERR_LAYOUT;
  const void* ins[6] = {q, k, v, cu_seqlens, kv_ptr, kv_idx};
  for (const void* in : ins)
    if (in != nullptr && (in == out || (lse != nullptr && in == static_cast<const void*>(lse))))
      return PFA_ERR_ALIAS;
  if (lse != nullptr && static_cast<const void*>(lse) == out) return PFA_ERR_ALIAS;
  if ((int64_t)heads * head_dim > kMaxRowElems) return PFA_ERR_SIZE;
  if ((int64_t)max_seqlen > (int64_t)kSparseMaxBlocks * PFA_SPARSE_BLOCK_K) return PFA_ERR_SIZE;
  const int64_t qt_max = ((int64_t)max_seqlen + PFA_SPARSE_BLOCK_Q - 1) / PFA_SPARSE_BLOCK_Q;
  if ((int64_t)num_seqs * heads * qt_max > INT32_MAX) return PFA_ERR_SIZE;

  Params prm{};
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(v);
  prm.cu_q = cu_seqlens;
  prm.cu_k = cu_seqlens;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.c = scale * kLog2e;
  prm.kv_ptr = kv_ptr;
  prm.kv_idx = kv_idx;
  prm.nnz = nnz;
  prm.layout_heads = layout_heads;
  return launch_fwd(prm, kModeSparse, max_seqlen, head_dim, stream);
}

PFA_API int pfa_check_block_layout(const int32_t* cu_host, int num_seqs, int max_seqlen, int heads,
                                   int layout_heads, const int32_t* kv_ptr_host,
                                   const int32_t* kv_idx_host, int nnz) {
  int64_t total = 0;
  const int rc = pfa_check_cu_seqlens(cu_host, num_seqs, max_seqlen, &total);
  if (rc != PFA_OK) return rc;
  if (kv_ptr_host == nullptr || (kv_idx_host == nullptr && nnz > 0)) return PFA_ERR_NULL;
  if (heads < 1) return PFA_ERR_HEADS;
  if (nnz < 0 || (layout_heads != 1 && layout_heads != heads)) return PFA_ERR_LAYOUT;
  if ((int64_t)max_seqlen > (int64_t)kSparseMaxBlocks * PFA_SPARSE_BLOCK_K) return PFA_ERR_SIZE;
  const int64_t qt_max = ((int64_t)max_seqlen + PFA_SPARSE_BLOCK_Q - 1) / PFA_SPARSE_BLOCK_Q;
  const int64_t rows = (int64_t)num_seqs * layout_heads * qt_max;
  if (rows > INT32_MAX) return PFA_ERR_SIZE;
  if (kv_ptr_host[0] != 0 || kv_ptr_host[rows] != nnz) return PFA_ERR_LAYOUT;
  std::vector<int> seen((size_t)kSparseMaxBlocks, -1);   // row that last listed each block
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t e0 = kv_ptr_host[r], e1 = kv_ptr_host[r + 1];
    if (e1 < e0 || e1 > nnz) return PFA_ERR_LAYOUT;
    const int64_t qt = r % qt_max;
    const int s = (int)(r / qt_max / layout_heads);
    const int64_t L = (int64_t)cu_host[s + 1] - cu_host[s];
    const int64_t tiles = (L + PFA_SPARSE_BLOCK_Q - 1) / PFA_SPARSE_BLOCK_Q;
    const int64_t nkb = (L + PFA_SPARSE_BLOCK_K - 1) / PFA_SPARSE_BLOCK_K;
    if (qt >= tiles) {                 // no such query tile: the row must be empty
      if (e1 != e0) return PFA_ERR_LAYOUT;
      continue;
    }
    if (e1 == e0) return PFA_ERR_LAYOUT;   // a query block with no keys has no softmax
    for (int64_t e = e0; e < e1; ++e) {
      const int b = kv_idx_host[e];
      if (b < 0 || b >= nkb || seen[(size_t)b] == (int)r) return PFA_ERR_LAYOUT;
      seen[(size_t)b] = (int)r;
    }
  }
  return PFA_OK;
}

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
  if (misaligned16(v) || (reinterpret_cast<uintptr_t>(v8) & 7) != 0 || (reinterpret_cast<uintptr_t>(v_scale) & 3) != 0)
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
  const unsigned grids[4] = {(unsigned)cus, (unsigned)cus * 8, (unsigned)cus * 8, (unsigned)cus};
  for (int i = 0; i < 4; ++i)
    if (hipLaunchKernel(fns[i], dim3(grids[i]), dim3(kQuantThreads), args, 0, stream) != hipSuccess)
      return PFA_ERR_LAUNCH;
  return PFA_OK;
}

PFA_API int pfa_varlen_fwd_fp8pv(const void* q, const void* k, const void* v8, const float* v_scale,
                                 const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int heads,
                                 int head_dim, float scale, void* out, float* lse, hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v8 == nullptr || v_scale == nullptr || cu_seqlens == nullptr ||
      out == nullptr)
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[5] = {q, k, v8, v_scale, cu_seqlens};
  for (const void* in : ins)
    if (in == out || (lse != nullptr && in == static_cast<const void*>(lse))) return PFA_ERR_ALIAS;
  if (lse != nullptr && static_cast<const void*>(lse) == out) return PFA_ERR_ALIAS;
  if (misaligned16(v8) || misaligned16(v_scale)) return PFA_ERR_ALIGN;
  if ((int64_t)heads * head_dim > kMaxRowElems) return PFA_ERR_SIZE;

  Params prm{};
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(k);   // unused by this mode
  prm.cu_q = cu_seqlens;
  prm.cu_k = cu_seqlens;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.c = scale * kLog2e;
  prm.v8 = static_cast<const uint8_t*>(v8);
  prm.v_scale = v_scale;
  return launch_fwd(prm, kModeFp8, max_seqlen, head_dim, stream);
}

PFA_API int pfa_varlen_fwd_blocksparse_fp8pv(const void* q, const void* k, const void* v8,
                                             const float* v_scale, const int32_t* cu_seqlens,
                                             int num_seqs, int max_seqlen, int heads, int head_dim,
                                             float scale, const int32_t* kv_ptr, const int32_t* kv_idx,
                                             int nnz, int layout_heads, void* out, float* lse,
                                             hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v8 == nullptr || v_scale == nullptr || cu_seqlens == nullptr ||
      out == nullptr || kv_ptr == nullptr || (kv_idx == nullptr && nnz > 0))
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  if (nnz < 0 || (layout_heads != 1 && layout_heads != heads)) return PFA_ERR_LAYOUT;
  const void* ins[7] = {q, k, v8, v_scale, cu_seqlens, kv_ptr, kv_idx};
  for (const void* in : ins)
    if (in != nullptr && (in == out || (lse != nullptr && in == static_cast<const void*>(lse))))
      return PFA_ERR_ALIAS;
  if (lse != nullptr && static_cast<const void*>(lse) == out) return PFA_ERR_ALIAS;
  if (misaligned16(v8) || misaligned16(v_scale)) return PFA_ERR_ALIGN;
  if ((int64_t)heads * head_dim > kMaxRowElems) return PFA_ERR_SIZE;
  if ((int64_t)max_seqlen > (int64_t)kSparseMaxBlocks * PFA_SPARSE_BLOCK_K) return PFA_ERR_SIZE;

  Params prm{};
  prm.q = static_cast<const __bf16*>(q);
  prm.k = static_cast<const __bf16*>(k);
  prm.v = static_cast<const __bf16*>(k);   // unused by this mode
  prm.cu_q = cu_seqlens;
  prm.cu_k = cu_seqlens;
  prm.out = static_cast<__bf16*>(out);
  prm.lse = lse;
  prm.num_seqs = num_seqs;
  prm.heads = heads;
  prm.c = scale * kLog2e;
  prm.kv_ptr = kv_ptr;
  prm.kv_idx = kv_idx;
  prm.nnz = nnz;
  prm.layout_heads = layout_heads;
  prm.v8 = static_cast<const uint8_t*>(v8);
  prm.v_scale = v_scale;
  return launch_fwd(prm, kModeSparseFp8, max_seqlen, head_dim, stream);
}

PFA_API int pfa_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* dq, void* dk, void* dv, float* workspace, hipStream_t stream) {
  // ---- argument checks: all before any HIP runtime call
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || cu_seqlens == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
      workspace == nullptr)
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[7] = {q, k, v, out, dout, lse, cu_seqlens};
  const void* outs[4] = {dq, dk, dv, workspace};
  for (int a = 0; a < 4; ++a) {
    for (const void* in : ins)
      if (in == outs[a]) return PFA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (outs[a] == outs[b]) return PFA_ERR_ALIAS;
  }
  const int64_t tiles_max = ((int64_t)max_seqlen + kBwdRows - 1) / kBwdRows;
  const int64_t slots = (int64_t)num_seqs * heads * tiles_max;
  if ((int64_t)heads * head_dim > kMaxRowElems || slots > INT32_MAX) return PFA_ERR_SIZE;

  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != PFA_OK) return rc;
  const void* prep = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_bwd_prep_kernel<64>)
                                    : reinterpret_cast<const void*>(&pfa_bwd_prep_kernel<128>);
  const void* dkdv = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_bwd_dkdv_kernel<64>)
                                    : reinterpret_cast<const void*>(&pfa_bwd_dkdv_kernel<128>);
  const void* dqk = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_bwd_dq_kernel<64>)
                                   : reinterpret_cast<const void*>(&pfa_bwd_dq_kernel<128>);
  const size_t lds_dkdv = head_dim == 64 ? BwdTile<64>::LDS_DKDV : BwdTile<128>::LDS_DKDV;
  const size_t lds_dq = head_dim == 64 ? BwdTile<64>::LDS_DQ : BwdTile<128>::LDS_DQ;
  const int threads = kWave * kBwdNW;
  const int vi = head_dim == 64 ? 0 : 1;
  int occ_kv = g_bwd_occ[dev][vi][0].load(std::memory_order_relaxed);
  int occ_q = g_bwd_occ[dev][vi][1].load(std::memory_order_relaxed);
  if (occ_kv <= 0 || occ_q <= 0) {
    if (hipFuncSetAttribute(dkdv, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dkdv) != hipSuccess ||
        hipFuncSetAttribute(dqk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dq) != hipSuccess)
      return PFA_ERR_DEVICE;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_kv, dkdv, threads, lds_dkdv) != hipSuccess ||
        occ_kv <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_q, dqk, threads, lds_dq) != hipSuccess || occ_q <= 0)
      return PFA_ERR_DEVICE;
    g_bwd_occ[dev][vi][0].store(occ_kv, std::memory_order_relaxed);
    g_bwd_occ[dev][vi][1].store(occ_q, std::memory_order_relaxed);
  }
  auto grid_for = [&](int occ) {
    int64_t grid = (int64_t)cus * occ;
    if (grid > slots) grid = slots;
    if (grid >= 8) grid -= grid % 8;
    return (unsigned)grid;
  };

  BwdParams bp;
  bp.q = static_cast<const __bf16*>(q);
  bp.k = static_cast<const __bf16*>(k);
  bp.v = static_cast<const __bf16*>(v);
  bp.out = static_cast<const __bf16*>(out);
  bp.dout = static_cast<const __bf16*>(dout);
  bp.lse = lse;
  bp.ws = workspace;
  bp.cu = cu_seqlens;
  bp.dq = static_cast<__bf16*>(dq);
  bp.dk = static_cast<__bf16*>(dk);
  bp.dv = static_cast<__bf16*>(dv);
  bp.num_seqs = num_seqs;
  bp.heads = heads;
  bp.tiles_max = (int)tiles_max;
  bp.c = scale * kLog2e;
  bp.scale = scale;
  void* args[] = {&bp};
  if (hipLaunchKernel(prep, dim3((unsigned)cus * 8), dim3(256), args, 0, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  if (hipLaunchKernel(dkdv, dim3(grid_for(occ_kv)), dim3(threads), args, lds_dkdv, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  if (hipLaunchKernel(dqk, dim3(grid_for(occ_q)), dim3(threads), args, lds_dq, stream) != hipSuccess)
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
