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
// d = 64: 4 wave64s, or 8 for query segments of 512 rows or more):
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
//   * one kernel template, six modes fixed at compile time: one segment table; separate
//     query and key tables; q, k, v read through row strides from a fused projection
//     output (q rotated on load); listed key blocks only; P.V in FP8; listed key blocks
//     with P.V in FP8.  The modes share the tile routine and differ only where noted.
#include <vector>

#include "pfa_common.h"

namespace {

// How far (base 2) a block max may exceed the running max before O and l are rescaled.
// 0 keeps the reference equal to the exact running max, so the largest weight of a row is
// exactly 1 and carries no bf16 rounding; a positive slack saves rescales (about 5% on
// 4096-token segments) but leaves that weight rounded, which on sharp softmax rows pushes
// the worst output error past 1e-2 of the exact result.
constexpr float kRescaleSlack = 0.0f;

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
  int sort_cap;    // schedule capacity held in LDS (tables up to it are sorted)
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
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Block-sparse variant: a compacted copy of the tile's key-block list lives in LDS after
// the schedule (count in the last slot), so segments are limited to this many key blocks.
constexpr int kSparseMaxBlocks = 1024;
constexpr int kSparseLdsBytes = (kSparseMaxBlocks + 4) * 4;

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
  // the K/V ring, which the epilogue reuses to stage each wave's output block
  static constexpr int RING_BYTES = (kStages * 2 * TILE_BYTES > NW * QB * 32 * D * 2)
                                        ? kStages * 2 * TILE_BYTES : NW * QB * 32 * D * 2;
  static constexpr size_t LDS_BYTES = (size_t)RING_BYTES + sizeof(int) * SCHED_INTS;
  static_assert(CPT * THREADS == SK * CPR, "stage must split evenly");
  static_assert(SK % kHalf == 0, "stages hold whole 64-key halves");
  static_assert(sizeof(int) * kSortMax <= (size_t)kStages * TILE_BYTES, "len scratch fits");
};

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
  float l_run[QB];               // row sum of the fp32 weights (gives the LSE; normalises FP8 O)
  float l_rnd[QB];               // row sum of the bf16 weights (normalises bf16 O)
};

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

#ifndef PFA_QK_AHEAD_64
#define PFA_QK_AHEAD_64 0
#endif
#ifndef PFA_QK_AHEAD_128
#define PFA_QK_AHEAD_128 4
#endif

// Order of the QK phase of a stage: the two K operand reads of each 16-deep step (one per
// 32-key sub-block) are issued `ahead` steps before the 2 QB MFMAs that consume them; left
// to itself the compiler waits on each pair right before its MFMAs.
template <int D, int QB>
__device__ __forceinline__ void qk_schedule() {
  constexpr int ahead = D == 128 ? PFA_QK_AHEAD_128 : PFA_QK_AHEAD_64;
  static_assert(ahead >= 0 && ahead < D / 16, "prefetch distance within the contraction");
  if constexpr (ahead > 0) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * ahead, 0);
#pragma unroll
    for (int t = 0; t < D / 16 - ahead; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB * ahead, 0);
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
      st.l_rnd[b] *= a;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][dt][i] *= a;
    }
  }
}

// Online softmax, second half (straight-line): P = 2^(s*c - m) as bf16 B operands and two
// row sums.  l_run adds the fp32 weights and gives the LSE (a sum of bf16-rounded weights
// can carry up to 2^-8 relative error, 3.9e-3, into the LSE of a sharp row).  l_rnd adds
// the bf16 weights the PV product actually uses and normalises O: each weight's rounding
// then enters numerator and denominator alike, so the error is sum_j dp_j (v_j - O) / l
// rather than sum_j dp_j v_j / l.  That matters on rows with few keys and large, similar
// values (|O| in [2, 4), where bf16 rounding of O already takes 2^-7 of the 1e-2 bar);
// normalising by l_run there was measured past the bar.  Both sums chain straight into
// their running values (one add, resp. one bf16 dot of a weight pair, per step).
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
      st.l_rnd[b] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, st.l_rnd[b], false);
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
  qk_schedule<D, QB>();
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
    qk_schedule<D, QB>();
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
    st.l_rnd[b] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[b][dt][i] = 0.f;
  }

  // ---- per-lane LDS offsets (fixed for the whole tile)
  int koff[C::KSTEP], voff[C::DT];
#pragma unroll
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, Swz::K>(n32, 2 * t + g);
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
      voff[dt] = phys_off<D, Swz::V>(4 * g + (i16 >> 2), 4 * dt + 2 * hh + ((i16 & 3) >> 1)) + 8 * (i16 & 1);
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
    src_k[i] = logical_src<D, Swz::K>(P, kbytes);
    if constexpr (mode_fp8(MODE)) {
      if (i < C::CPT8) src_v[i] = logical_src8<D>((wave * C::CPT8 + i) * 64 + lane, (int)rs);
    } else {
      src_v[i] = logical_src<D, Swz::V>(P, vbytes);
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

  // ---- epilogue: O = acc / l_rnd (FP8: acc / l_run) in bf16 (round to nearest even),
  // LSE = ln2 * (m + log2 l_run).  O goes out through LDS: each wave writes its (QB*32) x D block into the free
  // ring in the swizzled K layout, then reads it back as whole 16-byte chunks of
  // consecutive rows, so 16 lanes store 256 contiguous bytes instead of every store
  // instruction touching 16-byte pieces of 32 different rows.
  static_assert(NW * QB * 32 * D * 2 <= C::RING_BYTES, "O staging fits the ring");
  char* const ost = kring + wave * (QB * 32 * D * 2);
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lt = partner_sum(st.l_run[b]);
    const float lr = mode_fp8(MODE) ? lt : partner_sum(st.l_rnd[b]);
    const float inv = lr > 0.f ? 1.0f / lr : 0.f;   // no keys: O = 0 (and LSE = -inf)
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
        *reinterpret_cast<bf16x4*>(ost + phys_off<D, Swz::K>(r, 4 * dt + ii) + 8 * g) = w;
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
    const u32x4 x = *reinterpret_cast<const u32x4*>(ost + phys_off<D, Swz::K>(r, ch));
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
  int* s_order = reinterpret_cast<int*>(smem + C::RING_BYTES);
  int* s_prefix = s_order + p.sort_cap;
  int* s_blk = s_order + 2 * p.sort_cap + 8;   // block-sparse variant only (its LDS is larger)
  int* s_len = reinterpret_cast<int*>(ks);     // scratch, dead before the first K tile lands

  const int Tq = ld_table(p.cu_q, p.num_seqs);
  const int Tk = ld_table(cu_k, p.num_seqs);
  const bool sorted = p.num_seqs <= p.sort_cap;
  int total;
  if (sorted) {
    total = build_schedule<C::BM, C::THREADS>(p.cu_q, cu_k, p.num_seqs, p.heads, s_len, s_order,
                                              s_prefix, p.sort_cap);
  } else {
    total = p.num_seqs * p.heads * p.qt_max;
  }

  // Items of a segment: head-major, so consecutive items (one XCD's run in a round) share
  // a (segment, head) and its K/V.  Block-sparse lists differ from tile to tile (a band
  // lists fewer key blocks at a segment's edges), and with head-major order a workgroup
  // would meet the same tile index in every round whenever the tiles per segment divide
  // the grid; there the items are tile-major (heads fastest) instead.
  constexpr bool kTileMajor = mode_sparse(MODE);
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
        if (__builtin_amdgcn_readfirstlane(s_prefix[mid]) <= u) lo = mid; else hi = mid - 1;
      }
      s = __builtin_amdgcn_readfirstlane(s_order[lo]);
      const int ntiles = (ld_table(p.cu_q, s + 1) - ld_table(p.cu_q, s) + C::BM - 1) / C::BM;
      const int local = u - __builtin_amdgcn_readfirstlane(s_prefix[lo]);
      if constexpr (kTileMajor) {
        qt = local / p.heads;
        h = local - qt * p.heads;
      } else {
        h = local / ntiles;
        qt = local - h * ntiles;
      }
    } else {
      const int per_seg = p.heads * p.qt_max;
      s = u / per_seg;
      const int rem = u - s * per_seg;
      if constexpr (kTileMajor) {
        qt = rem / p.heads;
        h = rem - qt * p.heads;
      } else {
        h = rem / p.qt_max;
        qt = rem - h * p.qt_max;
      }
    }
    const int qa = ld_table(p.cu_q, s);
    int Lq = ld_table(p.cu_q, s + 1) - qa;
    // never touch rows outside [0, Tq) / [0, Tk), whatever the tables say
    if (qa < 0 || qa >= Tq) continue;
    if (Lq > Tq - qa) Lq = Tq - qa;
    if (Lq <= 0 || qt * C::BM >= Lq) continue;
    int ka = qa, Lk = Lq;
    if (MODE == kModeCross) {
      ka = ld_table(cu_k, s);
      Lk = ld_table(cu_k, s + 1) - ka;
      if (ka < 0 || ka > Tk) ka = Tk;
      if (Lk > Tk - ka) Lk = Tk - ka;
      if (Lk < 0) Lk = 0;
    }
    process_tile<D, QB, NW, SK, MODE>(p, ks, vs, s_blk, s, qa, Lq, ka, Lk, h, qt, Tq);
  }
}

// ---------------------------------------------------------------------------------
// Cross-attention over short key segments, with each key segment's K and V resident in
// LDS for all of its query tiles.
//
// The xxmr.cn editing-network article (section 4.1) describes cross-attention whose keys
// and values come from a condition or edit sequence much shorter than the image-token
// query sequence.  With a key segment of a few hundred tokens, the streaming kernel above
// reloads all of it for every 256-query tile and spends most of each tile starting up.
// Here a workgroup takes a contiguous run of the longest-first item list, loads the key
// segment's K and V once per (segment, head) it meets, keeps them in LDS, and streams
// only Q in and O out: no stage loads and no stage barriers inside a tile.  The stage
// routine is the streaming kernel's own.
// ---------------------------------------------------------------------------------
// Longest key segment held in LDS: K and V of 256 keys at d = 128 (128 KiB) or 128 keys
// at d = 64 (32 KiB, so two workgroups still share a CU).
template <int D>
constexpr int resident_keys() { return D == 128 ? 256 : 128; }

template <int D, int QB, int NW>
struct ResidentTile {
  using C = Tile<D, QB, NW, 64>;
  static constexpr int KMAX = resident_keys<D>();
  static constexpr int NSMAX = KMAX / 64;                 // resident 64-key stages
  static constexpr int KV_BYTES = KMAX * D * 2;           // K area; the V area follows
  static constexpr int OUT_ROWS = QB * 32;                // one wave's query rows
  static constexpr int STAGE_OUT = NW * OUT_ROWS * 64;    // output staging: 32 channels a time
  static constexpr int CU_INTS = 2 * (kSortMax + 1);       // cu_seqlens_q and _k, sorted mode
  // vector-memory instructions of one tile's epilogue: the output stores, then one LSE
  // store per query block (all issued, rows past the segment end dropped by the buffer
  // bounds)
  static constexpr int EPI_STORES = C::DT * (OUT_ROWS * 4 / kWave) + QB;
  static constexpr size_t LDS_BYTES =
      (size_t)2 * KV_BYTES + STAGE_OUT + sizeof(int) * (C::SCHED_INTS + CU_INTS);
  static_assert(sizeof(int) * kSortMax <= (size_t)KV_BYTES, "len scratch fits the K area");
  static_assert(EPI_STORES < 64, "fits the vmcnt field");
};

// Stages [i0, i1) of one key segment's K and V, global -> LDS (stage i at offset
// i * TILE_BYTES of each area, in the streaming kernel's stage layout), bounded at the
// segment end.  (A device function: the HIP host pass does not instantiate a kernel
// template that calls the buffer-to-LDS load builtin itself.)
template <int D, int QB, int NW>
__device__ __forceinline__ void resident_load(const __bf16* kbase, const __bf16* vbase, int Lk, int i0, int i1,
                                              int64_t rs, char* kres, char* vres, int wave,
                                              const int (&src_k)[Tile<D, QB, NW, 64>::CPT],
                                              const int (&src_v)[Tile<D, QB, NW, 64>::CPT]) {
  using C = Tile<D, QB, NW, 64>;
  const int kbytes = (int)(rs * 2);
  for (int i = i0; i < i1; ++i) {
    const int rows = (Lk - 64 * i < 64) ? (Lk - 64 * i) : 64;
    __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)64 * i * rs), 0, rows * kbytes, kRsrcFlags);
    __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)64 * i * rs), 0, rows * kbytes, kRsrcFlags);
    char* kd = kres + i * C::TILE_BYTES + wave * C::CPT * 1024;
    char* vd = vres + i * C::TILE_BYTES + wave * C::CPT * 1024;
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kd + j * 1024), 16, src_k[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vd + j * 1024), 16, src_v[j], 0, 0, 0);
    }
  }
}

template <int D, int QB, int NW, int WPE>
__global__ void __launch_bounds__(kWave * NW) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
pfa_fwd_resident_kernel(Params p) {
  using R = ResidentTile<D, QB, NW>;
  using C = typename R::C;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* const kres = reinterpret_cast<char*>(smem);
  char* const vres = kres + R::KV_BYTES;
  char* const ostg = vres + R::KV_BYTES;
  int* s_order = reinterpret_cast<int*>(ostg + R::STAGE_OUT);
  int* s_prefix = s_order + kSortMax;
  int* s_cuq = s_order + C::SCHED_INTS;        // sorted mode: cu_seqlens_q, then _k
  int* s_cuk = s_cuq + kSortMax + 1;
  int* s_len = reinterpret_cast<int*>(kres);   // scratch, dead before the first K/V load

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;
  const int g = lane >> 5;
  const int i16 = lane & 15;
  const int hh = (lane >> 4) & 1;
  const int64_t rs = (int64_t)p.heads * D;
  const int kbytes = (int)(rs * 2);
  const float c = p.c;

  const int Tq = ld_table(p.cu_q, p.num_seqs);
  const int Tk = ld_table(p.cu_k, p.num_seqs);
  const bool sorted = p.num_seqs <= kSortMax;
  // Item decoding reads the segment tables from LDS (sorted mode), so that no vector-memory
  // load sits between the next tile's Q loads and the wait for them.
  if (sorted)
    for (int i = tid; i <= p.num_seqs; i += C::THREADS) {
      s_cuq[i] = p.cu_q[i];
      s_cuk[i] = p.cu_k[i];
    }
  const int total = sorted ? build_schedule<C::BM, C::THREADS>(p.cu_q, p.cu_k, p.num_seqs, p.heads, s_len,
                                                               s_order, s_prefix, kSortMax)
                           : p.num_seqs * p.heads * p.qt_max;
  // a contiguous run of the item list per workgroup: consecutive items share a
  // (segment, head) and its resident K/V
  const int64_t u_begin = (int64_t)total * blockIdx.x / gridDim.x;
  const int64_t u_end = (int64_t)total * (blockIdx.x + 1) / gridDim.x;

  // per-lane offsets: K rows (A operand of S^T), transposed V reads, stage-load sources
  int koff[C::KSTEP], voff[C::DT];
#pragma unroll
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, Swz::K>(n32, 2 * t + g);
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    voff[dt] = phys_off<D, Swz::V>(4 * g + (i16 >> 2), 4 * dt + 2 * hh + ((i16 & 3) >> 1)) + 8 * (i16 & 1);
  int src_k[C::CPT], src_v[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int P = (wave * C::CPT + i) * 64 + lane;
    src_k[i] = logical_src<D, Swz::K>(P, kbytes);
    src_v[i] = logical_src<D, Swz::V>(P, kbytes);
  }

  // work item u -> (segment, head, query tile) and the tile's query rows (all fields
  // wave-uniform; rank and nt: sorted mode only)
  struct Item {
    int s, h, qt, qa, Lq, rank, nt;
  };
  auto rfl = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  // false if the tile holds no query rows
  auto rows_of = [&](Item& it, int qe) -> bool {
    it.Lq = qe - it.qa;
    if (it.qa < 0 || it.qa >= Tq) return false;
    if (it.Lq > Tq - it.qa) it.Lq = Tq - it.qa;
    return it.Lq > 0 && it.qt * C::BM < it.Lq;
  };
  auto decode = [&](int64_t u, Item& it) -> bool {
    int qe;
    if (sorted) {
      int lo = 0, hi = p.num_seqs - 1;   // last rank r with s_prefix[r] <= u
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rfl(s_prefix[mid]) <= u) lo = mid; else hi = mid - 1;
      }
      it.rank = lo;
      it.s = rfl(s_order[lo]);
      it.qa = rfl(s_cuq[it.s]);
      qe = rfl(s_cuq[it.s + 1]);
      it.nt = (qe - it.qa + C::BM - 1) / C::BM;   // >= 1: a rank that holds item u has items
      const int local = (int)u - rfl(s_prefix[lo]);
      it.h = local / it.nt;
      it.qt = local - it.h * it.nt;
    } else {
      const int per_seg = p.heads * p.qt_max;
      it.s = (int)u / per_seg;
      const int rem = (int)u - it.s * per_seg;
      it.h = rem / p.qt_max;
      it.qt = rem - it.h * p.qt_max;
      it.qa = ld_table(p.cu_q, it.s);
      qe = ld_table(p.cu_q, it.s + 1);
    }
    return rows_of(it, qe);
  };
  // it holds item u - 1 (sorted mode: as decode left it); step it to item u.  Sorted mode
  // walks the list (next query tile, then head, then rank) instead of searching it.
  auto advance = [&](int64_t u, Item& it) -> bool {
    if (!sorted) return decode(u, it);
    if (++it.qt >= it.nt) {
      it.qt = 0;
      if (++it.h >= p.heads) {
        it.h = 0;
        while (it.rank + 1 < p.num_seqs && rfl(s_prefix[it.rank + 1]) <= u) ++it.rank;
        it.s = rfl(s_order[it.rank]);
        it.qa = rfl(s_cuq[it.s]);
        it.nt = (rfl(s_cuq[it.s + 1]) - it.qa + C::BM - 1) / C::BM;
      }
    }
    return rows_of(it, rfl(s_cuq[it.s + 1]));
  };
  // Q fragments of an item's tile (rows past the segment end are zero)
  auto load_q = [&](const Item& it, bf16x8 (&dst)[QB][C::KSTEP]) {
    const __bf16* qbase = p.q + (int64_t)it.qa * rs + (int64_t)it.h * D;
    const int q0 = it.qt * C::BM + wave * (QB * 32);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int row = q0 + b * 32 + n32;
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < it.Lq) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)row * rs + 16 * t + 8 * g);
        dst[b][t] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };

  // At d = 128 the next item's Q is loaded while the current tile computes, and before
  // its output stores: waiting for it then waits for no store.  (At d = 64 the second Q
  // register set does not fit beside two query blocks.)
  constexpr bool kPrefetchQ = D == 128;
  int64_t u = u_begin;
  Item cur;
  bool have = false;
  while (u < u_end && !(have = decode(u, cur))) ++u;
  bf16x8 qn[QB][C::KSTEP];
  if (kPrefetchQ && have) load_q(cur, qn);
  // nothing is in flight at the loop head but what the loop itself issued: without this
  // wait the compiler guards the stage loop's first products with a full vmcnt wait (it
  // cannot tell which path reaches them), and that wait would take in the next tile's Q
  __builtin_amdgcn_s_waitcnt(kWaitVmem);
  // first row and length of segment s's keys, clamped to the table and to the LDS bound (a
  // longer segment breaks the caller's max_seqlen_k; the kernel still stays in LDS)
  auto key_span = [&](int s_, int& ka, int& len) {
    if (sorted) {
      ka = rfl(s_cuk[s_]);
      len = rfl(s_cuk[s_ + 1]) - ka;
    } else {
      ka = ld_table(p.cu_k, s_);
      len = ld_table(p.cu_k, s_ + 1) - ka;
      // keeps the two branches' loads apart: merged, they become one generic-address load
      // whose wait would take in the next tile's Q loads
      asm volatile("" ::: "memory");
    }
    if (ka < 0 || ka > Tk) ka = Tk;
    if (len > Tk - ka) len = Tk - ka;
    if (len < 0) len = 0;
    if (len > R::KMAX) len = R::KMAX;
  };
  int res_s = -1, res_h = -1, ns = 0, Lk = 0;
  while (have) {
    const int s = cur.s, h = cur.h, qt = cur.qt, qa = cur.qa, Lq = cur.Lq;
    if (s != res_s || h != res_h) {
      // a new (segment, head): every wave is done with the old K/V, then all of the key
      // segment's stages come in global -> LDS, bounded at its end
      __syncthreads();
      int ka;
      key_span(s, ka, Lk);
      ns = (Lk + 63) / 64;
      resident_load<D, QB, NW>(p.k + (int64_t)ka * rs + (int64_t)h * D, p.v + (int64_t)ka * rs + (int64_t)h * D,
                               Lk, 0, ns, rs, kres, vres, wave, src_k, src_v);
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      res_s = s;
      res_h = h;
    }

    // ---- one query tile against the resident stages
    const int64_t head_off = (int64_t)h * D;
    const int q0 = qt * C::BM + wave * (QB * 32);
    TileState<D, QB> st;
    if constexpr (kPrefetchQ)
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(R::EPI_STORES));   // the Q loads, not the stores after them
    else
      load_q(cur, qn);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) st.qr[b][t] = qn[b][t];
      st.m_run[b] = -INFINITY;
      st.l_run[b] = 0.f;
      st.l_rnd[b] = 0.f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[b][dt][i] = 0.f;
    }
    Item nxt;
    bool have_next = false;
    int64_t un = u + 1;
    if (un < u_end) {
      nxt = cur;
      while (!(have_next = advance(un, nxt)) && ++un < u_end) {}
    }
    if (kPrefetchQ && have_next) load_q(nxt, qn);
    auto no_issue = [](char*, char*, int) {};
#pragma unroll 1
    for (int i = 0; i < ns; ++i)
      stage_body<D, QB, 64>(st, nullptr, nullptr, kres + i * C::TILE_BYTES, vres + i * C::TILE_BYTES, false,
                            no_issue, i, 64 * i, Lk, koff, voff, c, g);

    // ---- epilogue: O = acc / l_rnd in bf16, LSE; O leaves 32 channels at a time through
    // the wave's part of the staging area (rows of 64 bytes, 16-byte chunks XORed with
    // bits 2-3 of the row), read back as whole 64-byte row pieces
    // Every store is issued; the buffer bounds (this wave's valid rows) drop the rest, so
    // the count of vector-memory instructions after the next tile's Q loads is fixed.
    char* const ost = ostg + wave * (R::OUT_ROWS * 64);
    int vrows = Lq - q0;
    vrows = vrows < 0 ? 0 : (vrows > R::OUT_ROWS ? R::OUT_ROWS : vrows);
    vrows = __builtin_amdgcn_readfirstlane(vrows);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(p.out + (int64_t)(qa + q0) * rs + head_off), 0, vrows * kbytes, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        p.lse != nullptr ? uniform_ptr(p.lse + (int64_t)h * Tq + qa + q0) : nullptr, 0,
        p.lse != nullptr ? vrows * 4 : 0, kRsrcFlags);
    float inv[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float lt = partner_sum(st.l_run[b]);
      const float lr = partner_sum(st.l_rnd[b]);
      inv[b] = lr > 0.f ? 1.0f / lr : 0.f;   // no keys: O = 0 (and LSE = -inf)
      const int r = b * 32 + n32;
      const float lse_r = (st.m_run[b] + __builtin_amdgcn_logf(lt)) * kLn2;
      // the second half-wave holds the same rows: its offset lies past every bound
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_r), rl,
                                            g == 0 ? 4 * r : 0x40000000, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const int r = b * 32 + n32;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          bf16x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[b][dt][4 * ii + e] * inv[b]);
          *reinterpret_cast<bf16x4*>(ost + r * 64 + ((ii ^ ((r >> 2) & 3)) << 4) + 8 * g) = w;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave reads back what it wrote
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < R::OUT_ROWS * 4 / kWave; ++k) {
        const int P = k * kWave + lane;
        const int r = P >> 2, ch = P & 3;
        const u32x4 x = *reinterpret_cast<const u32x4*>(ost + r * 64 + ((ch ^ ((r >> 2) & 3)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(x, ro, r * kbytes + 64 * dt + 16 * ch, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // reads done before the next tile of channels
      __builtin_amdgcn_wave_barrier();
    }
    cur = nxt;
    u = un;
    have = have_next;
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

// head_dim 64, 128 x (the six kernel modes, the resident-K/V cross kernel), plus the
// eight-wave d = 64 variants of the self, cross and fused-QKV modes
constexpr int kModeResident = 6;
constexpr int kVariants = 17;
constexpr int kSortClasses = 4;   // schedule capacities 512, 1024, 2048, 4096
std::atomic<int> g_occ[kMaxDevices][kVariants][kSortClasses];

int variant_index(int head_dim, int mode, bool wide) {
  return wide ? 14 + (mode == kModeCross ? 1 : mode == kModeQkv ? 2 : 0) : (head_dim == 64 ? 0 : 1) + 2 * mode;
}

template <int D, int QB, int NW, int WPE>
Variant make_resident_variant() {
  using R = ResidentTile<D, QB, NW>;
  return Variant{reinterpret_cast<const void*>(&pfa_fwd_resident_kernel<D, QB, NW, WPE>), R::C::BM,
                 R::C::THREADS, R::LDS_BYTES};
}

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

template <int MODE, int NW64 = PFA_D64_NW>
Variant variant_of(int head_dim) {
  if (head_dim == 64) return make_variant<64, PFA_D64_QB, NW64, PFA_D64_SK, PFA_D64_WPE, MODE>();
  return make_variant<128, PFA_D128_QB, PFA_D128_NW, PFA_D128_SK, PFA_D128_WPE, MODE>();
}

// d = 64 with query segments of 512 rows or more: eight waves (512-query tiles), so each
// K/V stage load feeds twice the queries.  Shorter segments keep four waves, which would
// otherwise idle half of a 512-query tile.  The block-sparse modes keep the 256-query
// tile their layouts are made of, the FP8 modes the four-wave split of their V loads.
constexpr int kD64WideNW = 8;
constexpr int kWideMinQ = 512;
bool use_wide64(int head_dim, int mode, int max_seqlen_q) {
  return head_dim == 64 && max_seqlen_q >= kWideMinQ &&
         (mode == kModeSelf || mode == kModeCross || mode == kModeQkv);
}
Variant wide64_for(int mode) {
  return mode == kModeCross ? variant_of<kModeCross, kD64WideNW>(64)
       : mode == kModeQkv   ? variant_of<kModeQkv, kD64WideNW>(64)
                            : variant_of<kModeSelf, kD64WideNW>(64);
}

Variant variant_for(int head_dim, int mode) {
  if (mode == kModeResident)
    return head_dim == 64 ? make_resident_variant<64, PFA_D64_QB, PFA_D64_NW, PFA_D64_WPE>()
                          : make_resident_variant<128, PFA_D128_QB, PFA_D128_NW, PFA_D128_WPE>();
  return mode == kModeCross  ? variant_of<kModeCross>(head_dim)
       : mode == kModeQkv    ? variant_of<kModeQkv>(head_dim)
       : mode == kModeSparse ? variant_of<kModeSparse>(head_dim)
       : mode == kModeFp8    ? variant_of<kModeFp8>(head_dim)
       : mode == kModeSparseFp8 ? variant_of<kModeSparseFp8>(head_dim)
                             : variant_of<kModeSelf>(head_dim);
}

// Size the persistent grid of one forward variant and launch it.  prm carries every
// field but qt_max; the caller has checked the arguments.
int launch_fwd(Params prm, int mode, int max_seqlen_q, int head_dim, hipStream_t stream) {
  const bool wide = use_wide64(head_dim, mode, max_seqlen_q);
  const Variant var = wide ? wide64_for(mode) : variant_for(head_dim, mode);
  const int64_t qt_max = ((int64_t)max_seqlen_q + var.bm - 1) / var.bm;
  const int64_t slots = (int64_t)prm.num_seqs * prm.heads * qt_max;
  if (slots > INT32_MAX) return PFA_ERR_SIZE;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != PFA_OK) return rc;
  // Schedule capacity: the streaming kernel's LDS grows (two ints per entry) so that tables
  // of up to kSortCapMax segments are sorted longest-first; the resident kernel's LDS is
  // full and keeps kSortMax.  Beyond the capacity the kernels walk the unsorted slots.
  int cap = kSortMax, cls = 0;
  if (mode != kModeResident && prm.num_seqs > kSortMax && prm.num_seqs <= kSortCapMax)
    while (cap < prm.num_seqs) {
      cap <<= 1;
      ++cls;
    }
  const size_t lds = var.lds + sizeof(int) * 2 * (size_t)(cap - kSortMax);
  const size_t lds_max = mode == kModeResident ? var.lds : var.lds + sizeof(int) * 2 * (size_t)(kSortCapMax - kSortMax);
  const int vi = variant_index(head_dim, mode, wide);
  int occ = g_occ[dev][vi][cls].load(std::memory_order_relaxed);
  if (occ <= 0) {
    if (hipFuncSetAttribute(var.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max) != hipSuccess)
      return PFA_ERR_DEVICE;
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, var.fn, var.threads, lds) != hipSuccess || o <= 0)
      return PFA_ERR_DEVICE;
    occ = o;
    g_occ[dev][vi][cls].store(occ, std::memory_order_relaxed);
  }
  int64_t grid = (int64_t)cus * occ;
  if (grid > slots) grid = slots;
  if (grid >= 8) grid -= grid % 8;   // keep whole rounds on every XCD
  prm.qt_max = (int)qt_max;
  prm.sort_cap = cap;
  void* args[] = {&prm};
  const hipError_t err = hipLaunchKernel(var.fn, dim3((unsigned)grid), dim3(var.threads), args, lds, stream);
  return err == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
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
  // q, k, v and out move in 16-byte vectors
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned4(lse) ||
      misaligned4(cu_seqlens_q) || misaligned4(cu_seqlens_k))
    return PFA_ERR_ALIGN;
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
  // key segments that all fit in LDS: the resident-K/V kernel, for self-attention too (a
  // short segment's tiles then load its K/V in one go; with one tile per segment there is
  // nothing to reuse, but the tile's stages no longer wait on a streamed ring)
  const int resident_max = head_dim == 64 ? resident_keys<64>() : resident_keys<128>();
  const int mode = max_seqlen_k <= resident_max        ? kModeResident
                 : cu_seqlens_k == cu_seqlens_q ? kModeSelf
                                                 : kModeCross;
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
  if (misaligned16(qkv) || misaligned16(out) || misaligned4(lse) || misaligned4(cu_seqlens) ||
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
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned4(lse) ||
      misaligned4(cu_seqlens) || misaligned4(kv_ptr) || misaligned4(kv_idx))
    return PFA_ERR_ALIGN;
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
  if (misaligned16(v8) || misaligned16(v_scale) || misaligned16(q) || misaligned16(k) || misaligned16(out) ||
      misaligned4(lse) || misaligned4(cu_seqlens))
    return PFA_ERR_ALIGN;
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
  if (misaligned16(v8) || misaligned16(v_scale) || misaligned16(q) || misaligned16(k) || misaligned16(out) ||
      misaligned4(lse) || misaligned4(cu_seqlens) || misaligned4(kv_ptr) || misaligned4(kv_idx))
    return PFA_ERR_ALIGN;
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

}  // extern "C"
