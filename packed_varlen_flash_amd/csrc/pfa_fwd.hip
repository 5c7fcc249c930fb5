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
// gfx950 mapping (both head sizes: one workgroup = 8 wave64s on one CU, two per SIMD):
//   * work unit = (segment, head, 256-row query tile); a tile never spans two segments.
//     Tiles are listed longest segment first and handed out round-robin by a persistent
//     grid; each XCD receives contiguous runs of the list so the query tiles that share
//     one (segment, head) K/V stream sit behind the same L2.
//   * each wave owns 32 queries and keeps their Q fragments in VGPRs.
//   * the two waves of a SIMD belong to different groups, one slot apart: while one runs
//     the MFMAs of a stage (QK of the next stage, PV of the current one), the other runs
//     the softmax of a stage on the vector ALU, and they swap at the next workgroup
//     barrier, so the matrix cores and the VALU work side by side.
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
#include <type_traits>
#include <vector>

#include "pfa_common.h"

namespace {

// How far (base 2) a block max may exceed the running max before O and l are rescaled.
// 0 keeps the reference equal to the exact running max, so the largest weight of a row is
// exactly 1 and carries no bf16 rounding; a positive slack saves rescales (about 5% on
// 4096-token segments) but leaves that weight rounded, which on sharp softmax rows pushes
// the worst output error past 1e-2 of the exact result.
#ifndef PFA_RESCALE_SLACK
#define PFA_RESCALE_SLACK 0.0f
#endif
constexpr float kRescaleSlack = PFA_RESCALE_SLACK;

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
__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
// Block-sparse variant: a compacted copy of the tile's key-block list lives in LDS after
// the schedule (count in the last slot), so segments are limited to this many key blocks.
constexpr int kSparseMaxBlocks = 1024;
constexpr int kSparseLdsBytes = (kSparseMaxBlocks + 4) * 4;

#ifndef PFA_LOAD_ALL
#define PFA_LOAD_ALL 1
#endif

// Workgroup geometry at both head sizes: 8 wave64s, wave w owns query rows 32w .. 32w+31 of
// a 256-row tile.  The hardware places wave w on SIMD w % 4, so waves 0-3 (group 0) and
// 4-7 (group 1) put one wave of each group on every SIMD.  Keys come in 64-key stages.
template <int D>
struct Tile {
  static constexpr int NW = 8;
  static constexpr int THREADS = kWave * NW;
  static constexpr int BM = NW * 32;                // query rows per workgroup tile
  static constexpr int SK = 64;                     // keys per LDS stage
  static constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  static constexpr int TILE_BYTES = SK * D * 2;     // one K (or V) stage
  static constexpr int NCH = SK * CPR;              // 16-byte chunks of one stage
  static constexpr int CPT = NCH / THREADS;         // ... per thread
  static constexpr int NCH8 = SK * D / 16;          // 16-byte chunks of one e4m3 V stage
  // Stage loads are issued by the waves of one group (the one in its softmax step at
  // the even slots where loads go out), or by all waves with PFA_LOAD_ALL.
  static constexpr int LW = PFA_LOAD_ALL ? NW : NW / 2;   // loading waves
  static constexpr int CPL = NCH / (LW * kWave);           // bf16 chunks per loading lane
  static constexpr int CPL8 = NCH8 >= LW * kWave ? NCH8 / (LW * kWave) : 1;   // e4m3 chunks
  static constexpr int DT = D / 32;                 // 32-row output tiles along head_dim
  static constexpr int KSTEP = D / 16;              // 16-deep steps of the Q.K contraction
  static constexpr int SCHED_INTS = 2 * kSortMax + 8;
  static constexpr int RING_BYTES = 2 * TILE_BYTES; // two-slot K ring; the V ring follows
  static constexpr size_t LDS_BYTES = (size_t)2 * RING_BYTES + sizeof(int) * SCHED_INTS;
  static_assert(CPT * THREADS == NCH, "stage must split evenly");
  static_assert(NCH8 % kWave == 0 && NCH8 <= THREADS, "e4m3 stage in whole waves");
  static_assert(sizeof(int) * kSortMax <= (size_t)RING_BYTES, "len scratch fits");
  static_assert(4 * 32 * D * 2 <= RING_BYTES, "a group's output blocks fit one ring");
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

// Register arithmetic is free to move across a workgroup barrier (the barrier orders
// memory only).  An empty volatile asm that takes a value as in/out operand keeps its
// computation on this side of the next barrier: the step that produced it stays in its
// slot instead of sinking into the next one.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Workgroup barrier without a memory fence.  __syncthreads() adds one, and since the
// global -> LDS stage loads count as outstanding LDS writes, its fence waits for every
// load in flight, including those issued in the slot that just started and not needed for
// two more slots.  The slot loop waits for exactly the loads it needs (s_waitcnt before
// the barrier of every even slot) and consumes every LDS read of a step inside that step,
// so the plain barrier suffices; the memory clobber keeps the compiler from moving LDS
// accesses across it.
__device__ __forceinline__ void slot_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------
// One query tile of one (segment, head): the per-wave state and the two kinds of step.
//
// Every wave alternates two kinds of step, one per "slot" (the time between two workgroup
// barriers):
//   MFMA step j:  S_{j+1}^T = K_{j+1} Q^T (QK of the next stage) and O^T += V_j^T P_j^T
//                 (PV of the current one): 32 MFMAs at d = 128, their LDS reads, no VALU;
//   softmax step j:  mask, row max, rescale decision (and O rescale) and the weights P_j
//                 of stage j from S_j: VALU only.
// Group 1 runs one slot behind group 0, so in every slot each SIMD holds one wave in an
// MFMA step and one in a softmax step, and the matrix cores and the vector ALU work side
// by side.  In lockstep (both waves of a SIMD in the same kind of step, which a barrier
// per stage brings about) the two pipes mostly take turns.
// ---------------------------------------------------------------------------------
template <int D>
struct TileState {
  bf16x8 qr[D / 16];             // Q fragments (B operand of K Q^T)
  f32x16 o[D / 32];              // O^T accumulators
  float m_run;                   // running max (base-2 scaled)
  float l_run;                   // row sum of the fp32 weights (gives the LSE; normalises FP8 O)
  float l_rnd;                   // row sum of the bf16 weights (normalises bf16 O)
};

// V^T operand of output tile dt, 16-key step cc of the 32-key sub-block at vst: two
// transposed reads 8 rows apart (voff[dt]: this lane's offset for rows 4g + i16/4).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* vst, int voff) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vst + voff));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vst + voff + 8 * D * 2));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

#ifndef PFA_MFMA_PRIO
#define PFA_MFMA_PRIO 2
#endif
#ifndef PFA_PV_AHEAD
#define PFA_PV_AHEAD 2
#endif

// MFMA step (bf16 P.V).  QK: whether a next stage exists.  kst: K stage j+1 (both 32-key
// sub-blocks, koff[t] = this lane's offset of row n32, chunk 2t+g); vst: V stage j.  The
// 2 D/16 QK MFMAs and as many PV MFMAs alternate two and two; every accumulator chain
// has at least three independent MFMAs between two of its links.  LDS reads run
// PFA_PV_AHEAD contraction steps ahead of the MFMAs that use them.
template <int D, bool QK>
__device__ __forceinline__ void mfma_step(TileState<D>& st, f32x16& s0, f32x16& s1, const bf16x8 (&pb)[2][2],
                                          const char* __restrict__ kst, const char* __restrict__ vst,
                                          const int (&koff)[D / 16], const int (&voff)[D / 32]) {
  constexpr int KS = D / 16, DT = D / 32;
  if constexpr (QK) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    if constexpr (QK) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kst + koff[t]);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kst + 32 * D * 2 + koff[t]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.qr[t], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, st.qr[t], s1, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * t + e;                 // sub-block i / (2 DT), key step (i / DT) & 1, tile i % DT
      const int sub = i / (2 * DT), cc = (i / DT) & 1, dt = i % DT;
      const bf16x8 va = v_operand<D>(vst + sub * 32 * D * 2 + cc * 16 * D * 2, voff[dt]);
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[sub][cc], st.o[dt], 0, 0, 0);
    }
  }
  // order: the reads of PFA_PV_AHEAD steps first, then per step its MFMAs and the reads
  // of the step PFA_PV_AHEAD further on
  constexpr int RD = QK ? 6 : 4;   // LDS reads per step: 2 K rows (QK only) + 4 transposed V
  constexpr int MF = QK ? 4 : 2;   // MFMAs per step
  constexpr int AH = PFA_PV_AHEAD < KS ? PFA_PV_AHEAD : KS - 1;
  __builtin_amdgcn_sched_group_barrier(0x100, RD * AH, 0);
#pragma unroll
  for (int t = 0; t < KS - AH; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, MF * AH, 0);
}

// MFMA step with P.V in FP8: the QK of mfma_step, then one 32x32x64 FP8 MFMA per output
// tile over all 64 keys (weights pw from softmax_body8, V^T from the e4m3 stage).
template <int D, bool QK>
__device__ __forceinline__ void mfma_step8(TileState<D>& st, f32x16& s0, f32x16& s1, const i32x8& pw,
                                           const char* __restrict__ kst, const char* __restrict__ vst,
                                           const int (&koff)[D / 16], const int (&voff8)[D / 32]) {
  constexpr int KS = D / 16, DT = D / 32;
  if constexpr (QK) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < KS; ++t) {
    if constexpr (QK) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kst + koff[t]);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kst + 32 * D * 2 + koff[t]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.qr[t], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, st.qr[t], s1, 0, 0, 0);
    }
    if (t % 2 == 1) {
      const int dt = t / 2;
      const i32x8 va = v8_operand<D>(vst, voff8[dt]);
      st.o[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pw, st.o[dt], 0, 0, 0, 0, 0, 0);
    }
  }
}

// Softmax step, first part, over a whole 64-key stage (both sub-blocks): key mask on the
// segment's last stage, row max, one rescale decision.  O is rescaled in place: the
// wave's MFMAs that accumulate into it ran in its previous slot.
template <int D>
__device__ __forceinline__ void softmax_head64(TileState<D>& st, f32x16& s0, f32x16& s1, int key0, int L,
                                               float c, int g, float slack) {
  if (key0 + 64 > L) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + (i >> 2) * 8 + 4 * g + (i & 3);
      if (key >= L) s0[i] = -INFINITY;
      if (key + 32 >= L) s1[i] = -INFINITY;
    }
  }
  float mx = fmaxf(s0[0], s0[1]);
#pragma unroll
  for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
  mx = partner_max(mx);
  const float mb = mx * c;
  if (__builtin_amdgcn_ballot_w64(mb > st.m_run + slack) != 0) {
    const float m_new = fmaxf(st.m_run, mb);
    const float a = __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= a;
    st.l_rnd *= a;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[dt][i] *= a;
  }
}

// Softmax step, second part (straight-line): P = 2^(s*c - m) as bf16 B operands and two
// row sums.  l_run adds the fp32 weights and gives the LSE (a sum of bf16-rounded weights
// can carry up to 2^-8 relative error, 3.9e-3, into the LSE of a sharp row).  l_rnd adds
// the bf16 weights the PV product actually uses and normalises O: each weight's rounding
// then enters numerator and denominator alike, so the error is sum_j dp_j (v_j - O) / l
// rather than sum_j dp_j v_j / l.  That matters on rows with few keys and large, similar
// values (|O| in [2, 4), where bf16 rounding of O already takes 2^-7 of the 1e-2 bar);
// normalising by l_run there was measured past the bar.  Both sums chain straight into
// their running values (one add, resp. one bf16 dot of a weight pair, per step).
template <int D>
__device__ __forceinline__ void softmax_body(TileState<D>& st, const f32x16& s, bf16x8 (&pb)[2], float c) {
  const float neg_m = -st.m_run;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[i], c, neg_m));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, neg_m));
    st.l_run += e0;
    st.l_run += e1;
    const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
    st.l_rnd = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, st.l_rnd, false);
    pb[i >> 3][i & 7] = pr[0];
    pb[i >> 3][(i & 7) + 1] = pr[1];
  }
}

// FP8 variant of softmax_body: weights w = 2^(s c - m + 8) rounded to e4m3 (nearest even)
// four to a register, sub-block `half` filling bytes 16 half .. 16 half + 15 of the P^T
// operand in the order of the accumulator elements; l_run adds the unrounded weights,
// which also normalise O.
template <int D>
__device__ __forceinline__ void softmax_body8(TileState<D>& st, const f32x16& s, i32x8& pw, int half,
                                              float c) {
  const float off = kP8Log2 - st.m_run;
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(s[i], c, off));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c, off));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(s[i + 2], c, off));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(s[i + 3], c, off));
    st.l_run += e0;
    st.l_run += e1;
    st.l_run += e2;
    st.l_run += e3;
    int w = 0;
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
    pw[half * 4 + (i >> 2)] = w;
  }
}

// Rotary position embedding, rotate-half pairing, of one pair of 8-feature chunks: lo
// holds features i .. i+7 of a row and hi their partners i + D/2 .. i + D/2 + 7; cs and
// sn point at the cosines and sines of those 8 pairs' angles.  Each pair (a, b) turns to
// (a cos - b sin, b cos + a sin), evaluated in fp32 and rounded once to bf16 (nearest
// even).  The DiT block of the Mage-Flow page (section on its fusion opportunities)
// rotates q and k between the QKV projection and attention.
__device__ __forceinline__ void rope_rotate(bf16x8& lo, bf16x8& hi, const float* cs, const float* sn) {
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

// ---------------------------------------------------------------------------------
// One query tile of one (segment, head).
//
// Stage j's K is read by the MFMA step j-1 (QK of stage j), its V by MFMA step j (PV).
// With group 1 one slot behind group 0, K_j is read in slots 2j and 2j+1 and V_j in slots
// 2j+2 and 2j+3.  Both rings have two slots.  At every even slot 2u, right after its
// barrier, the workgroup issues K_{u+1} and V_u (global -> LDS, bounded at the segment
// end); each lands in the ring slot whose last readers the barrier just retired, and has
// two slots to arrive before its first reader.
// ---------------------------------------------------------------------------------
// MODE also keys the instantiation to its kernel variant (the HIP host pass rejects a
// device template specialisation shared by two kernel templates' instantiations).
template <int D, int MODE>
__device__ __forceinline__ void process_tile(const Params& p, char* kring, char* vring, int* s_blk, int seg,
                                             int qa, int Lq, int ka, int Lk, int h, int qt, int Tq) {
  using C = Tile<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int grp = wave >> 2;         // 0: waves 0-3, 1: waves 4-7 (one slot behind)
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
  const int q0 = qt * C::BM + wave * 32;
  int ns = (Lk + C::SK - 1) / C::SK;       // stages (0 when the key segment is empty)
  const float c = p.c;
  if constexpr (mode_sparse(MODE)) {
    // The tile's list, compacted by wave 0 into LDS: entries outside the segment's key
    // blocks are dropped, the rest keep their order.  ns becomes the number kept.  (The
    // previous tile's last barrier retired every reader of the old list.)
    static_assert(C::SK == 64, "key blocks are 64-key stages");
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
    if constexpr (mode_sparse(MODE)) return __builtin_amdgcn_readfirstlane(s_blk[i]) * C::SK;
    else return i * C::SK;
  };

  TileState<D> st;
  {
    const int row = q0 + n32;
#pragma unroll
    for (int t = 0; t < C::KSTEP; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < Lq) x = *reinterpret_cast<const u32x4*>(qbase + (int64_t)row * q_rs + 16 * t + 8 * g);
      st.qr[t] = __builtin_bit_cast(bf16x8, x);
    }
    if constexpr (MODE == kModeQkv) {
      // rotate-half RoPE: the lane's chunk t holds features 16t + 8g + 0..7 and chunk
      // t + KSTEP/2 their partners D/2 further on, so each pair is rotated in registers
      if (p.rope_cos != nullptr && row < Lq) {
        const int64_t tab = (int64_t)(qa + row) * (D / 2);
#pragma unroll
        for (int t = 0; t < C::KSTEP / 2; ++t)
          rope_rotate(st.qr[t], st.qr[t + C::KSTEP / 2], p.rope_cos + tab + 16 * t + 8 * g,
                      p.rope_sin + tab + 16 * t + 8 * g);
      }
    }
  }
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  st.l_rnd = 0.f;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[dt][i] = 0.f;

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
  // of a neighbouring segment is ever read.  The host keeps 64 rows of every stride
  // within int range.
  const int kbytes = (int)(k_rs * 2);
  const int vbytes = (int)(v_rs * 2);
  const bool loader = PFA_LOAD_ALL || grp == 1;
  const int lw = PFA_LOAD_ALL ? wave : wave - C::NW / 2;   // index among the loading waves
  int src_k[C::CPL], src_v[C::CPL];      // logical source offsets of this lane's chunks
#pragma unroll
  for (int i = 0; i < C::CPL; ++i) {
    const int P = (lw * C::CPL + i) * 64 + lane;
    src_k[i] = logical_src<D, Swz::K>(P, kbytes);
    if constexpr (mode_fp8(MODE)) {
      if (i < C::CPL8) src_v[i] = logical_src8<D>((lw * C::CPL8 + i) * 64 + lane, (int)rs);
    } else {
      src_v[i] = logical_src<D, Swz::V>(P, vbytes);
    }
  }
  auto issue_k = [&](int stage) {
    if (!loader) return;
    const int kb = stage_key(stage);
    const int rows = (Lk - kb < C::SK) ? (Lk - kb) : C::SK;
    __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)kb * k_rs), 0, rows * kbytes, kRsrcFlags);
    char* kdst = kring + (stage & 1) * C::TILE_BYTES + lw * C::CPL * 1024;
#pragma unroll
    for (int i = 0; i < C::CPL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kdst + i * 1024), 16, src_k[i], 0, 0, 0);
  };
  auto issue_v = [&](int stage) {
    if (!loader) return;
    const int kb = stage_key(stage);
    const int rows = (Lk - kb < C::SK) ? (Lk - kb) : C::SK;
    if constexpr (mode_fp8(MODE)) {
      if (lw * C::CPL8 * kWave < C::NCH8) {
        __amdgpu_buffer_rsrc_t r8 = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v8base + (int64_t)kb * rs), 0, rows * (int)rs, kRsrcFlags);
        char* vdst = vring + (stage & 1) * C::TILE_BYTES + lw * C::CPL8 * 1024;
#pragma unroll
        for (int i = 0; i < C::CPL8; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r8, (lds_void*)(vdst + i * 1024), 16, src_v[i], 0, 0, 0);
      }
    } else {
      __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)kb * v_rs), 0, rows * vbytes, kRsrcFlags);
      char* vdst = vring + (stage & 1) * C::TILE_BYTES + lw * C::CPL * 1024;
#pragma unroll
      for (int i = 0; i < C::CPL; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vdst + i * 1024), 16, src_v[i], 0, 0, 0);
    }
  };
  // Start of slot t: at even slots the loads issued two slots earlier must have landed
  // (each wave waits for its own, the barrier for everyone's); then the next go out.
  auto slot = [&](int t) {
    if ((t & 1) == 0 && t > 0 && loader) __builtin_amdgcn_s_waitcnt(kWaitVmem);
    slot_barrier();
    if ((t & 1) == 0) {
      const int u = t >> 1;
      if (u + 1 < ns) issue_k(u + 1);
      if (u < ns) issue_v(u);
    }
  };

  f32x16 s0, s1;                  // scores of the stage after the current one
  bf16x8 pb[2][2];                // bf16 weights of the current stage (B operands)
  i32x8 pw;                       // FP8 variant: its e4m3 weights
  auto pin_o = [&]() {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) pin(st.o[dt]);
  };
  auto softmax_step = [&](int j) {
    // FP8 weights must stay below 448: no slack there
    softmax_head64<D>(st, s0, s1, stage_key(j), Lk, c, g, mode_fp8(MODE) ? 0.f : kRescaleSlack);
    if constexpr (mode_fp8(MODE)) {
      softmax_body8<D>(st, s0, pw, 0, c);
      softmax_body8<D>(st, s1, pw, 1, c);
      pin(pw);
    } else {
      softmax_body<D>(st, s0, pb[0], c);
      softmax_body<D>(st, s1, pb[1], c);
      pin(pb[0][0]);
      pin(pb[0][1]);
      pin(pb[1][0]);
      pin(pb[1][1]);
    }
    pin(st.m_run);
    pin(st.l_run);
    pin(st.l_rnd);
    pin_o();
  };
  // MFMA step j: K_{j+1} in K slot KS (when QK), V_j in V slot VS
  auto step_mfma = [&](auto qk, auto kslot, auto vslot) {
    constexpr bool QK = decltype(qk)::value;
    const char* kst = kring + decltype(kslot)::value * C::TILE_BYTES;
    const char* vst = vring + decltype(vslot)::value * C::TILE_BYTES;
    // the wave in its MFMA step issues first: its partner's VALU fills the gaps between
    // MFMAs instead of delaying them
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(PFA_MFMA_PRIO);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (mode_fp8(MODE)) mfma_step8<D, QK>(st, s0, s1, pw, kst, vst, koff, voff);
    else mfma_step<D, QK>(st, s0, s1, pb, kst, vst, koff, voff);
    if constexpr (QK) {
      pin(s0);
      pin(s1);
    }
    pin_o();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  if (ns > 0) {
    issue_k(0);
    if (loader) __builtin_amdgcn_s_waitcnt(kWaitVmem);
    if (grp == 1) slot(0);
    // QK of stage 0 (K slot 0): S_0
    slot(grp);
    {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = 0.f;
        s1[i] = 0.f;
      }
      bf16x8 ka[C::KSTEP], kb[C::KSTEP];
      k_operands2<D>(kring, kring + 32 * D * 2, koff, ka, kb);
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t], st.qr[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[t], st.qr[t], s1, 0, 0, 0);
      }
      pin(s0);
      pin(s1);
    }
    int j = 0;
    for (; j + 2 < ns; j += 2) {      // stages j and j+1 both have a next stage
      slot(2 * j + 1 + grp);
      softmax_step(j);
      slot(2 * j + 2 + grp);
      step_mfma(T_{}, I1{}, I0{});
      slot(2 * j + 3 + grp);
      softmax_step(j + 1);
      slot(2 * j + 4 + grp);
      step_mfma(T_{}, I0{}, I1{});
    }
    slot(2 * j + 1 + grp);
    softmax_step(j);
    slot(2 * j + 2 + grp);
    if (ns - j == 2) {
      step_mfma(T_{}, I1{}, I0{});
      slot(2 * j + 3 + grp);
      softmax_step(j + 1);
      slot(2 * j + 4 + grp);
      step_mfma(F_{}, I0{}, I1{});
    } else {
      step_mfma(F_{}, I0{}, I0{});
    }
    if (grp == 0) slot(2 * ns + 1);
  }

  // ---- epilogue: O = acc / l_rnd (FP8: acc / l_run) in bf16 (round to nearest even),
  // LSE = ln2 * (m + log2 l_run).  Group 0 finishes while group 1 runs its last MFMA step
  // on the V ring, and stages its output in the K ring; group 1 follows after a barrier
  // and stages in the V ring.  Each wave writes its 32 x D block into its own part of
  // the ring in the swizzled K layout, then reads it back as whole 16-byte chunks of
  // consecutive rows, so 16 lanes store 256 contiguous bytes instead of every store
  // instruction touching 16-byte pieces of 32 different rows.
  auto epilogue = [&](char* region) {
    char* const ost = region + (wave & 3) * (32 * D * 2);
    const float lt = partner_sum(st.l_run);
    const float lr = mode_fp8(MODE) ? lt : partner_sum(st.l_rnd);
    const float inv = lr > 0.f ? 1.0f / lr : 0.f;   // no keys: O = 0 (and LSE = -inf)
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
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[dt][4 * ii + e] * sc[e]);
        *reinterpret_cast<bf16x4*>(ost + phys_off<D, Swz::K>(n32, 4 * dt + ii) + 8 * g) = w;
      }
    const float mfix = mode_fp8(MODE) ? st.m_run - kP8Log2 : st.m_run;   // FP8 sums 2^8 p
    if (p.lse != nullptr && g == 0 && q0 + n32 < Lq)
      p.lse[(int64_t)h * Tq + qa + q0 + n32] = (mfix + __builtin_amdgcn_logf(lt)) * kLn2;
    // the wave reads back only what it wrote
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    constexpr int OCH = 32 * C::CPR;      // 16-byte chunks of the wave's block
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
  };
  if (grp == 0) epilogue(kring);
  __syncthreads();
  if (grp == 1) epilogue(vring);
  // the next tile's first barrier retires the V-ring readers above before any V load
}

// kModeCross: separate query and key tables; otherwise the key table is the query table
// (known at compile time, so the key-side offsets and lengths fold into the query ones).
template <int D, int MODE>
__global__ void __launch_bounds__(kWave * Tile<D>::NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
pfa_fwd_kernel(Params p) {
  const int32_t* const cu_k = MODE == kModeCross ? p.cu_k : p.cu_q;
  using C = Tile<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* kring = reinterpret_cast<char*>(smem);
  char* vring = kring + C::RING_BYTES;
  int* s_order = reinterpret_cast<int*>(smem + 2 * C::RING_BYTES);
  int* s_prefix = s_order + kSortMax;
  int* s_blk = s_order + C::SCHED_INTS;     // block-sparse variant only (its LDS is larger)
  int* s_len = reinterpret_cast<int*>(kring);  // scratch, dead before the first K tile lands

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
    process_tile<D, MODE>(p, kring, vring, s_blk, s, qa, Lq, ka, Lk, h, qt, Tq);
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

template <int D, int MODE>
Variant make_variant() {
  using C = Tile<D>;
  static_assert(!mode_sparse(MODE) || (C::BM == PFA_SPARSE_BLOCK_Q && C::SK == PFA_SPARSE_BLOCK_K),
                "the block-sparse layout's blocks are the kernel's query tile and key stage");
  return Variant{reinterpret_cast<const void*>(&pfa_fwd_kernel<D, MODE>), C::BM, C::THREADS,
                 C::LDS_BYTES + (mode_sparse(MODE) ? kSparseLdsBytes : 0)};
}

constexpr int kVariants = 12;  // head_dim 64, 128 x the six kernel modes
std::atomic<int> g_occ[kMaxDevices][kVariants];

int variant_index(int head_dim, int mode) { return (head_dim == 64 ? 0 : 1) + 2 * mode; }

template <int MODE>
Variant variant_of(int head_dim) {
  if (head_dim == 64) return make_variant<64, MODE>();
  return make_variant<128, MODE>();
}

Variant variant_for(int head_dim, int mode) {
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

}  // extern "C"
