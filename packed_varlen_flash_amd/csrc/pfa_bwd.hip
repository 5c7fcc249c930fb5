// pfa_bwd.hip -- backward (dQ, dK, dV) of the packed varlen attention forward for gfx950,
// behind the C ABI (pfa_varlen_bwd).
#include <type_traits>

#include "pfa_common.h"

namespace {

// ---------------------------------------------------------------------------------
// Backward.  For upstream gradient dO of O, with P the softmax of each query row over
// its segment (recomputed from the forward's LSE) and s = scale q.k, the chain rule of
// the forward definition gives (per segment and head)
//     dV = P^T dO,  dP = dO V^T,  delta_i = sum_j P_ij dP_ij = dO_i . O_i,
//     dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
// Two launches, no atomics and no scratch of the library's own:
//   * dQ (first): one work item = 256 queries; the forward's shape: S^T = K Q^T, dP^T = V dO^T
//     (lanes hold queries), dQ^T += K^T dS^T with K^T from transposed LDS reads.  It also
//     writes each query row's statistics, ws[0] = -LSE * log2(e) and ws[1] = delta =
//     rowsum(dO * O), fp32 [H, T] each, to the caller's workspace;
//   * dK/dV (second, reading ws): one work item = 128 keys of one (segment, head), stationary in VGPRs as the
//     B operands of S = Q K^T and dP = dO V^T (lanes hold keys); the segment's Q and dO
//     stream through LDS in 64-row stages; dV^T += dO^T P and dK^T += Q^T dS take their
//     A operands from transposed LDS reads of the same stages.
// Every stage tile is read both as rows and transposed, so it is stored in the KV swizzle,
// free of bank conflicts for both patterns; the transposed reads take explicit per-lane
// offsets for each 16-row step and 8-row half, since the swizzle does not keep a constant
// pattern 8 rows apart.
// ---------------------------------------------------------------------------------
// Waves per workgroup.  dK/dV at d = 128: four, one per SIMD; it holds two accumulators
// and the stationary K and V fragments (450 registers), so one workgroup fills a CU.  At
// d = 64 it fits 256 registers: eight waves, two per SIMD, 256 keys per item.  dQ: eight, two per
// SIMD; it loads its two operand sets one after the other and fits 256 registers (its few
// spills are per-item offsets, reloaded outside the stage loop), and one K/V stage load
// feeds 256 queries.
constexpr int kBwdNW = 4;
constexpr int kBwdRows = kBwdNW * 32;      // keys per dK/dV work item at d = 128 (bounds slot counts)
template <int D>
constexpr int kDkdvNW = D == 64 ? 8 : kBwdNW;   // dK/dV waves per workgroup
constexpr int kDqNW = 8;
constexpr int kDqRows = kDqNW * 32;        // queries per dQ work item
constexpr int kBwdStage = 64;              // rows per streamed stage

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* out;
  const __bf16* dout;
  const float* lse;
  float* ws;              // [2][heads][T]: -LSE*log2(e), then delta
  int ws_rows;            // largest T the workspace holds: the kernels do nothing beyond it
  const int32_t* cu;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  int num_seqs;
  int heads;
  int tiles_max;          // ceil(max_seqlen / dK/dV keys per item): slots per (segment, head), unsorted mode
  int tiles_max_q;        // ceil(max_seqlen / kDqRows): the same for dQ
  float c;                // scale * log2(e)
  float scale;
};

template <int D, int NW = kBwdNW>
struct BwdTile {
  static constexpr int THREADS = kWave * NW;
  static constexpr int CPR = D / 8;                          // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBwdStage * D * 2;       // one 64-row bf16 tile
  static constexpr int CPT = kBwdStage * CPR / THREADS;      // chunks per thread per tile
  static constexpr int DT = D / 32;
  static constexpr int KSTEP = D / 16;
  static constexpr int ROWF_BYTES = kBwdStage * 4;           // one 64-row fp32 vector
  // dK/dV: [Q ring][dO ring][row-vector ring: 2 x (neg_lse2, delta)], which the epilogue
  // reuses for the staged dK and dV blocks (one each per wave), then the schedule
  static constexpr int DKDV_RING = (kStages * 2 * TILE_BYTES + kStages * 2 * ROWF_BYTES > 2 * NW * 32 * D * 2)
                                       ? kStages * 2 * TILE_BYTES + kStages * 2 * ROWF_BYTES
                                       : 2 * NW * 32 * D * 2;
  static constexpr size_t LDS_DKDV = (size_t)DKDV_RING + sizeof(int) * (2 * kSortMax + 8);
  // dQ: [K ring][V ring] + schedule
  static constexpr size_t LDS_DQ = (size_t)kStages * 2 * TILE_BYTES + sizeof(int) * (2 * kSortMax + 8);
  static_assert(CPT * THREADS == kBwdStage * CPR, "stage must split evenly");
  static_assert(NW * 32 * D * 2 <= kStages * 2 * TILE_BYTES, "one output block per wave fits the ring");
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

// Offsets for t_operands over a KV-swizzled tile: the same (row, chunk, half) pattern the
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
        off[cc][h][dt] = phys_off<D, Swz::KV>(16 * cc + 8 * h + 4 * g + (i16 >> 2),
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
      *reinterpret_cast<bf16x4*>(ost + phys_off<D, Swz::K>(n32, 4 * dt + ii) + 8 * g) = w;
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
    const u32x4 x = *reinterpret_cast<const u32x4*>(ost + phys_off<D, Swz::K>(r, ch));
    if (r < valid) *reinterpret_cast<u32x4*>(dst + (int64_t)r * rs + ch * 8) = x;
  }
}

// Decode work item u of a sorted or slot-enumerated schedule into (segment start, length,
// head, tile); false if the item is empty.
template <int BT>
__device__ __forceinline__ bool bwd_item(const BwdParams& p, int tiles_max, int u, bool sorted, const int* s_order,
                                         const int* s_prefix, int T, int& a, int& L, int& h, int& tile) {
  int s;
  if (sorted) {
    int lo = 0, hi = p.num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_prefix[mid]) <= u) lo = mid; else hi = mid - 1;
    }
    s = __builtin_amdgcn_readfirstlane(s_order[lo]);
    const int ntiles = (ld_table(p.cu, s + 1) - ld_table(p.cu, s) + BT - 1) / BT;
    const int local = u - __builtin_amdgcn_readfirstlane(s_prefix[lo]);
    h = local / ntiles;
    tile = local - h * ntiles;
  } else {
    const int per_seg = p.heads * tiles_max;
    s = u / per_seg;
    const int rem = u - s * per_seg;
    h = rem / tiles_max;
    tile = rem - h * tiles_max;
  }
  a = ld_table(p.cu, s);
  L = ld_table(p.cu, s + 1) - a;
  if (a < 0 || a >= T) return false;
  if (L > T - a) L = T - a;
  return L > 0 && tile * BT < L;
}

// Loads of one 64-row bf16 stage (rows [r0, r0 + 64) of a segment starting at element
// base, bounded at L) into a KV-swizzled LDS tile; rows >= L read as zeros.
// TAG keys the instantiation to its kernel (the HIP host pass rejects a specialisation
// holding buffer-to-LDS load builtins once two kernel templates have used it).
template <int D, int CPT, int TAG>
__device__ __forceinline__ void bwd_issue_tile(const __bf16* base, int r0, int L, int64_t rs,
                                               int row_bytes, char* dst, const int (&src)[CPT],
                                               int wave) {
  const int rows = (L - r0 < kBwdStage) ? (L - r0) : kBwdStage;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)r0 * rs), 0, rows * row_bytes, kRsrcFlags);
  dst += wave * CPT * 1024;
#pragma unroll
  for (int i = 0; i < CPT; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, src[i], 0, 0, 0);
}


// Order of a contraction whose 16-deep steps each read two operand fragments from LDS
// (in consumption order) and issue two MFMAs: the reads run `ahead` steps before the MFMAs
// that consume them.  With one wave per SIMD nothing else hides the read latency.
template <int D, int AHEAD>
__device__ __forceinline__ void pair_read_ahead() {
  static_assert(AHEAD > 0 && AHEAD < D / 16, "prefetch distance within the contraction");
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
  for (int t = 0; t < D / 16 - AHEAD; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * AHEAD, 0);
}
constexpr int kDkdvReadAhead = 2;

// ---- dK / dV
// Waves per SIMD the dK/dV kernel is compiled for: at d = 128 it needs ~450 registers
// (one wave); at d = 64 the same code fits 256 without spills, so two workgroups share a CU.
template <int D>
constexpr int kDkdvWavesPerEu = D == 64 ? 2 : 1;

template <int D>
__global__ void __launch_bounds__(kWave * kDkdvNW<D>)
__attribute__((amdgpu_waves_per_eu(kDkdvWavesPerEu<D>, kDkdvWavesPerEu<D>)))
pfa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = kDkdvNW<D>;
  constexpr int ROWS = NW * 32;                                   // keys per work item
  using C = BwdTile<D, NW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* const qring = reinterpret_cast<char*>(smem);
  char* const dring = qring + kStages * C::TILE_BYTES;
  char* const fring = dring + kStages * C::TILE_BYTES;            // [slot][neg_lse2 | delta]
  int* s_order = reinterpret_cast<int*>(qring + C::DKDV_RING);
  int* s_prefix = s_order + kSortMax;
  int* s_len = reinterpret_cast<int*>(qring);

  const int T = ld_table(p.cu, p.num_seqs);
  if (T > p.ws_rows) return;   // uniform across the workgroup, before any barrier
  const bool sorted = p.num_seqs <= kSortMax;
  const int total = sorted ? build_schedule<ROWS, C::THREADS>(p.cu, p.cu, p.num_seqs, p.heads,
                                                               s_len, s_order, s_prefix, kSortMax)
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
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, Swz::KV>(n32, 2 * t + g);
  int toff[2][2][C::DT];
  t_offsets<D>(lane, toff);
  int src[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) src[i] = logical_src<D, Swz::KV>((wave * C::CPT + i) * 64 + lane, row_bytes);
  if (sorted) __syncthreads();   // s_len aliases the Q ring

  for (int u = slot; u < total; u += G) {
    int a, L, h, kt;
    if (!bwd_item<ROWS>(p, p.tiles_max, u, sorted, s_order, s_prefix, T, a, L, h, kt)) continue;
    const int64_t head_off = (int64_t)h * D;
    const int k0 = kt * ROWS + wave * 32;            // this wave's first key
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
    // One stage; the ring slot is a template constant, so every LDS address is a lane
    // offset plus an immediate (no per-stage address arithmetic) and the accumulators keep
    // their registers across the unrolled pair of stages.
    auto stage = [&](auto slot, int s) {
      constexpr int cur = decltype(slot)::value;
      __builtin_amdgcn_s_waitcnt(kWaitVmem);
      __syncthreads();
      if (s + 1 < ns) issue(cur ^ 1, s + 1);
      const char* qst = qring + cur * C::TILE_BYTES;
      const char* dst = dring + cur * C::TILE_BYTES;
      const float* nls = reinterpret_cast<const float*>(fring + (cur * 2) * C::ROWF_BYTES);
      const float* dls = reinterpret_cast<const float*>(fring + (cur * 2 + 1) * C::ROWF_BYTES);
      // Both sub-blocks' S and dP products first, then per sub-block the weights and the dV,
      // dK products: the second pair of products runs in the matrix pipe while the first
      // sub-block's weights are formed, and the first sub-block's dV/dK products while the
      // second's are.  One wave per SIMD has no partner to fill those gaps.
      f32x16 sc[2], dp[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 qa[C::KSTEP], da[C::KSTEP];
        k_operands2<D>(qst + j * 32 * D * 2, dst + j * 32 * D * 2, koff, qa, da);
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[j][i] = dp[j][i] = 0.f;
#pragma unroll
        for (int t = 0; t < C::KSTEP; ++t) {
          sc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], kr[t], sc[j], 0, 0, 0);
          dp[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[t], vr[t], dp[j], 0, 0, 0);
        }
        pair_read_ahead<D, kDkdvReadAhead>();   // each pair's operand reads run two steps ahead
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* qj = qst + j * 32 * D * 2;
        const char* dj = dst + j * 32 * D * 2;
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
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[j][i], p.c, nlv[e]));
            const float dsv = pv * (dp[j][i] - dlv[e]);
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
    };
    for (int s = 0; s < ns; s += 2) {   // the ring slot is a constant in each copy
      stage(std::integral_constant<int, 0>{}, s);
      if (s + 1 < ns) stage(std::integral_constant<int, 1>{}, s + 1);
    }
    __syncthreads();   // every wave has left the ring
    char* const ok = qring + wave * (32 * D * 2);
    char* const ov = qring + (NW + wave) * (32 * D * 2);       // 2 x NW blocks fit DKDV_RING
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
__global__ void __launch_bounds__(kWave * kDqNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
pfa_bwd_dq_kernel(BwdParams p) {
  using C = BwdTile<D, kDqNW>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  char* const kring = reinterpret_cast<char*>(smem);
  char* const vring = kring + kStages * C::TILE_BYTES;
  int* s_order = reinterpret_cast<int*>(vring + kStages * C::TILE_BYTES);
  int* s_prefix = s_order + kSortMax;
  int* s_len = reinterpret_cast<int*>(kring);

  const int T = ld_table(p.cu, p.num_seqs);
  if (T > p.ws_rows) return;   // uniform across the workgroup, before any barrier
  const bool sorted = p.num_seqs <= kSortMax;
  const int total = sorted ? build_schedule<kDqRows, C::THREADS>(p.cu, p.cu, p.num_seqs, p.heads,
                                                                  s_len, s_order, s_prefix, kSortMax)
                           : p.num_seqs * p.heads * p.tiles_max_q;
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
  for (int t = 0; t < C::KSTEP; ++t) koff[t] = phys_off<D, Swz::KV>(n32, 2 * t + g);
  int toff[2][2][C::DT];
  t_offsets<D>(lane, toff);
  int src[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) src[i] = logical_src<D, Swz::KV>((wave * C::CPT + i) * 64 + lane, row_bytes);
  if (sorted) __syncthreads();   // s_len aliases the K ring

  for (int u = slot; u < total; u += G) {
    int a, L, h, qt;
    if (!bwd_item<kDqRows>(p, p.tiles_max_q, u, sorted, s_order, s_prefix, T, a, L, h, qt)) continue;
    const int64_t head_off = (int64_t)h * D;
    const int q0 = qt * kDqRows + wave * 32;
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
    // The row statistics of this lane's query, for this pass and the dK/dV pass after it:
    // nl = -LSE * log2(e) and delta = dO . O.  The lane holds half of the row (values
    // 16t + 8g .. +7, the layout of dr); lanes n32 and n32 + 32 add their halves.
    float nl = 0.f, part = 0.f;
    if (row < L) {
      const __bf16* op = p.out + (int64_t)(a + row) * rs + head_off;
#pragma unroll
      for (int t = 0; t < C::KSTEP; ++t) {
        const bf16x8 o = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * t + 8 * g));
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf((float)o[e], (float)dr[t][e], part);
      }
      nl = -p.lse[(int64_t)h * T + a + row] * kLog2e;
    }
    const float dl = part + __shfl_xor(part, 32);
    if (g == 0 && row < L) {
      p.ws[(int64_t)h * T + a + row] = nl;
      p.ws[(int64_t)p.heads * T + (int64_t)h * T + a + row] = dl;
    }
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
    auto stage = [&](auto slot, int s) {
      constexpr int cur = decltype(slot)::value;
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
        if (key0 + 32 <= L) {                       // every key of the sub-block is in the segment
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sc[i], p.c, nl));
            dsp[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - dl));
          }
        } else {                                    // the segment's last keys: the rest weigh 0
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + (i >> 2) * 8 + 4 * g + (i & 3);
            const float pv = key < L ? __builtin_amdgcn_exp2f(fmaf(sc[i], p.c, nl)) : 0.f;
            dsp[i >> 3][i & 7] = (__bf16)(pv * (dp[i] - dl));
          }
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
    };
    for (int s = 0; s < ns; s += 2) {   // the ring slot is a constant in each copy
      stage(std::integral_constant<int, 0>{}, s);
      if (s + 1 < ns) stage(std::integral_constant<int, 1>{}, s + 1);
    }
    __syncthreads();   // every wave has left the ring
    char* const oq = kring + wave * (32 * D * 2);
    stage_rows<D>(dqt, p.scale, oq, n32, g);
    __syncthreads();
    store_rows<D>(oq, lane, p.dq + (int64_t)(a + q0) * rs + head_off, rs, L - q0);
    __syncthreads();   // the next item's first stage overwrites the ring
  }
}

std::atomic<int> g_bwd_occ[kMaxDevices][2][2];   // [device][head_dim 64 / 128][dK-dV / dQ]

// Argument checks shared by both backward entry points, all before any HIP runtime call.
// workspace may be NULL only when the caller will not pass one (the allocation-free form).
int check_bwd_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                   const float* lse, const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int heads,
                   int head_dim, float scale, const void* dq, const void* dk, const void* dv,
                   const float* workspace, bool workspace_required) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr ||
      lse == nullptr || cu_seqlens == nullptr || dq == nullptr || dk == nullptr || dv == nullptr ||
      (workspace_required && workspace == nullptr))
    return PFA_ERR_NULL;
  if (num_seqs < 1) return PFA_ERR_NUM_SEQS;
  if (heads < 1) return PFA_ERR_HEADS;
  if (max_seqlen < 1) return PFA_ERR_MAX_SEQLEN;
  if (head_dim != 64 && head_dim != 128) return PFA_ERR_HEAD_DIM;
  if (!(std::isfinite(scale) && scale > 0.f)) return PFA_ERR_SCALE;
  const void* ins[7] = {q, k, v, out, dout, lse, cu_seqlens};
  const void* outs[4] = {dq, dk, dv, workspace};
  const int n_out = workspace != nullptr ? 4 : 3;
  for (int a = 0; a < n_out; ++a) {
    for (const void* in : ins)
      if (in == outs[a]) return PFA_ERR_ALIAS;
    for (int b = a + 1; b < n_out; ++b)
      if (outs[a] == outs[b]) return PFA_ERR_ALIAS;
  }
  // the [T, H, d] tensors move in 16-byte vectors; lse, workspace and the table element-wise
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out) || misaligned16(dout) ||
      misaligned16(dq) || misaligned16(dk) || misaligned16(dv) || misaligned4(lse) || misaligned4(workspace) ||
      misaligned4(cu_seqlens))
    return PFA_ERR_ALIGN;
  const int64_t tiles_max = ((int64_t)max_seqlen + kBwdRows - 1) / kBwdRows;
  const int64_t slots = (int64_t)num_seqs * heads * tiles_max;
  if ((int64_t)heads * head_dim > kMaxRowElems || slots > INT32_MAX) return PFA_ERR_SIZE;
  return PFA_OK;
}

// The two backward launches, with the row statistics in ws (room for ws_rows tokens).
int launch_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
               const float* lse, const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int heads,
               int head_dim, float scale, void* dq, void* dk, void* dv, float* ws, int ws_rows,
               hipStream_t stream) {
  const int rows_kv = 32 * (head_dim == 64 ? kDkdvNW<64> : kDkdvNW<128>);
  const int64_t tiles_max = ((int64_t)max_seqlen + rows_kv - 1) / rows_kv;
  const int64_t slots = (int64_t)num_seqs * heads * tiles_max;
  int dev = 0, cus = 0;
  const int rc = device_cus(&dev, &cus);
  if (rc != PFA_OK) return rc;
  const void* dkdv = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_bwd_dkdv_kernel<64>)
                                    : reinterpret_cast<const void*>(&pfa_bwd_dkdv_kernel<128>);
  const void* dqk = head_dim == 64 ? reinterpret_cast<const void*>(&pfa_bwd_dq_kernel<64>)
                                   : reinterpret_cast<const void*>(&pfa_bwd_dq_kernel<128>);
  const size_t lds_dkdv = head_dim == 64 ? BwdTile<64, kDkdvNW<64>>::LDS_DKDV : BwdTile<128, kDkdvNW<128>>::LDS_DKDV;
  const size_t lds_dq = head_dim == 64 ? BwdTile<64, kDqNW>::LDS_DQ : BwdTile<128, kDqNW>::LDS_DQ;
  const int threads = kWave * (head_dim == 64 ? kDkdvNW<64> : kDkdvNW<128>);
  const int threads_q = kWave * kDqNW;
  const int64_t tiles_max_q = ((int64_t)max_seqlen + kDqRows - 1) / kDqRows;
  const int64_t slots_q = (int64_t)num_seqs * heads * tiles_max_q;
  const int vi = head_dim == 64 ? 0 : 1;
  int occ_kv = g_bwd_occ[dev][vi][0].load(std::memory_order_relaxed);
  int occ_q = g_bwd_occ[dev][vi][1].load(std::memory_order_relaxed);
  if (occ_kv <= 0 || occ_q <= 0) {
    if (hipFuncSetAttribute(dkdv, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dkdv) != hipSuccess ||
        hipFuncSetAttribute(dqk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dq) != hipSuccess)
      return PFA_ERR_DEVICE;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_kv, dkdv, threads, lds_dkdv) != hipSuccess ||
        occ_kv <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_q, dqk, threads_q, lds_dq) != hipSuccess || occ_q <= 0)
      return PFA_ERR_DEVICE;
    g_bwd_occ[dev][vi][0].store(occ_kv, std::memory_order_relaxed);
    g_bwd_occ[dev][vi][1].store(occ_q, std::memory_order_relaxed);
  }
  auto grid_for = [&](int occ, int64_t n_slots) {
    int64_t grid = (int64_t)cus * occ;
    if (grid > n_slots) grid = n_slots;
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
  bp.ws = ws;
  bp.ws_rows = ws_rows;
  bp.cu = cu_seqlens;
  bp.dq = static_cast<__bf16*>(dq);
  bp.dk = static_cast<__bf16*>(dk);
  bp.dv = static_cast<__bf16*>(dv);
  bp.num_seqs = num_seqs;
  bp.heads = heads;
  bp.tiles_max = (int)tiles_max;
  bp.tiles_max_q = (int)tiles_max_q;
  bp.c = scale * kLog2e;
  bp.scale = scale;
  void* args[] = {&bp};
  // dQ first: it writes the row statistics the dK/dV pass reads
  if (hipLaunchKernel(dqk, dim3(grid_for(occ_q, slots_q)), dim3(threads_q), args, lds_dq, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  if (hipLaunchKernel(dkdv, dim3(grid_for(occ_kv, slots)), dim3(threads), args, lds_dkdv, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  return PFA_OK;
}

// ---- allocation-free form: the row statistics live in a library-held device array.
// One copy per device, allocated with the code object (it lives until the process ends).
// In host code the array's name is only a stand-in for its device address; each device's
// actual address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to a kernel.
static __device__ __align__(256) float scratch[PFA_BWD_SCRATCH_FLOATS];
std::atomic<float*> g_scratch[kMaxDevices];

int scratch_for_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PFA_ERR_DEVICE;
  float* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return PFA_ERR_DEVICE;
    ptr = static_cast<float*>(addr);
    g_scratch[dev].store(ptr, std::memory_order_release);   // a race stores the same address
  }
  *out = ptr;
  return PFA_OK;
}

}  // namespace

extern "C" {

PFA_API int pfa_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* dq, void* dk, void* dv, float* workspace, hipStream_t stream) {
  const int rc = check_bwd_args(q, k, v, out, dout, lse, cu_seqlens, num_seqs, max_seqlen, heads, head_dim,
                                scale, dq, dk, dv, workspace, true);
  if (rc != PFA_OK) return rc;
  return launch_bwd(q, k, v, out, dout, lse, cu_seqlens, num_seqs, max_seqlen, heads, head_dim, scale, dq, dk,
                    dv, workspace, INT32_MAX, stream);
}

PFA_API int pfa_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, const int32_t* cu_seqlens,
                                   int num_seqs, int max_seqlen, int64_t total_tokens, int heads,
                                   int head_dim, float scale, void* dq, void* dk, void* dv,
                                   hipStream_t stream) {
  int rc = check_bwd_args(q, k, v, out, dout, lse, cu_seqlens, num_seqs, max_seqlen, heads, head_dim, scale,
                          dq, dk, dv, nullptr, false);
  if (rc != PFA_OK) return rc;
  // 2 * heads * T fp32 values of row statistics must fit the array
  const int64_t ws_rows = (int64_t)PFA_BWD_SCRATCH_FLOATS / (2 * (int64_t)heads);
  if (total_tokens < 0 || total_tokens > ws_rows) return PFA_ERR_SIZE;
  float* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != PFA_OK) return rc;
  return launch_bwd(q, k, v, out, dout, lse, cu_seqlens, num_seqs, max_seqlen, heads, head_dim, scale, dq, dk,
                    dv, ws, (int)ws_rows, stream);
}

}  // extern "C"
