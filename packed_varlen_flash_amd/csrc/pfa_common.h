// pfa_common.h -- definitions shared by the library's kernels (gfx950): vector types,
// launch constants, the LDS swizzles of K/V stage tiles, the device-side longest-first
// scheduler, the K operand reads, and the host-side device query.  Everything sits in an
// anonymous namespace, so each translation unit has its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

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
constexpr int kSortMax = 512;    // schedule capacity every kernel's LDS holds
constexpr int kSortCapMax = 4096;   // largest table the streaming forward sorts (more LDS)
constexpr int kWaitVmem = 0x0F70;   // s_waitcnt vmcnt(0), other counters unconstrained
// s_waitcnt vmcnt(n), other counters unconstrained (vmcnt bits 3:0 and 15:14)
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Entry i of a read-only int32 table (the segment tables), i wave-uniform: read through
// the scalar cache (constant address space), so its wait is on lgkmcnt and never on the
// vector-memory counter, which also counts the output stores still in flight.
typedef const __attribute__((address_space(4))) int32_t cint32_t;
__device__ __forceinline__ int32_t ld_table(const int32_t* t, int i) {
  return ((cint32_t*)t)[i];   // an address-space cast (reinterpret_cast cannot express it)
}

// a pointer the caller knows to be wave-uniform, in scalar registers (a buffer resource
// built from it then needs no per-lane loop)
__device__ __forceinline__ void* uniform_ptr(const void* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Largest row stride (elements) of any input: 64 rows of it, in bytes, must stay within
// the 32-bit offsets of a buffer resource.
constexpr int64_t kMaxRowElems = int64_t(1) << 23;

// LDS layout of a stage tile: 16-byte chunks, row-major, with the chunk index XOR-swizzled
// inside each 256-byte line (64 banks of 4 bytes) so the read patterns are free of bank
// conflicts.  Row reads (the K operand: 16 lanes = 16 consecutive rows, one logical chunk)
// need the swizzle to be a bijection over 16 consecutive rows; transposed reads (4
// consecutive rows x 64 bytes per 32 lanes) need every aligned group of 4 rows spread
// over the line's four 64-byte quarters.
//   K:  row reads only (the forward's K tiles);
//   V:  transposed reads only (the forward's V tiles);
//   KV: both (the backward's tiles, read as rows for one product and transposed for
//       another): the line's two low bit pairs swapped (d = 128: one row per line), or
//       bit 0 moved above bits 1-2 (d = 64: two rows per line).
enum class Swz { K, V, KV };

template <int D, Swz SW>
__device__ __forceinline__ int swz(int line) {
  if constexpr (SW == Swz::K) return line & 15;
  if constexpr (SW == Swz::V) return (line & 3) << 2;
  return D == 128 ? (((line & 3) << 2) | ((line >> 2) & 3)) : (((line & 1) << 2) | ((line >> 1) & 3));
}

// byte offset of logical (row, chunk) within a stage
template <int D, Swz SW>
__device__ __forceinline__ int phys_off(int row, int chunk) {
  const int P = row * (D / 8) + chunk;
  const int line = P >> 4;
  return ((line << 4) | ((P & 15) ^ swz<D, SW>(line))) << 4;
}

// logical byte offset (row * row_bytes + chunk * 16) of the chunk stored at physical
// chunk position P; the XOR swizzle is its own inverse
template <int D, Swz SW>
__device__ __forceinline__ int logical_src(int P, int row_bytes) {
  const int line = P >> 4;
  const int Pl = (line << 4) | ((P & 15) ^ swz<D, SW>(line));
  return (Pl / (D / 8)) * row_bytes + (Pl % (D / 8)) * 16;
}

// ---------------------------------------------------------------------------------
// Device-side scheduler: decode cu_seqlens into a longest-first list of work items.
// ---------------------------------------------------------------------------------
// Sorted mode (num_seqs <= the kernel's schedule capacity cap): s_order[r] = segment of
// rank r (key length, i.e. the work per query tile, descending; ties by index), s_prefix[r]
// = first item of rank r; a segment has heads * ceil(query length / BM) items, ordered
// head-major, query-tile-minor.  Returns the item count.  s_order holds cap entries,
// s_prefix n + 1; scratch (dead LDS of the caller's tile area) at least max(n, THREADS)
// ints.  Up to kSortMax segments each thread ranks its segments by counting; above, a
// bitonic sort of (length, index) keys over cap (a power of two) entries.
constexpr int kSortIdxBits = 13;                          // segment index in a sort key
constexpr int kSortLenMax = (1 << (32 - kSortIdxBits)) - 1;   // longer keys tie (index order)
// every real key stays below the padding key 0xFFFFFFFF
static_assert((1 << kSortIdxBits) > kSortCapMax, "index field holds every segment, with room");

template <int BM, int THREADS>
__device__ int build_schedule(const int32_t* cu_q, const int32_t* cu_k, int n, int heads,
                              int* scratch, int* s_order, int* s_prefix, int cap) {
  const int tid = threadIdx.x;
  if (n <= kSortMax) {
    int* s_len = scratch;
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
  } else {
    // ascending keys = descending length, then ascending index; padding sorts last
    uint32_t* key = reinterpret_cast<uint32_t*>(s_order);
    for (int i = tid; i < cap; i += THREADS) {
      uint32_t kv = 0xFFFFFFFFu;
      if (i < n) {
        int L = cu_k[i + 1] - cu_k[i];
        L = L < 0 ? 0 : (L > kSortLenMax ? kSortLenMax : L);
        kv = ((uint32_t)(kSortLenMax - L) << kSortIdxBits) | (uint32_t)i;
      }
      key[i] = kv;
    }
    __syncthreads();
    for (int k = 2; k <= cap; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int t = tid; t < (cap >> 1); t += THREADS) {
          const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));   // lower element of the pair
          const uint32_t a = key[i], b = key[i + j];
          if ((a > b) == ((i & k) == 0)) {
            key[i] = b;
            key[i + j] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int r = tid; r < n; r += THREADS) s_order[r] = (int)(key[r] & ((1u << kSortIdxBits) - 1));
  }
  __syncthreads();
  // items per rank, then an inclusive scan: each thread runs over its own chunk of ranks,
  // a Hillis-Steele scan over the chunk totals, and the chunk offsets are added back
  for (int r = tid; r < n; r += THREADS) {
    const int sg = s_order[r];
    int Lq = cu_q[sg + 1] - cu_q[sg];
    Lq = Lq > 0 ? Lq : 0;
    s_prefix[r + 1] = heads * ((Lq + BM - 1) / BM);
  }
  if (tid == 0) s_prefix[0] = 0;
  __syncthreads();
  const int per = (n + THREADS - 1) / THREADS;
  const int chunks = (n + per - 1) / per;
  const int r0 = tid * per;
  const int r1 = r0 + per < n ? r0 + per : n;
  int run = 0;
  for (int r = r0; r < r1; ++r) {
    run += s_prefix[r + 1];
    s_prefix[r + 1] = run;
  }
  if (tid < chunks) scratch[tid] = run;
  __syncthreads();
  for (int off = 1; off < chunks; off <<= 1) {
    const int add = (tid < chunks && tid >= off) ? scratch[tid - off] : 0;
    __syncthreads();
    if (tid < chunks) scratch[tid] += add;
    __syncthreads();
  }
  const int before = (tid > 0 && tid < chunks) ? scratch[tid - 1] : 0;
  for (int r = r0; r < r1; ++r) s_prefix[r + 1] += before;
  __syncthreads();
  return s_prefix[n];
}

// K operand fragments of one 32-key sub-block: kst points at the sub-block's first row;
// koff[t] is this lane's byte offset of (row n32, chunk 2t+g).
template <int D>
__device__ __forceinline__ void k_operands(const char* kst, const int (&koff)[D / 16],
                                           bf16x8 (&a)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) a[t] = *reinterpret_cast<const bf16x8*>(kst + koff[t]);
}

// Operand fragments of two 32-row sub-blocks (same lane offsets), read interleaved in the
// order two MFMA chains that alternate between them consume them: a[0], b[0], a[1], ...
template <int D>
__device__ __forceinline__ void k_operands2(const char* ast, const char* bst, const int (&koff)[D / 16],
                                            bf16x8 (&a)[D / 16], bf16x8 (&b)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    a[t] = *reinterpret_cast<const bf16x8*>(ast + koff[t]);
    b[t] = *reinterpret_cast<const bf16x8*>(bst + koff[t]);
  }
}

// ---- host side
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // compute units per device, 0 until queried

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

inline bool misaligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; }
// fp32 and int32 arrays are read and written one element at a time
inline bool misaligned4(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3) != 0; }

}  // namespace
